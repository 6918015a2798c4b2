"""Whole-layer GPU parity: route -> layout -> permute -> grouped FFN (+ shared) -> combine.

Small versions of the five workloads are compared element by element at every
intermediate.  At the workloads' full sizes (in the launch configuration the
benchmark times) the routing and layout arrays and the permuted payload are
compared in full, bit for bit; h and the expert outputs on every row of a few
sampled experts (largest, smallest non-empty, one more); y and the shared
expert on sampled tokens, each computed one by one by the oracle.
"""
import numpy as np
import pytest
import torch

import combine_grouped_gemm_amd as moe
import workload as w
from combine_grouped_gemm_amd.layer import MoELayer, PipelinedMoE
from oracle import moe_oracle as oracle
from tests.gpu_util import decision_margin, f64, router_bound, say, sync, token_rel_err, with_logits

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

# per-token relative error bars on y (max over tokens of ||dy_t||_inf / ||y_t||_inf)
Y_BAR = {"f32": 2e-2, "bf16": 2e-2, "fp8": 6e-2}
# tighter bars expected from the arithmetic: fp32 end to end; bf16 rounding of h,
# the expert outputs and y (3 roundings of 2^-9 relative, on the row's scale)
Y_EXPECT = {"f32": 1e-5, "bf16": 1e-2, "fp8": 1e-2}
GEMM_BAR = {"f32": 1e-5, "bf16": 1e-2, "fp8": 1e-2}

SMALL = {
    "tiny_f32": w.CONFIGS["tiny_f32"],
    "mixtral_small": w.CONFIGS["mixtral_bf16"].scaled(N=512, H=1024, I=1024),
    "dsv3_small": w.CONFIGS["dsv3_bf16"].scaled(N=512, H=1024, E=64, I=256),
    "dsv3_zipf_small": w.CONFIGS["dsv3_zipf_bf16"].scaled(N=512, H=1024, E=64, I=256),
    "decode_fp8_small": w.CONFIGS["decode_fp8"].scaled(N=64, H=1024, E=64, I=256),
    # fp8 at a prefill batch (64 rows per expert: the tiled kernels, not the weight-streaming
    # ones); routed experts only, the fp8 shared expert has a test of its own below
    "dsv3_fp8_small": w.CONFIGS["dsv3_fp8"].scaled(N=512, H=1024, E=64, I=256, shared=False),
}


def _quantize_rows(a):
    """Oracle quantization of a float32 matrix, 512 rows at a time (same result as whole)."""
    qs, ss = [], []
    for r in range(0, a.shape[0], 512):
        q, s = oracle.quantize_blocks(a[r:r + 512])
        qs.append(q)
        ss.append(s)
    return np.concatenate(qs), np.concatenate(ss)


class OracleWeights:
    """Expert weights for the oracle, copied from the generator's device tensors on demand.

    bf16/f32 layers: float64 values.  fp8 layers: the oracle's own quantization
    of the same bf16 values, dequantized to float64.  Only the last few experts are
    kept (a DeepSeek-V3-sized layer holds 90 GB of float64 weights).
    """

    KEEP = 4

    def __init__(self, w13, w2, fp8):
        self.w13, self.w2, self.fp8 = w13, w2, fp8
        self.c13, self.c2 = {}, {}

    def _get(self, t, e, cache):
        if e not in cache:
            while len(cache) >= self.KEEP:
                cache.pop(next(iter(cache)))
            a = t[e].detach().cpu().to(torch.float32).numpy()
            cache[e] = oracle.dequantize_blocks(*_quantize_rows(a)) if self.fp8 else a.astype(np.float64)
        return cache[e]

    def g13(self, e):
        return self._get(self.w13, e, self.c13)

    def g2(self, e):
        return self._get(self.w2, e, self.c2)


def _build(cfg, sentinel=False):
    """The layer's forward from the oracle's logits.  sentinel: every output buffer (h, the
    expert and shared outputs, y) is filled with NaN first and must be finite afterwards, so
    a row that no tile wrote cannot go unnoticed."""
    say(f"layer {cfg.name} N={cfg.N} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I} {cfg.dtype}")
    inp = with_logits(w.make_layer_inputs(cfg, DEV))
    layer = MoELayer(cfg.N, cfg.H, cfg.E, cfg.k, cfg.I, cfg.dtype, inp["w13"], inp["w2"],
                     inp.get("sw13"), inp.get("sw2"), cfg.n_group, cfg.topk_group, inp["bias"])
    outs = []
    if sentinel:
        outs = [("h", layer.h_all if layer.fuse else layer.h),
                ("expert_out", layer.out_all if layer.fuse else layer.expert_out), ("y", layer.y)]
        if cfg.shared and not layer.fuse:
            outs.append(("shared_out", layer.shared_out))
        for _, t in outs:
            t.fill_(float("nan"))
    y = layer.forward(inp["x"], inp["z"])
    sync()
    for name, t in outs:
        assert bool(torch.isfinite(t).all()), f"{name}: rows left unwritten"
    return inp, layer, y


@pytest.mark.parametrize("name", ["dsv3_small", "decode_fp8_small"])
def test_device_bytes_accounts_for_every_allocation(name):
    """The layer's device_bytes sums to what the allocator handed out while the layer was
    built and ran (each block rounded up to 512 bytes), and the weights are the sizes of the
    weight tensors."""
    cfg = SMALL[name]
    inp = with_logits(w.make_layer_inputs(cfg, DEV))
    sync()
    before = torch.cuda.memory_allocated(DEV)
    layer = MoELayer(cfg.N, cfg.H, cfg.E, cfg.k, cfg.I, cfg.dtype, inp["w13"], inp["w2"],
                     inp.get("sw13"), inp.get("sw2"), cfg.n_group, cfg.topk_group, inp["bias"])
    layer.forward(inp["x"], inp["z"])
    sync()
    grown = torch.cuda.memory_allocated(DEV) - before
    got = layer.device_bytes()
    # the caller's tensors the layer keeps: the routing bias, and the weights unless fp8
    # (then it holds quantized copies of its own)
    callers = [inp["bias"]] + ([] if cfg.dtype == "fp8" else [inp["w13"], inp["w2"], inp.get("sw13"), inp.get("sw2")])
    caller_bytes = sum(t.nbytes for t in callers if t is not None)
    held = sum(got.values()) - caller_bytes
    n_blocks = sum(1 for v in vars(layer).values() for t in (v if isinstance(v, tuple) else (v,))
                   if isinstance(t, torch.Tensor))
    assert held <= grown <= held + 512 * n_blocks
    if cfg.dtype != "fp8":
        assert got["weights"] == caller_bytes
    assert got["activations"] >= layer.y.nbytes + layer.topk_idx.nbytes and got["workspace"] > 0


def _check_routing(cfg, inp, layer):
    b = inp["bias_cpu"]
    ridx, rgate = oracle.route(inp["z_cpu"].numpy(), cfg.k, None if b is None else b.numpy(),
                               cfg.n_group, cfg.topk_group)
    assert np.array_equal(layer.topk_idx.cpu().numpy(), ridx)
    assert np.abs(layer.topk_gate.cpu().numpy().astype(np.float64) - rgate).max() <= 1e-6
    lay = oracle.dispatch_layout(ridx, cfg.E)
    for got, ref in zip(layer.layout, lay):
        assert np.array_equal(got.cpu().numpy(), ref)
    return ridx, rgate, lay


def _check_permute(cfg, inp, layer, send_pos):
    """Bit-exact permuted payload; returns the oracle's permuted rows as float64 values."""
    x = inp["x"].cpu()
    if cfg.dtype == "fp8":
        q, s = _quantize_rows(x.to(torch.float32).numpy())
        if layer.x_perm is None:   # (gathered fp8: each token's codes and scales, once)
            assert np.array_equal(layer.x_q.cpu().numpy(), q)
            assert np.array_equal(layer.x_q_scale.cpu().numpy(), s)
            return None, (q, s)
        pq, ps = oracle.permute(q, send_pos, cfg.k), oracle.permute(s, send_pos, cfg.k)
        assert np.array_equal(layer.x_perm.cpu().numpy(), pq)
        assert np.array_equal(layer.x_perm_scale.cpu().numpy(), ps)
        return None, (q, s)
    view = torch.int32 if cfg.dtype == "f32" else torch.int16
    x_perm = layer.x_perm
    if x_perm is None:   # the gate/up GEMM gathered its rows from x: permute explicitly
        x_perm = moe.moe_permute(inp["x"], layer.layout[2], cfg.k)
    assert np.array_equal(x_perm.cpu().view(view).numpy(), oracle.permute(x.view(view).numpy(), send_pos, cfg.k))
    return x.to(torch.float64).numpy(), None


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_small_all_intermediates(name):
    cfg = SMALL[name]
    inp, layer, y = _build(cfg)
    ridx, rgate, (n_e, off, sp, ss) = _check_routing(cfg, inp, layer)
    xs, _ = _check_permute(cfg, inp, layer, sp)
    ow = OracleWeights(inp["w13"], inp["w2"], cfg.dtype == "fp8")
    kw = {}
    if cfg.shared:
        kw = dict(shared_w13=f64(inp["sw13"][0]), shared_w2=f64(inp["sw2"][0]))
    if cfg.dtype == "fp8":
        ref = oracle.moe_layer(inp["x"].cpu().to(torch.float32).numpy(), inp["z_cpu"].numpy(), cfg.k,
                               lambda e: _quantize_rows(inp["w13"][e].cpu().float().numpy())[0],
                               lambda e: _quantize_rows(inp["w2"][e].cpu().float().numpy())[0],
                               bias=None, n_group=cfg.n_group, topk_group=cfg.topk_group, fp8=True,
                               w13_scale=lambda e: _quantize_rows(inp["w13"][e].cpu().float().numpy())[1],
                               w2_scale=lambda e: _quantize_rows(inp["w2"][e].cpu().float().numpy())[1], **kw)
    else:
        b = inp["bias_cpu"]
        ref = oracle.moe_layer(xs, inp["z_cpu"].numpy(), cfg.k, ow.g13, ow.g2,
                               bias=None if b is None else b.numpy(), n_group=cfg.n_group,
                               topk_group=cfg.topk_group, **kw)
    assert np.array_equal(ref["topk_idx"], ridx)
    valid = ref["h"].shape[1] > 0
    if valid:
        assert token_rel_err(f64(layer.h), ref["h"]) <= GEMM_BAR[cfg.dtype]
        assert token_rel_err(f64(layer.expert_out), ref["expert_out"]) <= GEMM_BAR[cfg.dtype]
    if cfg.shared:
        assert token_rel_err(f64(layer.shared_out), ref["shared_out"]) <= GEMM_BAR[cfg.dtype]
    err = token_rel_err(f64(y), ref["y"])
    say(f"  y max per-token relative error {err:.3e}, imbalance {ref['imbalance']:.3f}")
    assert err <= Y_BAR[cfg.dtype]
    assert err <= Y_EXPECT[cfg.dtype]


def test_layer_fp8_shared_expert():
    """The shared expert of an fp8 layer runs on the fp8 path like the routed ones: x and its
    weights quantized per row and 128 columns, SwiGLU FFN on the dequantized values.  Checked
    against the oracle's codec and FFN composed the same way (quantize_blocks,
    dequantize_blocks, expert_ffn), every token row."""
    cfg = w.CONFIGS["dsv3_fp8"].scaled(N=512, H=1024, E=64, I=256)
    inp, layer, y = _build(cfg)
    x = inp["x"].cpu().to(torch.float32).numpy()
    deq = lambda m: oracle.dequantize_blocks(*_quantize_rows(m))
    a = deq(x)
    w13 = deq(inp["sw13"][0].cpu().float().numpy())
    w2 = deq(inp["sw2"][0].cpu().float().numpy())
    _, ref = oracle.expert_ffn(a, w13, w2)
    assert token_rel_err(f64(layer.shared_out), ref) <= GEMM_BAR["fp8"]


def test_layer_gathered_equals_permuted():
    """The bf16 layer with the permute folded into gate/up == the layer with the permute kernel, bit for bit."""
    cfg = SMALL["dsv3_small"]
    inp = with_logits(w.make_layer_inputs(cfg, DEV))
    ys = []
    for gather in (True, False):
        layer = MoELayer(cfg.N, cfg.H, cfg.E, cfg.k, cfg.I, cfg.dtype, inp["w13"], inp["w2"],
                         inp.get("sw13"), inp.get("sw2"), cfg.n_group, cfg.topk_group, inp["bias"], gather=gather)
        assert layer.gather == gather
        ys.append(layer.forward(inp["x"], inp["z"]).clone())
    sync()
    assert torch.equal(ys[0].view(torch.int16), ys[1].view(torch.int16))


def test_layer_shared_on_side_stream_equals_serial():
    """The shared expert on a second stream (combine waits for it) == all on one stream, bit for
    bit, over several forwards in a row."""
    cfg = SMALL["dsv3_small"]
    inp = with_logits(w.make_layer_inputs(cfg, DEV))
    ys = []
    for overlap in (True, False):
        layer = MoELayer(cfg.N, cfg.H, cfg.E, cfg.k, cfg.I, cfg.dtype, inp["w13"], inp["w2"],
                         inp.get("sw13"), inp.get("sw2"), cfg.n_group, cfg.topk_group, inp["bias"],
                         overlap_shared=overlap, fuse_shared=False)
        assert (layer.side is not None) == overlap
        for _ in range(3):
            y = layer.forward(inp["x"], inp["z"])
        ys.append(y.clone())
    sync()
    assert torch.equal(ys[0].view(torch.int16), ys[1].view(torch.int16))


def test_layer_shared_fused_equals_separate():
    """The shared expert inside the routed launches == its own launches: the gate/up rows
    bit for bit (same kernel), the down rows and y within the bf16 bar (the separate dense
    down runs the 128-row-tile kernel)."""
    cfg = SMALL["dsv3_small"]
    inp = with_logits(w.make_layer_inputs(cfg, DEV))
    outs = []
    for fuse in (True, False):
        layer = MoELayer(cfg.N, cfg.H, cfg.E, cfg.k, cfg.I, cfg.dtype, inp["w13"], inp["w2"],
                         inp.get("sw13"), inp.get("sw2"), cfg.n_group, cfg.topk_group, inp["bias"],
                         fuse_shared=fuse)
        assert layer.fuse == fuse
        y = layer.forward(inp["x"], inp["z"]).clone()
        outs.append((layer.h.clone(), layer.expert_out.clone(), layer.shared_out.clone(), y))
    sync()
    (h0, e0, s0, y0), (h1, e1, s1, y1) = outs
    assert torch.equal(h0.view(torch.int16), h1.view(torch.int16))
    assert torch.equal(e0.view(torch.int16), e1.view(torch.int16))
    assert token_rel_err(f64(s0), f64(s1)) <= 1e-2
    assert token_rel_err(f64(y0), f64(y1)) <= 1e-2


def test_layer_gates_in_down_epilogue():
    """Gates applied in the down GEMM's epilogue (combine then sums with weight 1): the
    routed outputs equal the gate times the unscaled ones to bf16 rounding, and y matches
    the oracle's within the bf16 bar."""
    cfg = SMALL["dsv3_small"]
    inp = with_logits(w.make_layer_inputs(cfg, DEV))
    res = {}
    for gated in (False, True):
        layer = MoELayer(cfg.N, cfg.H, cfg.E, cfg.k, cfg.I, cfg.dtype, inp["w13"], inp["w2"],
                         inp.get("sw13"), inp.get("sw2"), cfg.n_group, cfg.topk_group, inp["bias"],
                         gate_in_down=gated)
        assert layer.gate_in_down == gated
        y = layer.forward(inp["x"], inp["z"]).clone()
        sync()
        gate_of_row = layer.topk_gate.reshape(-1)[layer.layout[3].long()].float()
        res[gated] = (y, layer.expert_out.float().clone(), layer.shared_out.clone(), gate_of_row)
    (y0, e0, s0, g), (y1, e1, s1, _) = res[False], res[True]
    assert torch.equal(s0.view(torch.int16), s1.view(torch.int16))     # shared rows: gate 1
    assert token_rel_err(f64(e1), f64(e0 * g[:, None])) <= 1e-2
    # y against the oracle (which weights the unscaled expert outputs in the combine)
    b = inp["bias_cpu"]
    ow = OracleWeights(inp["w13"], inp["w2"], False)
    ref = oracle.moe_layer(inp["x"].cpu().to(torch.float64).numpy(), inp["z_cpu"].numpy(), cfg.k, ow.g13, ow.g2,
                           bias=None if b is None else b.numpy(), n_group=cfg.n_group, topk_group=cfg.topk_group,
                           shared_w13=f64(inp["sw13"][0]), shared_w2=f64(inp["sw2"][0]))
    err = token_rel_err(f64(y1), ref["y"])
    say(f"  gates in the down epilogue: y max per-token relative error {err:.3e}")
    assert err <= Y_BAR[cfg.dtype]


@pytest.mark.parametrize("name", ["tiny_f32", "dsv3_small", "dsv3_zipf_small"])
def test_layer_with_router_logits(name):
    """The layer computes its logits z = x W_r^T itself (moe_router_logits) before the route:
    z within the fp32 summation bound of the oracle's; the experts equal the oracle's route
    on the oracle's z except at near ties; y on the other tokens within the layer's bar."""
    cfg = SMALL[name]
    say(f"layer with router {cfg.name}")
    inp = with_logits(w.make_layer_inputs(cfg, DEV))
    layer = MoELayer(cfg.N, cfg.H, cfg.E, cfg.k, cfg.I, cfg.dtype, inp["w13"], inp["w2"],
                     inp.get("sw13"), inp.get("sw2"), cfg.n_group, cfg.topk_group, inp["bias"], w_r=inp["w_r"])
    y = layer.forward(inp["x"])
    sync()
    zr = inp["z_cpu"].numpy()
    dz = np.abs(f64(layer.z) - zr)
    assert np.all(dz <= router_bound(f64(inp["x"]), f64(inp["w_r"]), cfg.H))
    b = inp["bias_cpu"]
    ow = OracleWeights(inp["w13"], inp["w2"], False)
    kw = dict(shared_w13=f64(inp["sw13"][0]), shared_w2=f64(inp["sw2"][0])) if cfg.shared else {}
    ref = oracle.moe_layer(f64(inp["x"]), zr, cfg.k, ow.g13, ow.g2, bias=None if b is None else b.numpy(),
                           n_group=cfg.n_group, topk_group=cfg.topk_group, **kw)
    diff = np.any(layer.topk_idx.cpu().numpy() != ref["topk_idx"], axis=1)
    if diff.any():
        zb = oracle.biased_logits(zr[diff], None if b is None else b.numpy())
        m = decision_margin(zb, cfg.k, cfg.n_group, cfg.topk_group)
        slack = 2 * np.spacing(np.abs(zb).max(axis=1).astype(np.float32)).astype(np.float64)
        assert np.all(m <= 2 * dz[diff].max(axis=1) + slack), "a route differs away from a near tie"
    same = ~diff
    err = token_rel_err(f64(y)[same], ref["y"][same])
    say(f"  z max abs error {dz.max():.3e}; {int(diff.sum())} near-tie tokens; y max per-token relative "
        f"error {err:.3e}")
    assert err <= Y_BAR[cfg.dtype] and err <= Y_EXPECT[cfg.dtype]


FULL = ["mixtral_bf16", "dsv3_bf16", "dsv3_zipf_bf16", "decode_fp8", "dsv3_fp8"]
# tokens of y computed by the oracle (decode: its fp8 weights are quantized by the oracle's
# own codec, expert by expert, which takes seconds per expert on the host)
SAMPLE_TOKENS = {"mixtral_bf16": 64, "dsv3_bf16": 64, "dsv3_zipf_bf16": 64, "decode_fp8": 4, "dsv3_fp8": 4}
SAMPLE_EXPERTS = {"mixtral_bf16": 8, "dsv3_bf16": 16, "dsv3_zipf_bf16": 16, "decode_fp8": 6, "dsv3_fp8": 8}


def sampled_experts(n_e, n_blk, want):
    """Experts whose tiles lie across the whole tile order of the routed launch: the routed
    tiles (expert -> n-block -> m-tile, 256-row m-tiles) are cut into 8 contiguous ranges, one
    per XCD; take the experts holding the first and the middle tile of each range, then the
    largest and the smallest non-empty expert and up to four experts split into several
    m-tiles; then experts spread over the ids until there are at least `want`."""
    n_e = np.asarray(n_e)
    mt = -(-n_e // 256)
    end = np.cumsum(mt) * n_blk
    total = int(end[-1])
    picks = []
    for x in range(8):
        lo, hi = total * x // 8, total * (x + 1) // 8
        for t in (lo, (lo + hi) // 2):
            picks.append(int(np.searchsorted(end, t, side="right")))
    nz = np.nonzero(n_e)[0]
    picks += [int(nz[np.argmax(n_e[nz])]), int(nz[np.argmin(n_e[nz])])]
    picks += [int(e) for e in np.nonzero(mt >= 2)[0][:4]]
    out = []
    for e in picks:
        if e < len(n_e) and n_e[e] > 0 and e not in out:
            out.append(e)
    for e in np.linspace(0, len(n_e) - 1, want).astype(int):   # (fill up, spread over the ids)
        if len(out) >= want:
            break
        if n_e[e] > 0 and int(e) not in out:
            out.append(int(e))
    return sorted(out)


@pytest.mark.parametrize("name", FULL)
def test_layer_full_size_sampled(name):
    cfg = w.CONFIGS[name]
    inp, layer, y = _build(cfg, sentinel=True)
    say("  every row of h, the expert outputs and y written")
    ridx, rgate, (n_e, off, sp, ss) = _check_routing(cfg, inp, layer)
    say(f"  routing + layout bit-exact; imbalance {oracle.imbalance(n_e):.3f}, "
        f"max n_e {n_e.max()}, empty experts {(n_e == 0).sum()}")
    xs, xq = _check_permute(cfg, inp, layer, sp)
    say("  permuted payload bit-exact")
    fp8 = cfg.dtype == "fp8"
    ow = OracleWeights(inp["w13"], inp["w2"], fp8)

    def a_rows(rows):  # the oracle's permuted activation rows (float64 values)
        toks = ss[rows] // cfg.k
        if fp8:
            q, s = xq
            return oracle.dequantize_blocks(q[toks], s[toks])
        return xs[toks]

    # every row of experts spread over the launch's tile order
    if fp8 and not layer.gather:   # (the weight-streaming kernel: 16-row m-tiles; experts spread over the ids)
        nz = np.nonzero(n_e)[0]
        experts = sorted({int(nz[np.argmax(n_e[nz])])} |
                         {int(e) for e in nz[np.linspace(0, len(nz) - 1, SAMPLE_EXPERTS[name] - 1).astype(int)]})
    else:
        experts = sampled_experts(n_e, -(-cfg.I // 128), SAMPLE_EXPERTS[name])
    h_gpu, eo_gpu = f64(layer.h), f64(layer.expert_out)
    for e in experts:
        rows = np.arange(off[e], off[e + 1])
        rh, ro = oracle.expert_ffn(a_rows(rows), ow.g13(e), ow.g2(e))
        assert token_rel_err(h_gpu[off[e]:off[e + 1]], rh) <= GEMM_BAR[cfg.dtype], e
        assert token_rel_err(eo_gpu[off[e]:off[e + 1]], ro) <= GEMM_BAR[cfg.dtype], e
    say(f"  grouped GEMMs match on experts {experts} (n_e {[int(n_e[e]) for e in experts]})")

    # y on sampled tokens: y_t = sum_j g_tj Expert_{I_t[j]}(x_t) (+ shared), by the oracle,
    # one expert at a time over the sampled (token, slot) pairs it serves
    S = SAMPLE_TOKENS[name]
    toks = np.linspace(0, cfg.N - 1, S).astype(np.int64)
    eo_s = np.zeros((S * cfg.k, cfg.H))
    by_expert = {}
    for i, t in enumerate(toks):
        for j in range(cfg.k):
            by_expert.setdefault(int(ridx[t, j]), []).append((i * cfg.k + j, int(sp[t * cfg.k + j])))
    for e in sorted(by_expert):
        pos = np.array([p for p, _ in by_expert[e]])
        rows = np.array([r for _, r in by_expert[e]])
        _, eo_s[pos] = oracle.expert_ffn(a_rows(rows), ow.g13(e), ow.g2(e))
    sh = None
    if cfg.shared and fp8:   # (the tokens' fp8 values against the oracle's quantized shared weights)
        sw = OracleWeights(inp["sw13"], inp["sw2"], True)
        _, sh = oracle.expert_ffn(a_rows(sp[toks * cfg.k]), sw.g13(0), sw.g2(0))
        assert token_rel_err(f64(layer.shared_out[torch.from_numpy(toks).to(DEV)]), sh) <= GEMM_BAR[cfg.dtype]
    elif cfg.shared:
        _, sh = oracle.expert_ffn(xs[toks], f64(inp["sw13"][0]), f64(inp["sw2"][0]))
        assert token_rel_err(f64(layer.shared_out[torch.from_numpy(toks).to(DEV)]), sh) <= GEMM_BAR[cfg.dtype]
    ref = oracle.combine(eo_s, np.arange(S * cfg.k), rgate[toks], cfg.k, sh)
    err = token_rel_err(f64(y[torch.from_numpy(toks).to(DEV)]), ref)
    say(f"  y on {S} tokens ({len(by_expert)} experts): max per-token relative error {err:.3e}")
    assert err <= Y_BAR[cfg.dtype]
    assert err <= Y_EXPECT[cfg.dtype]


@pytest.mark.parametrize("name", ["tiny_f32", "dsv3_small"])
def test_layer_forward_graph_replay(name):
    """A whole forward (router logits through combine) captured in a HIP graph: the library
    allocates, clears and synchronises nothing inside a call, so every replay equals the eager
    forward bit for bit, with eager work on the same buffers between the replays."""
    cfg = SMALL[name]
    say(f"graph replay {name}")
    inp = w.make_layer_inputs(cfg, DEV)
    layer = MoELayer(cfg.N, cfg.H, cfg.E, cfg.k, cfg.I, cfg.dtype, inp["w13"], inp["w2"],
                     inp.get("sw13"), inp.get("sw2"), cfg.n_group, cfg.topk_group, inp["bias"], w_r=inp["w_r"])
    x = inp["x"]
    ref = layer.forward(x).clone()
    view = torch.int32 if cfg.dtype == "f32" else torch.int16
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(x)
    torch.cuda.current_stream().wait_stream(side)
    sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x)
    for _ in range(3):
        layer.y.zero_()
        layer.topk_idx.fill_(-1)
        sync()
        g.replay()
        sync()
        assert torch.equal(layer.y.view(view), ref.view(view))
        eager = layer.forward(x)   # eager work between the replays
        sync()
        assert torch.equal(eager.view(view), ref.view(view))


@pytest.mark.parametrize("chunks", [2, 4])
def test_pipelined_chunks_match_oracle(chunks):
    """The layer cut into chunks of tokens, each chunk's combine on a second stream beside the
    next chunk's GEMMs: y on every token against the oracle's unchunked layer (routing is per
    token), over three forwards in a row; and equal to the unchunked layer's y within the bar."""
    cfg = SMALL["dsv3_small"]
    say(f"pipelined layer, {chunks} chunks")
    inp = with_logits(w.make_layer_inputs(cfg, DEV))
    pipe = PipelinedMoE(chunks, cfg.N, cfg.H, cfg.E, cfg.k, cfg.I, inp["w13"], inp["w2"], inp["sw13"], inp["sw2"],
                        cfg.n_group, cfg.topk_group, inp["bias"])
    for _ in range(3):
        y = pipe.forward(inp["x"], inp["z"])
    sync()
    ow = OracleWeights(inp["w13"], inp["w2"], False)
    ref = oracle.moe_layer(f64(inp["x"]), inp["z_cpu"].numpy(), cfg.k, ow.g13, ow.g2, n_group=cfg.n_group,
                           topk_group=cfg.topk_group, shared_w13=f64(inp["sw13"][0]), shared_w2=f64(inp["sw2"][0]))
    n = cfg.N // chunks
    got_idx = np.concatenate([lay.topk_idx.cpu().numpy() for lay in pipe.parts])
    assert np.array_equal(got_idx, ref["topk_idx"])
    err = token_rel_err(f64(y), ref["y"])
    say(f"  y max per-token relative error {err:.3e}")
    assert err <= Y_BAR["bf16"] and err <= Y_EXPECT["bf16"]
    layer = MoELayer(cfg.N, cfg.H, cfg.E, cfg.k, cfg.I, cfg.dtype, inp["w13"], inp["w2"], inp["sw13"], inp["sw2"],
                     cfg.n_group, cfg.topk_group, inp["bias"])
    y1 = layer.forward(inp["x"], inp["z"])
    sync()
    assert token_rel_err(f64(y), f64(y1)) <= 1e-2
    assert n * chunks == cfg.N
