"""GPU parity of the backward pass against the oracle's gradients (chain rule in float64).

Each entry point on ragged, seeded inputs with empty and one-row experts; the whole
layer's gradients on scaled-down workloads element by element; at the DeepSeek-V3 size the
weight gradients of sampled experts and the input gradient of sampled tokens, each computed
by the oracle one expert or one token at a time.  Every call goes through the C ABI.
"""
import numpy as np
import pytest
import torch

import combine_grouped_gemm_amd as moe
import workload as w
from combine_grouped_gemm_amd.layer import MoELayer
from oracle import moe_oracle as oracle
from tests.gpu_util import bf16_ulp, f64, say, sync, token_rel_err, with_logits
from tests.test_gpu_layer import sampled_experts

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
U32 = 2.0 ** -24
# per-row relative bar of the layer's gradients: bf16 intermediates (d_expert_out, the
# recomputed pre-activations, dh, d_au, the slots' input gradients, dx) each round by at
# most 2^-9 of their row's scale; fp32 sums
GRAD_BAR = 2e-2


def mat_rel_err(got, ref):
    """max |got - ref| / max |ref| over a whole weight gradient.  Per-row relative errors do
    not suit weight gradients: for an expert with one row, row j of dW13 is d_au[r, j] x_r,
    and a single element of d_au carries the cancellation error of dh = d_out W_down (its
    bf16 inputs round by 2^-9 of terms that can be far larger than their sum)."""
    den = np.abs(ref).max()
    return float(np.abs(np.asarray(got, np.float64) - ref).max() / den) if den > 0 else float(np.abs(got).max())


def _n(shape, sub, dt=torch.bfloat16, std=0.02):
    return w.normal(shape, w.stream_key(11, w.T_EO, sub), DEV, dt, std=std)


def _layout(N, E, k, seed, empty=()):
    idx = w.fixed_route(N, E, k, "random", seed=seed).numpy()
    for e in empty:   # move the slots of these experts to the next expert the token lacks
        for t in range(N):
            for j in range(k):
                if idx[t, j] == e:
                    free = [c for c in range(E) if c not in idx[t] and c not in empty]
                    idx[t, j] = free[0]
    n_e, off, sp, ss = oracle.dispatch_layout(idx, E)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).astype(np.int32)).to(DEV)
    return idx, n_e, off, sp, ss, dev(off), dev(sp), dev(ss)


@pytest.fixture(autouse=True, scope="module")
def _loaded():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    moe.lib()


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_combine_backward(dt):
    N, H, E, k = 300, 512, 16, 4
    say(f"combine backward {dt}")
    idx, n_e, off, sp, ss, doff, dsp, dss = _layout(N, E, k, 3)
    dy = _n((N, H), 1, dt)
    eo = _n((N * k, H), 2, dt)
    g = w.random_gates(N, k, seed=4)
    d_eo, dg = moe.moe_combine_backward(dy, dsp, g.to(DEV), eo)
    sync()
    r_eo, r_dg = oracle.combine_backward(f64(dy), sp, g.numpy(), f64(eo), k)
    err = np.abs(f64(d_eo) - r_eo)
    # one fp32 product, one rounding to dt
    ulp = bf16_ulp(r_eo) if dt == torch.bfloat16 else np.abs(r_eo) * 2.0 ** -23
    assert np.all(err <= ulp + 1e-30)
    bound = 2 * (H + 1) * U32 * (np.abs(f64(dy))[:, None, :] * np.abs(f64(eo))[sp.reshape(N, k)]).sum(axis=2)
    assert np.all(np.abs(f64(dg) - r_dg) <= bound)


def test_swiglu_backward():
    rows, I = 777, 256
    say("swiglu backward")
    au = _n((rows, 2 * I), 5, std=1.5)
    dh = _n((rows, I), 6, std=0.05)
    d_au, h = moe.moe_swiglu_backward(au, dh)
    sync()
    a, u = f64(au)[:, :I], f64(au)[:, I:]
    da, du = oracle.swiglu_backward(a, u, f64(dh))
    ref = np.concatenate([da, du], axis=1)
    scale = np.abs(f64(dh)).max(axis=1, keepdims=True) * (np.abs(a).max() + 1) * (np.abs(u).max() + 1)
    assert np.all(np.abs(f64(d_au) - ref) <= bf16_ulp(ref) + 1e-5 * scale)
    rh = oracle.silu(a) * u
    assert np.all(np.abs(f64(h) - rh) <= bf16_ulp(rh) + 1e-5 * (np.abs(rh).max() + 1e-30))


@pytest.mark.parametrize("gathered", [True, False])
def test_gate_up_preact(gathered):
    N, H, E, k, I = 200, 512, 8, 3, 256
    say(f"gate/up pre-activations gathered={gathered}")
    idx, n_e, off, sp, ss, doff, dsp, dss = _layout(N, E, k, 7, empty=(2,))
    x = _n((N, H), 8)
    w13 = _n((E, 2 * I, H), 9)
    xp = oracle.permute(f64(x), sp, k)
    if gathered:
        au = moe.moe_expert_gate_up_preact(x, doff, w13, N * k, dss, k)
    else:
        au = moe.moe_expert_gate_up_preact(torch.from_numpy(xp).to(torch.bfloat16).to(DEV), doff, w13)
    sync()
    ref = np.zeros((N * k, 2 * I))
    for e in range(E):
        ref[off[e]:off[e + 1]] = xp[off[e]:off[e + 1]] @ f64(w13[e]).T
    assert token_rel_err(f64(au), ref) <= 1e-2


DGRAD_CASES = [
    # name, N, k, E, K, Nout, empty experts (Nout % 256 == 0 and K % 64 == 0: the 128 x 256
    # tile kernel; otherwise the 128 x 128 one)
    ("wide_ragged", 400, 3, 8, 256, 512, (1,)),
    ("wide_one_expert", 300, 1, 1, 192, 256, ()),
    ("ragged", 400, 3, 8, 256, 384, (1,)),
    ("one_expert", 300, 1, 1, 96, 128, ()),
    ("many_small", 150, 2, 64, 128, 256, (0, 5)),
]


@pytest.mark.parametrize("case", DGRAD_CASES, ids=[c[0] for c in DGRAD_CASES])
def test_expert_dgrad(case):
    name, N, k, E, K, Nout, empty = case
    say(f"dgrad {name}")
    idx, n_e, off, sp, ss, doff, dsp, dss = _layout(N, E, k, 10, empty)
    rows = N * k
    dC = _n((rows, K), 11)
    W = _n((E, K, Nout), 12)
    out = moe.moe_expert_dgrad(dC, doff, W)
    sync()
    ref = np.zeros((rows, Nout))
    for e in range(E):
        ref[off[e]:off[e + 1]] = f64(dC[off[e]:off[e + 1]]) @ f64(W[e])
    assert token_rel_err(f64(out), ref) <= 1e-2


WGRAD_CASES = [
    # name, N, k, E, M, Nout, gathered, out dtype, empty experts (ungathered with Nout % 256
    # == 0: the 128 x 256 tile kernel; otherwise the 128 x 128 one)
    ("wide_ragged_f32", 400, 3, 8, 256, 512, False, torch.float32, (1,)),
    ("wide_bf16_m512", 300, 2, 8, 512, 256, False, torch.bfloat16, (2,)),
    ("wide_bf16_long", 700, 1, 2, 128, 256, False, torch.bfloat16, ()),
    ("wide_many_small", 150, 2, 64, 384, 256, False, torch.float32, (0, 5)),
    ("ragged_f32", 400, 3, 8, 256, 384, False, torch.float32, (1,)),
    ("gathered_bf16", 300, 4, 16, 128, 256, True, torch.bfloat16, (3, 9)),
    ("one_expert_long", 700, 1, 1, 128, 128, False, torch.float32, ()),
]


@pytest.mark.parametrize("case", WGRAD_CASES, ids=[c[0] for c in WGRAD_CASES])
def test_expert_wgrad(case):
    name, N, k, E, M, Nout, gathered, odt, empty = case
    say(f"wgrad {name}")
    idx, n_e, off, sp, ss, doff, dsp, dss = _layout(N, E, k, 13, empty)
    rows = N * k
    A = _n((rows, M), 14)
    if gathered:
        B = _n((N, Nout), 15)
        dw = moe.moe_expert_wgrad(A, B, doff, b_rows=dss, b_div=k, dw_dtype=odt)
        Brows = f64(B)[ss // k]
    else:
        B = _n((rows, Nout), 15)
        dw = moe.moe_expert_wgrad(A, B, doff, dw_dtype=odt)
        Brows = f64(B)
    sync()
    got = f64(dw)
    Af = f64(A)
    for e in range(E):
        a, b = Af[off[e]:off[e + 1]], Brows[off[e]:off[e + 1]]
        ref = a.T @ b
        bound = 2 * (len(a) + 1) * U32 * (np.abs(a).T @ np.abs(b))
        if odt == torch.bfloat16:
            bound = bound + bf16_ulp(ref)
        assert np.all(np.abs(got[e] - ref) <= bound + 1e-30), f"expert {e} (n_e {n_e[e]})"
    assert not got[list(empty)].any() if empty else True


def test_expert_wgrad_chunked_deal_skewed():
    """A weight-gradient launch of 2048 tiles (32 experts x 4 x 16 tiles of 128 x 256), large
    enough that tiles go to the XCDs in chunks of 32, with one hot expert (~80% of the
    tokens), an empty expert and ragged row counts: every expert's gradient within the fp32
    sum bound plus one bf16 rounding."""
    say("wgrad chunked deal, skewed")
    N, k, E, M, Nout = 600, 2, 32, 512, 4096
    rng = np.random.default_rng(31)
    idx = np.zeros((N, k), np.int64)
    for t in range(N):
        first = 0 if rng.random() < 0.8 else int(rng.choice([c for c in range(1, E) if c != 5]))
        pool = [c for c in range(E) if c != first and c != 5]
        idx[t] = [first, pool[int(rng.integers(len(pool)))]]
    n_e, off, sp, ss = oracle.dispatch_layout(idx, E)
    assert n_e[5] == 0 and n_e[0] > 400
    doff = torch.from_numpy(off.astype(np.int32)).to(DEV)
    rows = N * k
    A = _n((rows, M), 16)
    B = _n((rows, Nout), 17)
    dw = moe.moe_expert_wgrad(A, B, doff, dw_dtype=torch.bfloat16)
    sync()
    got = f64(dw)
    Af, Bf = f64(A), f64(B)
    for e in range(E):
        a, b = Af[off[e]:off[e + 1]], Bf[off[e]:off[e + 1]]
        ref = a.T @ b
        bound = 2 * (len(a) + 1) * U32 * (np.abs(a).T @ np.abs(b)) + bf16_ulp(ref)
        assert np.all(np.abs(got[e] - ref) <= bound + 1e-30), f"expert {e} (n_e {n_e[e]})"
    assert not got[5].any()


def test_router_backward():
    N, H, E, k = 500, 256, 32, 6
    say("router backward")
    idx, n_e, off, sp, ss, doff, dsp, dss = _layout(N, E, k, 16, empty=(4,))
    zsel = w.normal((N, k), w.stream_key(16, w.T_GATE), "cpu", torch.float32, std=1.0).numpy().astype(np.float64)
    g = np.exp(zsel - zsel.max(axis=1, keepdims=True))
    g = (g / g.sum(axis=1, keepdims=True)).astype(np.float32)
    dg = w.normal((N, k), w.stream_key(17, w.T_GATE), "cpu", torch.float32, std=1.0).numpy()
    x = _n((N, H), 18)
    dz, dw_r = moe.moe_router_backward(torch.from_numpy(g).to(DEV), torch.from_numpy(dg).to(DEV), doff, dss, x)
    sync()
    rdz = oracle.gates_backward(g, dg)
    g64, d64 = g.astype(np.float64), dg.astype(np.float64)
    zb = 4 * (k + 2) * U32 * g64 * (np.abs(d64) + (np.abs(g64 * d64)).sum(axis=1, keepdims=True))
    assert np.all(np.abs(f64(dz) - rdz) <= zb)
    _, rdw = oracle.router_backward(f64(x), np.zeros((E, H)), idx, rdz)
    xs = np.abs(f64(x))
    rz, zbf = np.abs(rdz).reshape(-1), zb.reshape(-1)
    for e in range(E):
        slots = ss[off[e]:off[e + 1]]
        # the fp32 sum over the expert's slots, plus what the dz differences above can carry
        bound = ((2 * (len(slots) + 1) * U32 * (rz[slots] + zbf[slots]) + zbf[slots])[:, None] *
                 xs[slots // k]).sum(axis=0)
        assert np.all(np.abs(f64(dw_r[e]) - rdw[e]) <= bound + 1e-30)
    assert not f64(dw_r[4]).any()


@pytest.mark.parametrize("E,k,shared", [(256, 8, True), (8, 2, False), (64, 6, True)])
def test_router_input_grad(E, k, shared):
    """The router's input gradient dx_t = sum_j dz_tj W_r[e_tj] (+ rest): equal to moe_combine's
    gather-sum over the rows of W_r bit for bit (the same arithmetic; only the loads' cache hint
    differs), and within one bf16 step plus the fp32 sum bound of the exactly rounded sum."""
    N, H = 300, 1024
    say(f"router input gradient E={E} k={k}")
    w_r = _n((E, H), 21)
    idx = w.fixed_route(N, E, k, "random", seed=E + k)
    dz = w.normal((N, k), w.stream_key(22, w.T_GATE, E), "cpu", torch.float32, std=1.0)
    rest = _n((N, H), 23) if shared else None
    got = moe.moe_router_input_grad(w_r, idx.to(DEV), dz.to(DEV), rest)
    ref_c = moe.moe_combine(w_r, idx.to(DEV), dz.to(DEV), rest)
    sync()
    assert torch.equal(got.view(torch.int16), ref_c.view(torch.int16))
    wr, d = f64(w_r), dz.numpy().astype(np.float64)
    ref = np.zeros((N, H))
    mag = np.zeros((N, H))
    for j in range(k):
        ref += d[:, j:j + 1] * wr[idx[:, j].numpy()]
        mag += np.abs(d[:, j:j + 1] * wr[idx[:, j].numpy()])
    if shared:
        ref += f64(rest)
        mag += np.abs(f64(rest))
    tol = bf16_ulp(ref) * 1.0001 + (k + 1) * U32 * mag
    assert np.all(np.abs(f64(got) - ref) <= tol + bf16_ulp(ref))


SMALL = {
    "dsv3_small": w.CONFIGS["dsv3_bf16"].scaled(N=512, H=1024, E=64, I=256),
    "dsv3_zipf_small": w.CONFIGS["dsv3_zipf_bf16"].scaled(N=512, H=1024, E=64, I=256),
    "mixtral_small": w.CONFIGS["mixtral_bf16"].scaled(N=512, H=1024, I=1024),
}


def _layer_for_backward(cfg, save=False):
    inp = with_logits(w.make_layer_inputs(cfg, DEV))
    layer = MoELayer(cfg.N, cfg.H, cfg.E, cfg.k, cfg.I, cfg.dtype, inp["w13"], inp["w2"], inp.get("sw13"),
                     inp.get("sw2"), cfg.n_group, cfg.topk_group, inp["bias"], w_r=inp["w_r"])
    layer.forward(inp["x"], inp["z"], save_for_backward=save)
    dy = w.normal((cfg.N, cfg.H), w.stream_key(cfg.seed, w.T_EO, 5), DEV, torch.bfloat16, std=1.0)
    return inp, layer, dy


@pytest.mark.parametrize("save", [False, True], ids=["recomputed", "saved"])
@pytest.mark.parametrize("name", list(SMALL))
def test_layer_backward_small(name, save):
    """The layer's gradients against the oracle's, with the gate/up pre-activations
    recomputed by the backward or kept by the forward (layers that fuse the shared expert)."""
    cfg = SMALL[name]
    say(f"layer backward {name} N={cfg.N} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I} saved={save}")
    inp, layer, dy = _layer_for_backward(cfg, save)
    assert layer.au_saved == (save and layer.fuse)
    gr = layer.backward(inp["x"], dy, dw_dtype=torch.float32)
    sync()
    b = inp["bias_cpu"]
    kw = dict(shared_w13=f64(inp["sw13"][0]), shared_w2=f64(inp["sw2"][0])) if cfg.shared else {}
    ref = oracle.moe_layer_backward(f64(inp["x"]), inp["z_cpu"].numpy(), cfg.k, lambda e: f64(inp["w13"][e]),
                                    lambda e: f64(inp["w2"][e]), f64(dy), bias=None if b is None else b.numpy(),
                                    n_group=cfg.n_group, topk_group=cfg.topk_group, w_r=f64(inp["w_r"]), **kw)
    assert np.array_equal(layer.topk_idx.cpu().numpy(), ref["fwd"]["topk_idx"])
    errs = {}
    errs["d_expert_out"] = token_rel_err(f64(gr["d_eo"]), ref["d_expert_out"])
    errs["d_gate"] = float(np.abs(f64(gr["dg"]) - ref["dg"]).max() / np.abs(ref["dg"]).max())
    errs["dh"] = token_rel_err(f64(gr["dh"]), ref["dh"])
    errs["d_au"] = token_rel_err(f64(gr["d_au"]), ref["d_au"])
    errs["dx"] = token_rel_err(f64(gr["dx"]), ref["dx"])
    errs["dw13"] = max(mat_rel_err(f64(gr["dw13"][e]), v) for e, v in ref["dw13"].items())
    errs["dw2"] = max(mat_rel_err(f64(gr["dw2"][e]), v) for e, v in ref["dw2"].items())
    untouched = [e for e in range(cfg.E) if e not in ref["dw13"]]
    assert not f64(gr["dw13"][untouched]).any() and not f64(gr["dw2"][untouched]).any()
    if cfg.shared:
        errs["dsw13"] = mat_rel_err(f64(gr["dsw13"][0]), ref["shared_dw13"])
        errs["dsw2"] = mat_rel_err(f64(gr["dsw2"][0]), ref["shared_dw2"])
    errs["dz"] = float(np.abs(f64(gr["dz"]) - ref["dz_sel"]).max() / np.abs(ref["dz_sel"]).max())
    errs["dw_r"] = mat_rel_err(f64(gr["dw_r"]), ref["dw_r"])
    say("  " + ", ".join(f"{n} {v:.2e}" for n, v in errs.items()))
    for n, v in errs.items():
        assert v <= GRAD_BAR, n


def test_layer_backward_full_size_sampled():
    """DeepSeek-V3 size: every gradient buffer starts as NaN and must be finite afterwards (no
    row or expert left unwritten); the weight gradients of experts spread over the tile order
    (and the largest, the smallest non-empty and split ones) and the input gradient of 16
    tokens, each from the oracle on that expert's rows or that token alone."""
    cfg = w.CONFIGS["dsv3_bf16"]
    say("layer backward dsv3_bf16 full size")
    inp, layer, dy = _layer_for_backward(cfg, save=True)
    layer.backward_steps(inp["x"], dy)   # (allocates the gradient buffers)
    outs = ("d_eo", "dg", "dh", "d_au", "h", "d_perm", "x_perm", "dw13", "dw2", "dh_s", "d_au_s", "h_s",
            "dx_s", "dsw13", "dsw2", "dz", "dw_r", "dx_r", "dx")
    for n in outs:
        layer.grads[n].fill_(float("nan"))
    gr = layer.backward(inp["x"], dy)
    sync()
    for n in outs:
        assert bool(torch.isfinite(gr[n]).all()), f"{n}: left unwritten"
    k = cfg.k
    n_e = layer.layout[0].cpu().numpy()
    off = layer.layout[1].cpu().numpy()
    ss = layer.layout[3].cpu().numpy()
    idx = layer.topk_idx.cpu().numpy()
    gates = layer.topk_gate.cpu().numpy().astype(np.float64)
    xs = f64(inp["x"])
    dys = f64(dy)
    experts = sampled_experts(n_e, -(-cfg.I // 128), 8)
    for e in experts:
        slots = ss[off[e]:off[e + 1]]
        toks = slots // k
        d_out = gates.reshape(-1)[slots, None] * dys[toks]
        r = oracle.expert_ffn_backward(xs[toks], f64(inp["w13"][e]), f64(inp["w2"][e]), d_out)
        e13 = mat_rel_err(f64(gr["dw13"][e]), r["dw13"])
        e2 = mat_rel_err(f64(gr["dw2"][e]), r["dw2"])
        say(f"  expert {e} (n_e {n_e[e]}): dw13 {e13:.2e}, dw2 {e2:.2e}")
        assert e13 <= GRAD_BAR and e2 <= GRAD_BAR
    # dx of sampled tokens: the slots' input gradients, the shared expert's, the router's
    w_r = f64(inp["w_r"])
    sw13, sw2 = f64(inp["sw13"][0]), f64(inp["sw2"][0])
    for t in np.linspace(0, cfg.N - 1, 16).astype(np.int64):
        dx = np.zeros(cfg.H)
        dg = np.zeros(k)
        for j in range(k):
            e = int(idx[t, j])
            w13e, w2e = f64(inp["w13"][e]), f64(inp["w2"][e])
            _, o = oracle.expert_ffn(xs[t:t + 1], w13e, w2e)
            dg[j] = float(dys[t] @ o[0])
            r = oracle.expert_ffn_backward(xs[t:t + 1], w13e, w2e, gates[t, j] * dys[t:t + 1])
            dx += r["d_in"][0]
        dx += oracle.expert_ffn_backward(xs[t:t + 1], sw13, sw2, dys[t:t + 1])["d_in"][0]
        dz = oracle.gates_backward(gates[t:t + 1], dg[None])[0]
        dx += dz @ w_r[idx[t]]
        err = float(np.abs(f64(gr["dx"][t]) - dx).max() / np.abs(dx).max())
        say(f"  token {t}: dx relative error {err:.2e}")
        assert err <= GRAD_BAR


def test_saved_preactivations_equal_recomputed():
    """The forward's kept pre-activations of the routed rows equal the backward's recomputed
    ones bit for bit (the same tile kernel and k order); the gradients agree."""
    cfg = SMALL["dsv3_small"]
    say("saved vs recomputed pre-activations")
    inp, layer, dy = _layer_for_backward(cfg, save=True)
    rows = cfg.N * cfg.k
    au_saved = layer.au_all[:rows].clone()
    g1 = {n: layer.backward(inp["x"], dy)[n].clone() for n in ("dx", "dw13", "dw2", "dsw13", "dw_r")}
    layer.forward(inp["x"], inp["z"], save_for_backward=False)
    assert not layer.au_saved
    g2 = layer.backward(inp["x"], dy)
    sync()
    assert torch.equal(au_saved.view(torch.int16), layer.grads["au"].view(torch.int16))
    for n, v in g1.items():
        assert mat_rel_err(f64(g2[n]), f64(v)) <= 1e-2, n


def test_backward_shared_on_side_stream_equals_serial():
    """The shared expert's backward on a second stream == all on one stream, bit for bit,
    over several steps in a row."""
    cfg = SMALL["dsv3_small"]
    say("backward with the shared expert on a side stream")
    inp, layer, dy = _layer_for_backward(cfg, save=True)
    names = ("dx", "dw13", "dw2", "dsw13", "dsw2", "dw_r")
    ref = {n: layer.backward(inp["x"], dy)[n].clone() for n in names}
    for _ in range(3):
        got = layer.backward(inp["x"], dy, overlap_shared=True)
    sync()
    for n in names:
        assert torch.equal(got[n], ref[n]), n
