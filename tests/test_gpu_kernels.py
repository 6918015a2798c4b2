"""GPU parity of each libmoe entry point against the CPU oracle, on seeded inputs.

Indices and layout maps are compared bit for bit; the fp8 codec bit for bit;
floating-point outputs within bars derived from the arithmetic (see each test).
Every call goes through the C ABI (combine_grouped_gemm_amd -> libmoe.so).
"""
import numpy as np
import pytest
import torch

import combine_grouped_gemm_amd as moe
import workload as w
from oracle import moe_oracle as oracle
from tests.gpu_util import bf16_round, bf16_ulp, decision_margin, f64, router_bound, say, sync, token_rel_err

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True, scope="module")
def _loaded():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    moe.lib()


def _logits(N, E, seed, ties=False):
    z = w.normal((N, E), w.stream_key(seed, w.T_WR, 77), "cpu", torch.float32, std=1.0)
    if ties:
        z = torch.floor(z * 2.0) / 2.0  # few distinct values: ties everywhere
    return z


# ------------------------------------------------------------------------------------------
# route
# ------------------------------------------------------------------------------------------

ROUTE_CASES = [
    # name, N, E, k, n_group, topk_group, bias, ties
    ("tiny", 256, 8, 2, 0, 0, False, False),
    ("decode", 128, 256, 8, 0, 0, False, False),
    ("groups_8_of_4", 1000, 256, 8, 8, 4, False, False),
    ("groups_bias", 777, 256, 8, 8, 4, True, False),
    ("E1_k1", 33, 1, 1, 0, 0, False, False),
    ("k_eq_E", 65, 16, 16, 0, 0, False, False),
    ("E1024_k32", 70, 1024, 32, 0, 0, True, False),
    ("E100_groups", 90, 100, 7, 4, 3, False, False),
    ("E64_groups64", 50, 64, 5, 64, 5, False, False),
    ("ties", 500, 32, 6, 0, 0, False, True),
    ("ties_groups", 500, 32, 6, 4, 2, False, True),
]


@pytest.mark.parametrize("case", ROUTE_CASES, ids=[c[0] for c in ROUTE_CASES])
def test_route_matches_oracle(case):
    name, N, E, k, ng, tg, use_bias, ties = case
    say(f"route {name}")
    z = _logits(N, E, seed=sum(map(ord, name)), ties=ties)
    bias = (w.normal((E,), w.stream_key(5, w.T_PERM, E), "cpu", torch.float32, std=0.5)
            if use_bias else None)
    idx, gate = moe.moe_route(z.to(DEV), k, None if bias is None else bias.to(DEV), ng, tg)
    sync()
    ridx, rgate = oracle.route(z.numpy(), k, None if bias is None else bias.numpy(), ng, tg)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(gate.cpu().numpy().astype(np.float64) - rgate).max() <= 1e-6


# ------------------------------------------------------------------------------------------
# router logits
# ------------------------------------------------------------------------------------------

def _check_router(x, w_r, z, rows=None):
    """z vs the oracle on every row (or on the given rows), within the summation bound."""
    xs = f64(x) if rows is None else f64(x[rows])
    ws = f64(w_r)
    ref = oracle.router_logits(xs, ws).astype(np.float64)
    got = f64(z) if rows is None else f64(z[rows])
    err = np.abs(got - ref)
    bound = router_bound(xs, ws, x.shape[1])
    assert got.shape == ref.shape
    assert np.all(err <= bound), f"router logits off by {err.max():.3e} (bound {bound.min():.3e})"
    scale = np.abs(ref).max() if ref.size else 1.0
    say(f"  router logits max abs error {err.max() if err.size else 0:.3e} (max |z| {scale:.3e})")
    return ref


ROUTER_CASES = [
    # name, N, H, E, dtype
    ("f32_tiny", 256, 128, 8, torch.float32),           # plain fp32-FMA kernel
    ("bf16_E_not_mult4", 300, 256, 6, torch.bfloat16),   # plain kernel, bf16 loads, ragged tokens
    ("bf16_ragged_tiles", 300, 1024, 64, torch.bfloat16),   # MFMA tiles of 160 + 140 rows, 8 parts
    ("bf16_two_nblocks", 1000, 512, 260, torch.bfloat16),   # 256 + 4 experts, 4 parts
    ("bf16_one_row", 1, 256, 16, torch.bfloat16),
]


@pytest.mark.parametrize("case", ROUTER_CASES, ids=[c[0] for c in ROUTER_CASES])
def test_router_logits_small(case):
    name, N, H, E, dt = case
    say(f"router {name} N={N} H={H} E={E} {dt}")
    x = w.normal((N, H), w.stream_key(5, w.T_X, N), DEV, dt)
    w_r = w.normal((E, H), w.stream_key(5, w.T_WR, E), DEV, dt)
    z = moe.moe_router_logits(x, w_r)
    sync()
    _check_router(x, w_r, z)


@pytest.mark.parametrize("name", ["tiny_f32", "mixtral_bf16", "dsv3_bf16", "decode_fp8"])
def test_router_logits_full_config(name):
    """Every logit of the workloads' full sizes (8 parts of K at the DeepSeek-V3 shape, 14 at
    the decode batch, 16 for Mixtral's 8 experts); two calls give identical bits."""
    cfg = w.CONFIGS[name]
    say(f"router config {name} N={cfg.N} H={cfg.H} E={cfg.E}")
    x = w.hidden_states(cfg, DEV)
    w_r = w.router_weight(cfg, DEV)
    z = moe.moe_router_logits(x, w_r)
    z2 = moe.moe_router_logits(x, w_r)
    sync()
    assert torch.equal(z, z2)
    _check_router(x, w_r, z)


def test_router_logits_many_tiles_sampled():
    """257 m-tiles (more tiles than CUs: K is not split, sums go straight to z); the oracle
    checks the first and last tiles' rows and a random sample."""
    N, H, E = 257 * 256 - 100, 1024, 256
    say(f"router many tiles N={N} H={H} E={E}")
    x = w.normal((N, H), w.stream_key(6, w.T_X), DEV, torch.bfloat16)
    w_r = w.normal((E, H), w.stream_key(6, w.T_WR), DEV, torch.bfloat16)
    assert moe.moe_workspace_bytes(moe.MOE_OP_ROUTER, N, H, 0, E, 0, moe.MOE_BF16) == 0
    z = moe.moe_router_logits(x, w_r)
    sync()
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([np.arange(300), np.arange(N - 400, N), rng.integers(0, N, 500)]))
    _check_router(x, w_r, z, torch.from_numpy(rows).to(DEV))


def test_router_logits_empty_batch_is_noop():
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    w_r = torch.zeros((16, 256), dtype=torch.bfloat16, device=DEV)
    z = torch.full((0, 16), 7.0, device=DEV)
    assert moe.moe_router_logits(x, w_r, z).shape == (0, 16)


@pytest.mark.parametrize("name", ["dsv3_bf16", "dsv3_zipf_bf16", "decode_fp8"])
def test_router_then_route_full_config(name):
    """Route on the GPU's logits: wherever its experts differ from the oracle's route on the
    oracle's logits, the oracle's own decision margin there is within twice the logits'
    measured difference (a near tie); everywhere else the same experts and gates."""
    cfg = w.CONFIGS[name]
    say(f"router + route config {name}")
    x = w.hidden_states(cfg, DEV)
    w_r = w.router_weight(cfg, DEV)
    b = w.zipf_bias(cfg)
    z = moe.moe_router_logits(x, w_r)
    idx, gate = moe.moe_route(z, cfg.k, None if b is None else b.to(DEV), cfg.n_group, cfg.topk_group)
    sync()
    zr = _check_router(x, w_r, z).astype(np.float32)
    ridx, rgate = oracle.route(zr, cfg.k, None if b is None else b.numpy(), cfg.n_group, cfg.topk_group)
    dz = np.abs(f64(z) - zr).max(axis=1)
    diff = np.any(idx.cpu().numpy() != ridx, axis=1)
    if diff.any():
        zb = oracle.biased_logits(zr[diff], None if b is None else b.numpy())
        m = decision_margin(zb, cfg.k, cfg.n_group, cfg.topk_group)
        slack = 2 * np.spacing(np.abs(zb).max(axis=1).astype(np.float32)).astype(np.float64)
        assert np.all(m <= 2 * dz[diff] + slack), "a route differs away from a near tie"
    say(f"  tokens routed differently (near ties): {int(diff.sum())} of {cfg.N}")
    same = ~diff
    gerr = np.abs(gate.cpu().numpy().astype(np.float64)[same] - rgate[same])
    assert np.all(gerr <= 1e-6 + 4 * dz[same, None])


@pytest.mark.parametrize("name", ["tiny_f32", "mixtral_bf16", "dsv3_bf16", "dsv3_zipf_bf16", "decode_fp8"])
def test_route_full_config_logits(name):
    cfg = w.CONFIGS[name]
    say(f"route config {name}")
    x = w.hidden_states(cfg, DEV)
    z = torch.from_numpy(oracle.router_logits(f64(x), f64(w.router_weight(cfg))))
    b = w.zipf_bias(cfg)
    idx, gate = moe.moe_route(z.to(DEV), cfg.k, None if b is None else b.to(DEV), cfg.n_group, cfg.topk_group)
    sync()
    ridx, rgate = oracle.route(z.numpy(), cfg.k, None if b is None else b.numpy(), cfg.n_group, cfg.topk_group)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(gate.cpu().numpy().astype(np.float64) - rgate).max() <= 1e-6


# ------------------------------------------------------------------------------------------
# dispatch layout
# ------------------------------------------------------------------------------------------

LAYOUT_CASES = [
    ("round_robin", 512, 256, 8, "round_robin"),
    ("hot", 1000, 64, 4, "hot"),
    ("random_small", 37, 5, 3, "random"),
    ("random_cfg3", 8192, 256, 8, "random"),
    ("random_ragged", 3001, 77, 6, "random"),
    ("N1", 1, 8, 2, "random"),
    ("E1", 129, 1, 1, "random"),
    ("k1", 4097, 8, 1, "random"),
    ("E1024", 700, 1024, 32, "random"),
    ("many_chunks", 600000, 64, 8, "random"),   # 4.8M slots: more than 4096 chunks of 1024
]


@pytest.mark.parametrize("case", LAYOUT_CASES, ids=[c[0] for c in LAYOUT_CASES])
def test_dispatch_layout_matches_oracle(case):
    name, N, E, k, kind = case
    say(f"layout {name}")
    idx = w.fixed_route(N, E, k, kind, seed=len(name))
    out1 = moe.moe_dispatch_layout(idx.to(DEV), E)
    out2 = moe.moe_dispatch_layout(idx.to(DEV), E)
    sync()
    ref = oracle.dispatch_layout(idx.numpy(), E)
    for got, r, again in zip(out1, ref, out2):
        g = got.cpu().numpy()
        assert np.array_equal(g, r)
        assert np.array_equal(g, again.cpu().numpy())  # deterministic


def test_dispatch_layout_skips_out_of_range_ids():
    N, E, k = 300, 16, 4
    idx = w.fixed_route(N, E, k, "random", seed=9).clone()
    idx[5, 1] = -1
    idx[17, 0] = E
    idx[200, 3] = 1 << 20
    n_e, off, sp, ss = moe.moe_dispatch_layout(idx.to(DEV), E)
    sync()
    flat = idx.reshape(-1).numpy()
    valid = (flat >= 0) & (flat < E)
    sp = sp.cpu().numpy()
    assert np.all(sp[~valid] == -1)
    assert np.array_equal(n_e.cpu().numpy(), np.bincount(flat[valid], minlength=E))
    assert off.cpu().numpy()[E] == valid.sum()
    assert np.array_equal(np.sort(sp[valid]), np.arange(valid.sum()))
    ss = ss.cpu().numpy()
    assert np.array_equal(ss[sp[valid]], np.nonzero(valid)[0])


# ------------------------------------------------------------------------------------------
# permute and the fp8 codec
# ------------------------------------------------------------------------------------------

PERMUTE_CASES = [
    # name, N, H, E, k, dtype
    ("bf16", 1000, 1024, 32, 4, torch.bfloat16),
    ("f32", 256, 128, 8, 2, torch.float32),
    ("bf16_H8", 33, 8, 4, 2, torch.bfloat16),
    ("bf16_k1", 100, 7168, 8, 1, torch.bfloat16),
]


@pytest.mark.parametrize("case", PERMUTE_CASES, ids=[c[0] for c in PERMUTE_CASES])
def test_permute_copy_bit_exact(case):
    name, N, H, E, k, dt = case
    say(f"permute {name}")
    x = w.normal((N, H), w.stream_key(3, w.T_X, H), DEV, dt)
    idx = w.fixed_route(N, E, k, "random", seed=N)
    _, _, sp, _ = moe.moe_dispatch_layout(idx.to(DEV), E)
    xp = moe.moe_permute(x, sp, k)
    sync()
    _, _, rsp, _ = oracle.dispatch_layout(idx.numpy(), E)
    view = torch.int16 if dt == torch.bfloat16 else torch.int32
    ref = oracle.permute(x.cpu().view(view).numpy(), rsp, k)
    assert np.array_equal(xp.cpu().view(view).numpy(), ref)


def test_round_trip_identity_experts_and_token_ids():
    """permute -> identity experts -> combine gives back x; printable ids survive."""
    N, H, E, k = 1500, 256, 64, 6
    x = torch.zeros((N, H), dtype=torch.bfloat16)
    x[:, 0] = (torch.arange(N) // 256).to(torch.bfloat16)
    x[:, 1] = (torch.arange(N) % 256).to(torch.bfloat16)
    x[:, 2:] = w.normal((N, H - 2), w.stream_key(1, w.T_X, 5), "cpu", torch.bfloat16)
    z = _logits(N, E, seed=4)
    idx, gate = moe.moe_route(z.to(DEV), k)
    n_e, off, sp, ss = moe.moe_dispatch_layout(idx, E)
    xg = x.to(DEV)
    xp = moe.moe_permute(xg, sp, k)
    y = moe.moe_combine(xp, sp, gate)
    sync()
    tok = (xp[:, 0].float() * 256 + xp[:, 1].float()).long().cpu().numpy()
    assert np.array_equal(tok, ss.cpu().numpy() // k)
    assert torch.equal(y.cpu(), x)  # sum of the gates is 1 to within 1e-7, far below a bf16 step


def _blocky(rows, cols, seed, dt=torch.bfloat16):
    """Rows with per-block magnitudes from 2^-30 to 2^12, a zero block and exact ties."""
    x = w.normal((rows, cols), w.stream_key(seed, w.T_EO, cols), "cpu", torch.float32, std=1.0)
    nb = cols // 128
    expo = (torch.arange(rows * nb) % 43 - 30).reshape(rows, nb).to(torch.float32)
    x = x * torch.repeat_interleave(torch.exp2(expo), 128, dim=1)
    x[0, :128] = 0.0
    if rows > 1:
        x[1, :128] = 3.0  # all equal: every element maps to 448
    return x.to(dt)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=["bf16_in", "f32_in"])
def test_quantize_fp8_bit_exact(dt):
    say(f"quantize {dt}")
    x = _blocky(300, 1024, 2, dt)
    q, s = moe.moe_quantize_fp8(x.to(DEV))
    sync()
    rq, rs = oracle.quantize_blocks(x.to(torch.float32).numpy())
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(q.cpu().numpy(), rq)


def test_dequantize_fp8_values():
    """Every e4m3 code under scales spread over 2^-10 .. 2^10: each value is the exact product
    (the oracle's dequantization, float64) rounded to fp32 and then to bf16, so it lies within
    half a bf16 step (2^-8 relative) plus the fp32 rounding of it; the NaN codes give NaN; zero
    codes give zero.  A scale taken
    from the wrong block, or a code decoded wrongly, misses that bound."""
    rows, cols = 64, 1024
    say("dequantize fp8")
    codes = ((np.arange(cols)[None, :] + 37 * np.arange(rows)[:, None]) % 256).astype(np.uint8)
    bits = np.asarray(w.uniform_bits(rows * cols // 128, w.stream_key(29, w.T_PERM, 0), "cpu"))
    scales = (2.0 ** ((bits >> 27).astype(np.int64) - 16) * (1.0 + (bits & 0xFFFFFF) / 2.0 ** 24)).astype(
        np.float32).reshape(rows, cols // 128)
    out = moe.moe_dequantize_fp8(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV))
    sync()
    got = f64(out)
    ref = oracle.dequantize_blocks(codes, scales)
    nan = np.isnan(ref)
    assert nan.sum() == 2 * rows * cols // 256 and np.array_equal(np.isnan(got), nan)
    assert np.all(np.abs(got[~nan] - ref[~nan]) <= (2.0 ** -8 + 2.0 ** -23) * np.abs(ref[~nan]))
    assert np.all((got[~nan] == 0) == (ref[~nan] == 0))


def test_permute_fp8_bit_exact():
    N, H, E, k = 400, 2048, 16, 4
    say("permute fp8")
    x = _blocky(N, H, 7)
    idx = w.fixed_route(N, E, k, "random", seed=3)
    _, _, sp, _ = moe.moe_dispatch_layout(idx.to(DEV), E)
    xq, xs = moe.moe_permute(x.to(DEV), sp, k, moe.MOE_FP8_E4M3)
    sync()
    _, _, rsp, _ = oracle.dispatch_layout(idx.numpy(), E)
    rq, rs = oracle.quantize_blocks(x.to(torch.float32).numpy())
    assert np.array_equal(xq.cpu().numpy(), oracle.permute(rq, rsp, k))
    assert np.array_equal(xs.cpu().numpy(), oracle.permute(rs, rsp, k))


# ------------------------------------------------------------------------------------------
# grouped GEMMs
# ------------------------------------------------------------------------------------------

GEMM_CASES = [
    # name, n_e per expert, H, I, dtype
    ("bf16_ragged", [0, 1, 127, 128, 129, 300, 0, 5], 512, 256, "bf16"),
    ("bf16_one_expert", [1000], 1024, 384, "bf16"),
    ("bf16_empty_tail", [64, 0, 0, 0], 256, 128, "bf16"),
    ("f32_ragged", [60, 0, 200, 1, 70], 256, 256, "f32"),
    ("fp8_ragged", [3, 0, 17, 128, 130, 1], 512, 256, "fp8"),
    # fp8 with hundreds of rows per expert: the down GEMM on the 256 x 256 kernel with its e4m3
    # weights converted as they are read (ragged tails, an empty expert, a one-row one)
    ("fp8_wide_down", [300, 520, 0, 700, 129, 257, 1, 640], 1024, 1024, "fp8"),
    ("bf16_wide_K", [200, 90], 7168, 256, "bf16"),
    # experts of 257..320 rows as one 320-row tile, beside 256-row tiles with ragged column
    # blocks (H = 640: two and a half 256-column blocks of the down GEMM)
    ("bf16_tall", [257, 320, 288, 0, 289, 256, 321, 1], 640, 384, "bf16"),
    # the same at K = 128 and K = 256 (fewer stages than the 320-row tile's weight ring runs ahead)
    ("bf16_tall_k128", [300, 5, 260], 128, 128, "bf16"),
    ("bf16_tall_k256", [300, 257, 40], 256, 256, "bf16"),
    # at most 16 rows per expert on average with e4m3 weights: the weight-streaming kernels
    ("fp8_decode_ragged", [0, 1, 2, 5, 16, 17, 33, 0, 3, 0, 9, 1, 4, 0, 7, 12], 1024, 256, "fp8"),
    ("fp8_decode_one_k_block", [1, 0], 128, 128, "fp8"),
    ("fp8_decode_wide", [4, 0, 7], 7168, 2048, "fp8"),
    ("fp8_decode_odd_k_blocks", [2, 16, 0, 9], 1152, 384, "fp8"),   # 9 and 3 K blocks: scales one by one
    ("fp8_decode_16_per_expert", [16] * 8, 512, 256, "fp8"),        # rows = 16 E exactly
]


def _gemm_inputs(n_e, H, I, dtype, seed):
    E, rows = len(n_e), sum(n_e)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    a = w.normal((rows, H), w.stream_key(seed, w.T_X, 1), DEV, dt)
    w13 = w.normal((E, 2 * I, H), w.stream_key(seed, w.T_W13, 1), DEV, dt)
    w2 = w.normal((E, H, I), w.stream_key(seed, w.T_W2, 1), DEV, dt)
    offs = torch.tensor(np.concatenate([[0], np.cumsum(n_e)]), dtype=torch.int32, device=DEV)
    return a, w13, w2, offs


@pytest.mark.parametrize("case", GEMM_CASES, ids=[c[0] for c in GEMM_CASES])
def test_grouped_ffn_matches_oracle(case):
    name, n_e, H, I, dtype = case
    say(f"gemm {name}")
    a, w13, w2, offs = _gemm_inputs(n_e, H, I, dtype, seed=len(name))
    offs_np = offs.cpu().numpy()
    if dtype == "fp8":
        aq, asc = moe.moe_quantize_fp8(a)
        q13, s13 = moe.moe_quantize_fp8(w13)
        q2, s2 = moe.moe_quantize_fp8(w2)
        h = moe.moe_expert_gate_up(aq, offs, q13, asc, s13)
        out = moe.moe_expert_down(h, offs, q2, s2)
        out2 = moe.moe_grouped_ffn(aq, offs, q13, q2, asc, s13, s2)
        sync()
        ra = oracle.dequantize_blocks(*oracle.quantize_blocks(a.float().cpu().numpy()))
        E = len(n_e)
        r13 = [oracle.dequantize_blocks(*oracle.quantize_blocks(w13[e].float().cpu().numpy())) for e in range(E)]
        r2 = [oracle.dequantize_blocks(*oracle.quantize_blocks(w2[e].float().cpu().numpy())) for e in range(E)]
        rh, rout = oracle.grouped_ffn(ra, offs_np, lambda e: r13[e], lambda e: r2[e])
        bar = 1e-2
    else:
        h = moe.moe_expert_gate_up(a, offs, w13)
        out = moe.moe_expert_down(h, offs, w2)
        out2 = moe.moe_grouped_ffn(a, offs, w13, w2)
        sync()
        rh, rout = oracle.grouped_ffn(f64(a), offs_np, f64(w13), f64(w2))
        bar = 1e-5 if dtype == "f32" else 1e-2
    assert token_rel_err(f64(h), rh) <= bar
    assert token_rel_err(f64(out), rout) <= bar
    assert torch.equal(out, out2)


@pytest.mark.parametrize("E,k,N,H,I,mode", [(16, 4, 300, 512, 256, "random"), (8, 2, 1000, 1024, 384, "hot"),
                                             (64, 8, 96, 7168, 256, "random"), (4, 1, 333, 256, 128, "random")])
def test_gate_up_gathered_equals_permuted(E, k, N, H, I, mode):
    """Gate/up reading rows straight from x through src_slot == permute then gate/up, bit for bit."""
    say(f"gathered gate/up E={E} k={k} N={N} H={H} I={I} {mode}")
    x = w.normal((N, H), w.stream_key(11, w.T_X, E), DEV, torch.bfloat16)
    w13 = w.normal((E, 2 * I, H), w.stream_key(11, w.T_W13, E), DEV, torch.bfloat16)
    idx = w.fixed_route(N, E, k, mode, seed=E)
    n_e, offs, sp, ss = moe.moe_dispatch_layout(idx.to(DEV), E)
    xp = moe.moe_permute(x, sp, k)
    h_ref = moe.moe_expert_gate_up(xp, offs, w13)
    h = moe.moe_expert_gate_up_gathered(x, ss, k, offs, w13)
    sync()
    assert torch.equal(h.view(torch.int16), h_ref.view(torch.int16))
    # and against the oracle on every row
    rows = np.arange(N * k)
    o = offs.cpu().numpy()
    ref = np.zeros((N * k, I))
    xf, wf, toks = f64(x), f64(w13), ss.cpu().numpy() // k
    for e in range(E):
        r = rows[o[e]:o[e + 1]]
        if len(r):
            ref[r] = oracle.expert_ffn(xf[toks[r]], wf[e], np.zeros((H, I)))[0]
    assert token_rel_err(f64(h), ref) <= 1e-2


def test_expert_down_on_generated_h():
    """The down GEMM alone, on an h that no other kernel produced."""
    n_e, H, I = [70, 0, 300, 3], 1024, 512
    rows, E = sum(n_e), len(n_e)
    h = w.normal((rows, I), w.stream_key(8, w.T_EO, 2), DEV, torch.bfloat16, std=0.05)
    w2 = w.normal((E, H, I), w.stream_key(8, w.T_W2, 2), DEV, torch.bfloat16)
    offs = torch.tensor(np.concatenate([[0], np.cumsum(n_e)]), dtype=torch.int32, device=DEV)
    out = moe.moe_expert_down(h, offs, w2)
    sync()
    ref = np.zeros((rows, H))
    o = offs.cpu().numpy()
    hh, ww = f64(h), f64(w2)
    for e in range(E):
        ref[o[e]:o[e + 1]] = hh[o[e]:o[e + 1]] @ ww[e].T
    # fp32 accumulation then one bf16 rounding: within one bf16 step of the exact value
    got = f64(out)
    assert np.all(np.abs(got - ref) <= bf16_ulp(ref) + 1e-6 * np.abs(ref).max())


@pytest.mark.parametrize("n_e", [[16] * 16, [128, 128]], ids=["streaming", "tiled"])
def test_expert_down_e4m3_weights_every_code(n_e):
    """Down GEMM on e4m3 weights holding every finite code, read back exactly.

    Row r of h is one-hot at K index r, so out[r, n] = decode(W_e[n, r]) * s_e[n, r // 128]
    with no rounding, also not in the bf16 output: the scales 1, 1.25, 1.5, 1.75 keep every
    product within 8 significant bits.  Across n the codes (n + 7 r + 3 e) mod 256 take
    every value (NaN codes 0x7f and 0xff replaced by 0), so each row checks every code's
    conversion.
    """
    E, rows, I, H = len(n_e), sum(n_e), 256, 256
    say(f"down e4m3 every code, n_e {n_e[:2]}...")
    h = torch.zeros((rows, I), dtype=torch.bfloat16)
    h[torch.arange(rows), torch.arange(rows)] = 1.0
    n = np.arange(H)[None, :, None]
    kk = np.arange(I)[None, None, :]
    ee = np.arange(E)[:, None, None]
    codes = ((n + 7 * kk + 3 * ee) % 256).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    scale = (1.0 + ((np.arange(H)[None, :, None] + np.arange(I // 128)[None, None, :]) % 4) / 4.0)
    scale = np.broadcast_to(scale, (E, H, I // 128)).astype(np.float32)
    offs = torch.tensor(np.concatenate([[0], np.cumsum(n_e)]), dtype=torch.int32, device=DEV)
    q2, s2 = torch.from_numpy(codes).to(DEV), torch.from_numpy(np.ascontiguousarray(scale)).to(DEV)
    out = moe.moe_expert_down(h.to(DEV), offs, q2, s2)
    sync()
    expert = np.repeat(np.arange(E), n_e)
    r = np.arange(rows)
    ref = oracle.e4m3_decode(codes[expert, :, r]) * scale[expert, :, r // 128].astype(np.float64)
    assert np.array_equal(f64(out), ref)


# ------------------------------------------------------------------------------------------
# combine
# ------------------------------------------------------------------------------------------

COMBINE_CASES = [
    ("bf16_shared", 700, 1024, 32, 8, torch.bfloat16, True),
    ("bf16", 513, 7168, 16, 2, torch.bfloat16, False),
    ("f32", 256, 128, 8, 2, torch.float32, False),
    ("k3", 100, 64, 8, 3, torch.bfloat16, True),
    ("k32", 50, 256, 64, 32, torch.bfloat16, False),
    ("k5_f32_shared", 64, 512, 16, 5, torch.float32, True),
    ("k1", 77, 8, 4, 1, torch.bfloat16, False),
    ("k8_spans", 3, 7168, 256, 8, torch.bfloat16, True),     # a few tokens: rows split into spans
    ("k12", 40, 1024, 32, 12, torch.bfloat16, True),
]


@pytest.mark.parametrize("case", COMBINE_CASES, ids=[c[0] for c in COMBINE_CASES])
def test_combine_matches_oracle(case):
    name, N, H, E, k, dt, shared = case
    say(f"combine {name}")
    cfg = w.CONFIGS["tiny_f32"]
    eo = w.synthetic_rows(N * k, H, 11, cfg, DEV, dt)
    sh = w.synthetic_rows(N, H, 12, cfg, DEV, dt) if shared else None
    gate = w.random_gates(N, k, seed=5)
    idx = w.fixed_route(N, E, k, "random", seed=6)
    _, _, sp, _ = moe.moe_dispatch_layout(idx.to(DEV), E)
    y = moe.moe_combine(eo, sp, gate.to(DEV), sh)
    sync()
    _, _, rsp, _ = oracle.dispatch_layout(idx.numpy(), E)
    ref = oracle.combine(f64(eo), rsp, gate.numpy().astype(np.float64), k, None if sh is None else f64(sh))
    got = f64(y)
    if dt == torch.float32:
        assert token_rel_err(got, ref) <= 1e-6
    else:
        # fp32 sum of k+1 terms, then one rounding: within one bf16 step of the rounded
        # exact sum, plus the fp32 accumulation bound (k+1) * 2^-24 * sum of |terms|
        # (which dominates where the sum cancels to almost nothing)
        mag = oracle.combine(np.abs(f64(eo)), rsp, np.abs(gate.numpy().astype(np.float64)), k,
                             None if sh is None else np.abs(f64(sh)))
        tol = bf16_ulp(ref) * 1.0001 + (k + 1) * 2.0 ** -24 * mag
        assert np.all(np.abs(got - bf16_round(ref)) <= tol)


def test_generator_device_matches_host():
    """The counter-based generator gives the same tensors on the GPU as on the CPU."""
    cfg = w.CONFIGS["dsv3_bf16"].scaled(E=7, H=512, I=256)
    g13, g2 = w.all_expert_weights(cfg, DEV)
    c13, c2 = w.all_expert_weights(cfg, "cpu")
    assert torch.equal(g13.cpu(), c13) and torch.equal(g2.cpu(), c2)
    assert torch.equal(w.hidden_states(cfg, DEV).cpu(), w.hidden_states(cfg, "cpu"))


@pytest.mark.parametrize("ratio", [1, 9, 16])
def test_stream_probe_sums(ratio):
    """The read-mostly streaming probe (a measurement utility): dst[i] = the 32-bit integer
    sum of src[j * n + i] over j, lane by lane."""
    n16 = 3000
    src = (torch.arange(ratio * n16 * 4, dtype=torch.int64) * 2654435761 % (1 << 32)).to(torch.int64)
    src32 = (src - (src >= (1 << 31)).to(torch.int64) * (1 << 32)).to(torch.int32)
    dst = moe.moe_stream_probe(src32.to(DEV).view(torch.uint8), ratio)
    sync()
    ref = src.reshape(ratio, n16 * 4).sum(0) % (1 << 32)
    got = dst.cpu().view(torch.int32).to(torch.int64) % (1 << 32)
    assert torch.equal(got, ref)
