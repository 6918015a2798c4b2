"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: every expected value is a
closed form, an invariant, a library routine (torch / scipy), a brute force
written independently in this file, or a figure the pages print
(tests/golden).  Mutation tests at the end plant plausible mistakes in the
oracle and check that these pins catch each of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import expit, softmax

from oracle import moe_oracle as oracle
import workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------------------------------
# router logits
# ------------------------------------------------------------------------------------------

def brute_router_logits(x, w):
    """Each logit as the correctly rounded sum (math.fsum) of its H products, then fp32."""
    N, H = x.shape
    E = w.shape[0]
    z = np.empty((N, E), np.float32)
    for t in range(N):
        for e in range(E):
            z[t, e] = np.float32(math.fsum(float(x[t, h]) * float(w[e, h]) for h in range(H)))
    return z


def check_router_vs_bruteforce():
    rng = _rng(11)
    # dyadic values: every product and every partial sum is exact in float64
    x = rng.integers(-16, 17, size=(5, 9)) / 16.0
    w = rng.integers(-16, 17, size=(4, 9)) / 32.0
    if not np.array_equal(oracle.router_logits(x, w), brute_router_logits(x, w)):
        return False
    x = rng.standard_normal((7, 33)) * 0.02
    w = rng.standard_normal((6, 33)) * 0.02
    z = oracle.router_logits(x, w)
    ref = brute_router_logits(x, w)
    # a float64 sum lands within one fp32 ulp of the correctly rounded one
    return z.shape == (7, 6) and bool(np.all(np.abs(z.astype(np.float64) - ref) <= np.spacing(np.abs(ref))))


def check_router_selects_permuted_columns():
    """Rows of W_r that are unit vectors: W_r[e] = u_{pi(e)} gives z[:, e] = x[:, pi(e)] exactly."""
    perm = np.array([2, 0, 3, 5, 1, 4])   # not its own inverse: a transposed W_r would give pi^-1
    w = np.zeros((6, 6))
    w[np.arange(6), perm] = 1.0
    x = _rng(12).standard_normal((4, 6)).astype(np.float32)
    return bool(np.array_equal(oracle.router_logits(x, w), x[:, perm]))


def test_router_logits_match_bruteforce():
    assert check_router_vs_bruteforce()


def test_router_logits_unit_rows_select_columns():
    assert check_router_selects_permuted_columns()


def test_router_logits_ones_give_row_sums():
    w = _rng(13).standard_normal((5, 40))
    z = oracle.router_logits(np.ones((2, 40)), w)
    ref = np.array([math.fsum(r) for r in w])
    assert z.shape == (2, 5) and z.dtype == np.float32
    assert np.all(np.abs(z - ref[None, :]) <= np.spacing(np.abs(ref).astype(np.float32))[None, :])


# ------------------------------------------------------------------------------------------
# backward: analytic gradients against central differences of the forward
# ------------------------------------------------------------------------------------------

def _train_case(seed=21, N=5, H=8, E=4, k=2, I=4):
    rng = _rng(seed)
    return dict(x=rng.standard_normal((N, H)) * 0.5, w_r=rng.standard_normal((E, H)) * 0.5,
                w13=rng.standard_normal((E, 2 * I, H)) * 0.5, w2=rng.standard_normal((E, H, I)) * 0.5,
                sw13=rng.standard_normal((2 * I, H)) * 0.5, sw2=rng.standard_normal((H, I)) * 0.5,
                bias=rng.standard_normal(E) * 0.1, c=rng.standard_normal((N, H)), k=k)


def _smooth_loss(p, idx):
    """L = sum(c * y) with the routes fixed to idx and every step in float64: z = x W_r^T + b
    (no fp32 rounding), gates = scipy's softmax over the selected logits, each slot's expert
    and the shared expert evaluated token by token from the SwiGLU definition."""
    x, w13, w2 = p["x"], p["w13"], p["w2"]
    I = w13.shape[1] // 2
    zb = x @ p["w_r"].T + p["bias"][None, :]
    g = softmax(np.take_along_axis(zb, idx, axis=1), axis=1)

    def ffn(xt, a13, a2):
        ga, up = a13[:I] @ xt, a13[I:] @ xt
        return a2 @ (ga * expit(ga) * up)
    y = np.zeros_like(x)
    for t in range(x.shape[0]):
        for j in range(idx.shape[1]):
            y[t] += g[t, j] * ffn(x[t], w13[idx[t, j]], w2[idx[t, j]])
        y[t] += ffn(x[t], p["sw13"], p["sw2"])
    return float((p["c"] * y).sum())


def _central_diff(p, name, idx, eps=1e-6):
    base = p[name]
    out = np.zeros_like(base)
    for i in np.ndindex(base.shape):
        old = base[i]
        base[i] = old + eps
        lp = _smooth_loss(p, idx)
        base[i] = old - eps
        lm = _smooth_loss(p, idx)
        base[i] = old
        out[i] = (lp - lm) / (2 * eps)
    return out


def check_backward_fd(seed=21):
    p = _train_case(seed)
    E = p["w13"].shape[0]
    z = oracle.router_logits(p["x"], p["w_r"])
    b = oracle.moe_layer_backward(p["x"], z, p["k"], p["w13"], p["w2"], p["c"], bias=p["bias"],
                                  shared_w13=p["sw13"], shared_w2=p["sw2"], w_r=p["w_r"])
    idx = b["fwd"]["topk_idx"].astype(np.int64)
    dw13 = np.stack([b["dw13"].get(e, np.zeros_like(p["w13"][0])) for e in range(E)])
    dw2 = np.stack([b["dw2"].get(e, np.zeros_like(p["w2"][0])) for e in range(E)])
    got = dict(x=b["dx"], w_r=b["dw_r"], w13=dw13, w2=dw2, sw13=b["shared_dw13"], sw2=b["shared_dw2"])
    # the oracle's gates come from fp32 logits: ~1e-7 relative next to the smooth float64 ones
    return all(np.allclose(got[n], _central_diff(p, n, idx), rtol=1e-5, atol=1e-6) for n in got)


def test_backward_matches_central_differences():
    assert check_backward_fd(21)
    assert check_backward_fd(22)


def test_dispatch_backward_is_the_adjoint_of_permute():
    rng = _rng(23)
    N, k, H, E = 7, 3, 5, 6
    idx = workload.fixed_route(N, E, k, "random", seed=23).numpy()
    _, _, send_pos, _ = oracle.dispatch_layout(idx, E)
    x = rng.standard_normal((N, H))
    Y = rng.standard_normal((N * k, H))
    lhs = float((oracle.permute(x, send_pos, k) * Y).sum())
    rhs = float((x * oracle.dispatch_backward(Y, send_pos, N, k)).sum())
    assert abs(lhs - rhs) <= 1e-12 * (abs(lhs) + 1)


def test_gates_backward_matches_softmax_jacobian():
    rng = _rng(24)
    zsel = rng.standard_normal((4, 3))
    g = softmax(zsel, axis=1)
    dg = rng.standard_normal((4, 3))
    jac = np.einsum("ti,ij->tij", g, np.eye(3)) - np.einsum("ti,tj->tij", g, g)   # d g_i / d z_j
    assert np.allclose(oracle.gates_backward(g, dg), np.einsum("ti,tij->tj", dg, jac), rtol=1e-12, atol=1e-15)
    # one expert per token: the gate is constant 1, no gradient reaches the logit
    assert np.array_equal(oracle.gates_backward(np.ones((3, 1)), rng.standard_normal((3, 1))), np.zeros((3, 1)))


# ------------------------------------------------------------------------------------------
# top-k selection
# ------------------------------------------------------------------------------------------

def brute_topk_set(zrow, k, allowed=None):
    """Over all k-subsets of allowed experts, the one with the largest logit sum.

    For distinct logits this is exactly the set of the k largest ones.
    """
    cand = [e for e in range(len(zrow)) if allowed is None or allowed[e]]
    best = max(itertools.combinations(cand, k), key=lambda s: sum(float(zrow[e]) for e in s))
    return set(best)


def check_topk_vs_bruteforce(seed=0, N=40, E=7, k=3):
    z = _rng(seed).standard_normal((N, E)).astype(np.float32)
    idx = oracle.topk_select(z, k)
    for t in range(N):
        if set(idx[t].tolist()) != brute_topk_set(z[t], k):
            return False
        if not all(z[t, idx[t, j]] > z[t, idx[t, j + 1]] for j in range(k - 1)):
            return False
    return True


def test_topk_matches_bruteforce_subset_search():
    assert check_topk_vs_bruteforce()


def test_topk_matches_torch_topk_on_distinct_logits():
    z = _rng(1).standard_normal((500, 64)).astype(np.float32)
    ref = torch.topk(torch.from_numpy(z), 8, dim=1, sorted=True).indices.numpy()
    assert np.array_equal(oracle.topk_select(z, 8), ref)


def test_topk_tie_break_lower_index_first():
    z = np.array([[1, 3, 3, 2, 3], [0, 0, 0, 0, 0]], dtype=np.float32)
    assert oracle.topk_select(z, 2).tolist() == [[1, 2], [0, 1]]
    assert oracle.topk_select(z, 4).tolist() == [[1, 2, 4, 3], [0, 1, 2, 3]]


def test_topk_signed_zeros_are_equal():
    z = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], dtype=np.float32)
    assert oracle.topk_select(z, 1).tolist() == [[0], [0]]


def test_topk_k_equals_E_is_a_full_descending_sort():
    z = _rng(2).standard_normal((30, 9)).astype(np.float32)
    assert np.array_equal(oracle.topk_select(z, 9), np.argsort(-z, axis=1, kind="stable"))


# ------------------------------------------------------------------------------------------
# group-limited routing
# ------------------------------------------------------------------------------------------

def check_group_limit_vs_bruteforce(seed=3, N=30, n_group=4, G=3, topk_group=2, k=3):
    E = n_group * G
    z = _rng(seed).standard_normal((N, E)).astype(np.float32)
    idx, _ = oracle.route(z, k, n_group=n_group, topk_group=topk_group)
    for t in range(N):
        score = [float(z[t, g * G:(g + 1) * G].max()) for g in range(n_group)]
        groups = max(itertools.combinations(range(n_group), topk_group),
                     key=lambda s: sum(score[g] for g in s))
        allowed = np.zeros(E, dtype=bool)
        for g in groups:
            allowed[g * G:(g + 1) * G] = True
        if set(idx[t].tolist()) != brute_topk_set(z[t], k, allowed):
            return False
    return True


def test_group_limit_matches_bruteforce_over_group_subsets():
    assert check_group_limit_vs_bruteforce()


def test_group_limit_hand_example():
    # 4 groups of 2; group maxima 0.9, 0.6, 0.95, 0.3 -> groups 2 and 0 are kept
    z = np.array([[0.9, 0.1, 0.5, 0.6, 0.95, -1.0, 0.2, 0.3]], dtype=np.float32)
    idx, _ = oracle.route(z, 3, n_group=4, topk_group=2)
    assert idx.tolist() == [[4, 0, 1]]
    idx_plain, _ = oracle.route(z, 3)
    assert idx_plain.tolist() == [[4, 0, 3]]


def test_group_limit_all_groups_is_plain_topk():
    z = _rng(4).standard_normal((200, 32)).astype(np.float32)
    a, ga = oracle.route(z, 6, n_group=8, topk_group=8)
    b, gb = oracle.route(z, 6)
    assert np.array_equal(a, b) and np.array_equal(ga, gb)


def test_group_limit_pages_example_two_of_eight():
    fx = json.load(open(os.path.join(GOLDEN, "group_limited_example.json")))
    ng, tg = fx["n_group_example"], fx["topk_group_example"]
    E, k = 64, 8
    G = E // ng
    z = _rng(5).standard_normal((300, E)).astype(np.float32)
    idx, _ = oracle.route(z, k, n_group=ng, topk_group=tg)
    for t in range(300):
        used = {int(e) // G for e in idx[t]}
        assert len(used) <= tg
        gmax = z[t].reshape(ng, G).max(axis=1)
        assert used <= set(np.argsort(-gmax, kind="stable")[:tg].tolist())


# ------------------------------------------------------------------------------------------
# gates
# ------------------------------------------------------------------------------------------

def check_gates_vs_full_softmax(seed=6, N=100, E=16, k=4):
    z = _rng(seed).standard_normal((N, E)).astype(np.float32)
    idx, g = oracle.route(z, k)
    p = softmax(z.astype(np.float64), axis=1)
    sel = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    ref = sel / sel.sum(axis=1, keepdims=True)
    return np.allclose(g, ref, rtol=1e-12, atol=1e-15)


def test_gates_are_full_softmax_restricted_and_renormalized():
    assert check_gates_vs_full_softmax()


def test_gates_sum_to_one_and_k1_is_one():
    z = _rng(7).standard_normal((50, 12)).astype(np.float32)
    _, g = oracle.route(z, 5)
    assert np.allclose(g.sum(axis=1), 1.0, atol=1e-14)
    _, g1 = oracle.route(z, 1)
    assert np.all(g1 == 1.0)


def test_gates_two_experts_closed_form():
    z = np.array([[0.7, -0.2, -5.0], [2.0, 2.5, 0.0]], dtype=np.float32)
    idx, g = oracle.route(z, 2)
    zz = z.astype(np.float64)
    assert idx.tolist() == [[0, 1], [1, 0]]
    assert math.isclose(g[0, 0], expit(zz[0, 0] - zz[0, 1]), rel_tol=1e-14)
    assert math.isclose(g[1, 0], expit(zz[1, 1] - zz[1, 0]), rel_tol=1e-14)


def test_bias_enters_selection_and_gates():
    z = np.array([[1.0, 0.0, 0.5]], dtype=np.float32)
    b = np.array([0.0, 2.0, 0.0], dtype=np.float32)
    idx, g = oracle.route(z, 2, bias=b)
    assert idx.tolist() == [[1, 0]]
    assert math.isclose(g[0, 0], expit(2.0 - 1.0), rel_tol=1e-14)


def test_gates_shift_invariant():
    z = _rng(8).standard_normal((40, 10)).astype(np.float32)
    _, g = oracle.route(z, 3)
    _, g2 = oracle.route(z, 3, bias=np.full(10, 0.25, dtype=np.float32))
    assert np.allclose(g, g2, atol=1e-6)


# ------------------------------------------------------------------------------------------
# dispatch layout
# ------------------------------------------------------------------------------------------

def brute_layout(idx, E):
    """Direct counting from the definitions, one pair at a time."""
    N, k = len(idx), len(idx[0])
    n_e = [0] * E
    for t in range(N):
        for j in range(k):
            n_e[idx[t][j]] += 1
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + n_e[e])
    send_pos = []
    for t in range(N):
        for j in range(k):
            e = idx[t][j]
            before = sum(1 for t2 in range(t) for j2 in range(k) if idx[t2][j2] == e)
            send_pos.append(offsets[e] + before)
    return n_e, offsets, send_pos


def check_layout_invariants(idx, E):
    N, k = idx.shape
    n_e, off, sp, ss = oracle.dispatch_layout(idx, E)
    flat = idx.reshape(-1)
    ok = n_e.sum() == N * k and off[0] == 0 and off[E] == N * k
    ok &= np.array_equal(np.sort(sp), np.arange(N * k))          # bijection
    ok &= np.array_equal(ss[sp], np.arange(N * k))               # src_slot o send_pos = id
    for e in range(E):
        seg = ss[off[e]:off[e + 1]]
        ok &= bool(np.all(flat[seg] == e))                       # segment holds expert e only
        ok &= bool(np.all(np.diff(seg // k) > 0))                # ascending tokens
        ok &= len(seg) == n_e[e]
    return bool(ok)


def test_layout_bruteforce_tiny():
    for seed, (N, E, k) in enumerate([(9, 5, 2), (13, 8, 3), (1, 4, 4), (20, 3, 1)]):
        idx = workload.fixed_route(N, E, k, "random", seed=seed).numpy()
        n_e, off, sp, _ = oracle.dispatch_layout(idx, E)
        bn, bo, bs = brute_layout(idx.tolist(), E)
        assert n_e.tolist() == bn and off.tolist() == bo and sp.tolist() == bs


def test_layout_invariants_random_routes():
    for seed, (N, E, k) in enumerate([(300, 16, 4), (77, 256, 8), (64, 8, 2)]):
        idx = workload.fixed_route(N, E, k, "random", seed=seed).numpy()
        assert check_layout_invariants(idx, E)


def test_layout_round_robin_closed_form():
    N, E, k = 512, 256, 8
    idx = workload.fixed_route(N, E, k, "round_robin").numpy()
    n_e, off, _, _ = oracle.dispatch_layout(idx, E)
    assert np.all(n_e == N * k // E)
    assert np.array_equal(off, np.arange(E + 1) * (N * k // E))
    assert oracle.imbalance(n_e) == 1.0


def test_layout_hot_route_closed_form():
    N, E, k = 100, 16, 4
    idx = workload.fixed_route(N, E, k, "hot").numpy()
    n_e, off, sp, _ = oracle.dispatch_layout(idx, E)
    assert n_e.tolist() == [N] * k + [0] * (E - k)
    assert oracle.imbalance(n_e) == E / k
    # token t's j-th pair lands at row j*N + t
    assert np.array_equal(sp.reshape(N, k), np.arange(k)[None, :] * N + np.arange(N)[:, None])


def test_decode_capacity_example_from_pages():
    fx = json.load(open(os.path.join(GOLDEN, "decode_capacity.json")))
    E, k, N = fx["E"], fx["k"], fx["N_active"]
    for kind in ("round_robin", "random"):
        idx = workload.fixed_route(N, E, k, kind).numpy()
        n_e, _, _, _ = oracle.dispatch_layout(idx, E)
        assert n_e.mean() == fx["m_target"]            # mean n_e = N k / E
    assert N * k / E == fx["m_target"]


# ------------------------------------------------------------------------------------------
# permute / combine round trip (identity experts) and printable token ids
# ------------------------------------------------------------------------------------------

def test_round_trip_identity_experts():
    N, E, k, H = 200, 12, 3, 16
    z = _rng(9).standard_normal((N, E)).astype(np.float32)
    x = _rng(10).standard_normal((N, H))
    idx, g = oracle.route(z, k)
    _, _, sp, _ = oracle.dispatch_layout(idx, E)
    xp = oracle.permute(x, sp, k)
    y = oracle.combine(xp, sp, g, k)                 # identity experts
    assert np.allclose(y, x * g.sum(axis=1, keepdims=True), rtol=1e-14)
    assert np.allclose(y, x, rtol=1e-13)


def test_printable_token_ids_survive_permutation():
    N, E, k = 700, 32, 4
    idx = workload.fixed_route(N, E, k, "random", seed=11).numpy()
    x = np.zeros((N, 2), dtype=np.float32)
    x[:, 0] = np.arange(N) // 256
    x[:, 1] = np.arange(N) % 256
    n_e, off, sp, ss = oracle.dispatch_layout(idx, E)
    xp = oracle.permute(x, sp, k)
    tok = (xp[:, 0] * 256 + xp[:, 1]).astype(np.int64)
    assert np.array_equal(tok, ss // k)
    for e in range(E):
        rows = slice(off[e], off[e + 1])
        assert all(e in idx[t] for t in tok[rows])


def test_combine_bruteforce_per_token():
    N, k, H = 37, 3, 5
    eo = _rng(12).standard_normal((N * k, H))
    sp = _rng(13).permutation(N * k)
    g = _rng(14).random((N, k))
    sh = _rng(15).standard_normal((N, H))
    y = oracle.combine(eo, sp, g, k, sh)
    for t in range(N):
        ref = sh[t].copy()
        for j in range(k):
            ref = ref + g[t, j] * eo[sp[t * k + j]]
        assert np.allclose(y[t], ref, rtol=1e-14, atol=1e-15)


# ------------------------------------------------------------------------------------------
# fp8 e4m3 codec
# ------------------------------------------------------------------------------------------

def _all_finite_codes():
    return np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e4m3_encode_round_trips_every_code():
    codes = _all_finite_codes()
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    back = oracle.e4m3_encode(vals)
    zero_neg = codes == 0x80                      # -0 encodes to 0x80 as well (sign kept)
    assert np.array_equal(back, codes) or np.array_equal(back[~zero_neg], codes[~zero_neg])


def test_e4m3_encode_midpoints_round_to_even():
    pos = np.sort(oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = (pos[:-1] + pos[1:]) / 2
    got = oracle.e4m3_encode(mids.astype(np.float32))
    lo_code = oracle.e4m3_encode(pos[:-1].astype(np.float32))
    hi_code = oracle.e4m3_encode(pos[1:].astype(np.float32))
    want = np.where(lo_code % 2 == 0, lo_code, hi_code)
    assert np.array_equal(got, want)
    # a few by hand: 2^-10 is halfway between 0 and 2^-9 -> 0; 3*2^-10 -> 2^-8 (code 2)
    assert oracle.e4m3_encode(np.array([2.0 ** -10, 3 * 2.0 ** -10], np.float32)).tolist() == [0, 2]


def test_e4m3_encode_vs_torch_cast_after_clamp():
    v = (_rng(16).standard_normal(200000) * np.exp(_rng(17).uniform(-12, 7, 200000))).astype(np.float32)
    clamped = np.clip(v, -448, 448)
    ref = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(v), ref)


def test_e4m3_saturates():
    v = np.array([448, 449, 464, 479.9, 500, 1e30, -465, -1e9], dtype=np.float32)
    assert oracle.e4m3_decode(oracle.e4m3_encode(v)).tolist() == [448.0] * 6 + [-448.0] * 2


def test_quantize_blocks_properties():
    x = _rng(18).standard_normal((64, 512)).astype(np.float32) * 0.02
    x[3, 128:256] = 0.0
    q, s = oracle.quantize_blocks(x)
    assert q.shape == x.shape and s.shape == (64, 4) and s.dtype == np.float32
    xb = x.reshape(64, 4, 128)
    amax = np.abs(xb).max(axis=2)
    assert s[3, 1] == 1.0 and np.all(q[3, 128:256] == 0)
    nz = amax > 0
    assert np.array_equal(s[nz], (amax[nz] / np.float32(448)).astype(np.float32))
    deq = oracle.dequantize_blocks(q, s).reshape(64, 4, 128)
    # the block's largest magnitude maps to 448 (to within the fp32 rounding of s)
    arg = np.abs(xb).argmax(axis=2)
    top = np.abs(oracle.e4m3_decode(np.take_along_axis(q.reshape(64, 4, 128), arg[..., None], 2)))
    assert np.all(top[nz] == 448.0)
    # relative error of each element within half an e4m3 step (2^-4) plus the subnormal floor
    err = np.abs(deq - xb)
    assert np.all(err <= np.abs(xb) * 2.0 ** -4 + (s[..., None] * 2.0 ** -10) * 1.0001)


# ------------------------------------------------------------------------------------------
# expert SwiGLU FFN and the whole layer
# ------------------------------------------------------------------------------------------

def test_silu_closed_form():
    a = np.linspace(-20, 20, 1001)
    assert np.allclose(oracle.silu(a), a * expit(a), rtol=1e-14, atol=1e-300)
    assert oracle.silu(np.array([0.0]))[0] == 0.0


def test_expert_ffn_scalar_hand_example():
    # H = I = 1: gate = 2*x, up = 3*x, down = 0.5 -> out = 0.5 * silu(2) * 3 at x = 1
    h, out = oracle.expert_ffn(np.array([[1.0]]), np.array([[2.0], [3.0]]), np.array([[0.5]]))
    assert math.isclose(out[0, 0], 0.5 * 3.0 * 2.0 / (1.0 + math.exp(-2.0)), rel_tol=1e-15)
    assert math.isclose(h[0, 0], 3.0 * 2.0 / (1.0 + math.exp(-2.0)), rel_tol=1e-15)


def check_dense_reduction(seed=19, N=33, H=24, I=40):
    """E = 1, k = 1: the layer is one dense SwiGLU MLP (torch float64 as the library reference)."""
    x = _rng(seed).standard_normal((N, H))
    w13 = _rng(seed + 1).standard_normal((1, 2 * I, H)) * 0.2
    w2 = _rng(seed + 2).standard_normal((1, H, I)) * 0.2
    z = np.zeros((N, 1), dtype=np.float32)
    res = oracle.moe_layer(x, z, 1, w13, w2)
    xt = torch.from_numpy(x)
    wg, wu, wd = (torch.from_numpy(w13[0, :I]), torch.from_numpy(w13[0, I:]), torch.from_numpy(w2[0]))
    ref = (torch.nn.functional.silu(xt @ wg.T) * (xt @ wu.T)) @ wd.T
    return np.allclose(res["y"], ref.numpy(), rtol=1e-12, atol=1e-14)


def test_single_expert_layer_is_dense_swiglu_mlp():
    assert check_dense_reduction()


def check_layer_vs_per_token_definition(seed=20, N=24, H=16, E=6, k=2, I=12, n_group=0, topk_group=0,
                                        shared=False):
    r = _rng(seed)
    x = r.standard_normal((N, H))
    z = r.standard_normal((N, E)).astype(np.float32)
    w13 = r.standard_normal((E, 2 * I, H)) * 0.3
    w2 = r.standard_normal((E, H, I)) * 0.3
    sw13 = r.standard_normal((2 * I, H)) * 0.3 if shared else None
    sw2 = r.standard_normal((H, I)) * 0.3 if shared else None
    res = oracle.moe_layer(x, z, k, w13, w2, n_group=n_group, topk_group=topk_group,
                           shared_w13=sw13, shared_w2=sw2)
    ok = True
    for t in range(N):
        # y_t = sum_{e in I_t} g_{t,e} Expert_e(x_t), written out token by token with torch
        xt = torch.from_numpy(x[t:t + 1])
        acc = torch.zeros(1, H, dtype=torch.float64)
        for j in range(k):
            e = int(res["topk_idx"][t, j])
            wg, wu = torch.from_numpy(w13[e, :I]), torch.from_numpy(w13[e, I:])
            out = (torch.nn.functional.silu(xt @ wg.T) * (xt @ wu.T)) @ torch.from_numpy(w2[e]).T
            acc += float(res["gates"][t, j]) * out
        if shared:
            acc += (torch.nn.functional.silu(xt @ torch.from_numpy(sw13[:I]).T)
                    * (xt @ torch.from_numpy(sw13[I:]).T)) @ torch.from_numpy(sw2).T
        ok &= bool(np.allclose(res["y"][t], acc.numpy()[0], rtol=1e-12, atol=1e-13))
    return ok


def test_layer_matches_per_token_definition():
    assert check_layer_vs_per_token_definition()
    assert check_layer_vs_per_token_definition(seed=21, E=8, k=3, n_group=4, topk_group=2, shared=True)


def test_layer_invariant_under_expert_relabelling():
    r = _rng(22)
    N, H, E, k, I = 40, 8, 10, 3, 6
    x = r.standard_normal((N, H))
    z = r.standard_normal((N, E)).astype(np.float32)
    w13 = r.standard_normal((E, 2 * I, H)) * 0.3
    w2 = r.standard_normal((E, H, I)) * 0.3
    perm = r.permutation(E)
    a = oracle.moe_layer(x, z, k, w13, w2)["y"]
    b = oracle.moe_layer(x, z[:, perm], k, w13[perm], w2[perm])["y"]
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14)


def test_fp8_layer_uses_dequantized_operands():
    """fp8 chain = bf16-free chain run on the dequantized payload and weights."""
    r = _rng(23)
    N, H, E, k, I = 20, 256, 4, 2, 128
    x = (r.standard_normal((N, H)) * 0.02).astype(np.float32)
    z = r.standard_normal((N, E)).astype(np.float32)
    w13 = (r.standard_normal((E, 2 * I, H)) * 0.02).astype(np.float32)
    w2 = (r.standard_normal((E, H, I)) * 0.02).astype(np.float32)
    q13 = [oracle.quantize_blocks(w13[e]) for e in range(E)]
    q2 = [oracle.quantize_blocks(w2[e]) for e in range(E)]
    res = oracle.moe_layer(x, z, k, lambda e: q13[e][0], lambda e: q2[e][0], fp8=True,
                           w13_scale=lambda e: q13[e][1], w2_scale=lambda e: q2[e][1])
    xq, xs = oracle.quantize_blocks(x)
    xd = oracle.dequantize_blocks(xq, xs)
    ref = oracle.moe_layer(xd, z, k, np.stack([oracle.dequantize_blocks(*q13[e]) for e in range(E)]),
                           np.stack([oracle.dequantize_blocks(*q2[e]) for e in range(E)]))
    assert np.allclose(res["y"], ref["y"], rtol=1e-13, atol=1e-18)
    # and the fp8 result stays within the codec's error of the unquantized layer
    full = oracle.moe_layer(x.astype(np.float64), z, k, w13.astype(np.float64), w2.astype(np.float64))
    rel = np.abs(res["y"] - full["y"]).max(axis=1) / np.abs(full["y"]).max(axis=1)
    assert rel.max() < 0.1


def test_imbalance_closed_forms():
    assert oracle.imbalance(np.array([4, 4, 4, 4])) == 1.0
    assert oracle.imbalance(np.array([8, 0, 0, 0])) == 4.0
    assert oracle.imbalance(np.array([3, 1, 2, 2])) == 1.5


# ------------------------------------------------------------------------------------------
# mutation tests: plausible mistakes planted in the oracle must fail a pin
# ------------------------------------------------------------------------------------------

def _mut_topk_ascending_ties(zb, k, allowed=None):
    key = zb.astype(np.float32)
    if allowed is not None:
        key = np.where(allowed, key, np.float32(-np.inf))
    return np.argsort(key, axis=1, kind="stable")[:, ::-1][:, :k].astype(np.int32)


def _mut_silu_wrong_sign(a):
    return a / (1.0 + np.exp(a))


def _mut_ffn_gate_up_swapped(a, w13, w2):
    I = w13.shape[0] // 2
    gate = a @ w13[I:].T
    up = a @ w13[:I].T
    h = gate / (1.0 + np.exp(-gate)) * up
    return h, h @ w2.T


def _mut_gates_unnormalized(zb, idx):
    sel = np.take_along_axis(zb.astype(np.float64), idx.astype(np.int64), axis=1)
    return np.exp(sel) / np.exp(zb.astype(np.float64)).sum(axis=1, keepdims=True)


def _mut_group_mask_sum_score(zb, n_group, topk_group):
    N, E = zb.shape
    G = E // n_group
    score = zb.reshape(N, n_group, G).min(axis=2)
    chosen = np.argsort(-score, axis=1, kind="stable")[:, :topk_group]
    ok = np.zeros((N, n_group), dtype=bool)
    np.put_along_axis(ok, chosen, True, axis=1)
    return np.repeat(ok, G, axis=1)


def _mut_router_experts_reversed(x, w_r):
    return (np.asarray(x, np.float64) @ np.asarray(w_r, np.float64).T)[:, ::-1].astype(np.float32)


def _mut_router_drops_last_column(x, w_r):
    x, w_r = np.asarray(x, np.float64), np.asarray(w_r, np.float64)
    return (x[:, :-1] @ w_r[:, :-1].T).astype(np.float32)


def _mut_swiglu_backward_no_chain(gate, up, dh):
    s = 1.0 / (1.0 + np.exp(-gate))
    return dh * up * s, dh * gate * s


def _mut_gates_backward_no_center(gates, dg):
    return np.asarray(gates, np.float64) * np.asarray(dg, np.float64)


def _mut_combine_backward_unscaled(dy, send_pos, gates, expert_out, k):
    d_eo, dg = _ORIG_COMBINE_BACKWARD(dy, send_pos, np.ones_like(np.asarray(gates, np.float64)), expert_out, k)
    return d_eo, dg


def _mut_expert_backward_halves_swapped(a, w13, w2, d_out):
    r = _ORIG_EXPERT_BACKWARD(a, w13, w2, d_out)
    I = r["d_au"].shape[1] // 2
    r["dw13"] = np.concatenate([r["d_au"][:, I:], r["d_au"][:, :I]], axis=1).T @ np.asarray(a, np.float64)
    return r


_ORIG_COMBINE_BACKWARD = oracle.combine_backward
_ORIG_EXPERT_BACKWARD = oracle.expert_ffn_backward

MUTATIONS = [
    ("swiglu_backward", _mut_swiglu_backward_no_chain, check_backward_fd),
    ("gates_backward", _mut_gates_backward_no_center, check_backward_fd),
    ("combine_backward", _mut_combine_backward_unscaled, check_backward_fd),
    ("expert_ffn_backward", _mut_expert_backward_halves_swapped, check_backward_fd),
    ("router_logits", _mut_router_experts_reversed, check_router_selects_permuted_columns),
    ("router_logits", _mut_router_drops_last_column, check_router_vs_bruteforce),
    ("topk_select", _mut_topk_ascending_ties,
     lambda: check_topk_vs_bruteforce() and bool(np.array_equal(
         oracle.topk_select(np.array([[1, 3, 3, 2, 3]], np.float32), 2), [[1, 2]]))),
    ("silu", _mut_silu_wrong_sign, check_dense_reduction),
    ("expert_ffn", _mut_ffn_gate_up_swapped, check_dense_reduction),
    ("renormalized_gates", _mut_gates_unnormalized, check_gates_vs_full_softmax),
    ("group_limit_mask", _mut_group_mask_sum_score, check_group_limit_vs_bruteforce),
]


@pytest.mark.parametrize("name,mutant,pin", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistakes(monkeypatch, name, mutant, pin):
    assert pin(), "pin must pass on the unmodified oracle"
    monkeypatch.setattr(oracle, name, mutant)
    assert not pin(), f"pin did not notice a planted mistake in {name}"


def test_pins_catch_layout_mistake(monkeypatch):
    idx = workload.fixed_route(50, 8, 3, "random", seed=3).numpy()
    orig = oracle.dispatch_layout

    def bad_layout(topk_idx, E):  # rows of an expert in descending token order
        n_e, off, sp, ss = orig(topk_idx, E)
        ss2 = ss.copy()
        for e in range(E):
            ss2[off[e]:off[e + 1]] = ss[off[e]:off[e + 1]][::-1]
        sp2 = np.empty_like(sp)
        sp2[ss2] = np.arange(ss.size)
        return n_e, off, sp2, ss2

    assert check_layout_invariants(idx, 8)
    monkeypatch.setattr(oracle, "dispatch_layout", bad_layout)
    assert not check_layout_invariants(idx, 8)


def test_pins_catch_combine_mistake(monkeypatch):
    orig = oracle.combine

    def bad_combine(expert_out, send_pos, gates, k, shared_out=None):  # drops the last slot
        g2 = np.array(gates, dtype=np.float64)
        g2[:, -1] = 0.0
        return orig(expert_out, send_pos, g2, k, shared_out)

    assert check_layer_vs_per_token_definition()
    monkeypatch.setattr(oracle, "combine", bad_combine)
    assert not check_layer_vs_per_token_definition()
