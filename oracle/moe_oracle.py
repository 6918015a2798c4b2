"""Plain, slow, obviously-correct CPU implementation of the MoE layer's hot path.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Every function restates a definition from the pages, cited by page and
section.  Floating point is float64, except where fp32 takes a decision that
fixes an integer result (biased logits that decide the top-k; the fp32 scale
and the fp32 quotient that decide an e4m3 code): there the oracle computes in
fp32 exactly as IEEE-754 defines the operation, which is the precision the
kernel uses too.

Pages cited:
  [EPX]  "EP / DeepEP explanation" (Mainline, ep_deepep), sections 2, 3, 4, 6
  [WEP]  "Wide EP: MoE expert parallel across dozens of GPUs", sections
         "Group-limited routing" and "Decode" capacity estimate
  [DGG]  "MoE part 4: DeepEP and GroupedGEMM", sections 2, 4, 4.1, 4.2
  [FSDP] "DeepSeek MoE: EP and FSDP guide", the naive MoE forward list
  [DEP]  "DeepEP" (scholia-log), sections 1 and 7
  The backward functions follow "DeepSeek MoE: EP and FSDP guide" (the backward
  mirrors the forward; dispatch's backward is combine) and the chain rule.
"""
from __future__ import annotations

from typing import Callable, Optional, Sequence, Union

import numpy as np

__all__ = [
    "E4M3_MAX", "router_logits", "biased_logits", "group_limit_mask", "topk_select", "renormalized_gates", "route",
    "dispatch_layout", "permute", "e4m3_decode", "e4m3_encode", "quantize_blocks",
    "dequantize_blocks", "silu", "expert_ffn", "grouped_ffn", "combine", "imbalance", "moe_layer",
    "combine_backward", "dispatch_backward", "swiglu_backward", "expert_ffn_backward", "gates_backward",
    "router_backward", "moe_layer_backward",
]

E4M3_MAX = 448.0  # largest finite OCP e4m3fn value: 1.75 * 2^8


# --------------------------------------------------------------------------------------
# router: logits, top-k over them, optional group limit, renormalised gates
# --------------------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_r: np.ndarray) -> np.ndarray:
    """z_{t,e} = sum_h x_{t,h} W_r[e, h], summed in float64 and rounded once to fp32.

    [EPX] 2: the router maps each token's hidden state to logits z in R^{N x E}.
    Readings: a linear map without bias; W_r has one row of H weights per expert
    (the weight layout of a linear layer); both operands are taken as stored.
    """
    x64 = np.asarray(x, dtype=np.float64)
    w64 = np.asarray(w_r, dtype=np.float64)
    return (x64 @ w64.T).astype(np.float32)


def biased_logits(z: np.ndarray, bias: Optional[np.ndarray]) -> np.ndarray:
    """z'_{t,e} = z_{t,e} + b_e, one IEEE fp32 addition per element.

    [DGG] 4.2: the router's top-k takes an additive per-expert correction bias.
    Reading: the bias is a term of the router logits, so it enters both the
    selection and the gates.
    """
    z = np.asarray(z, dtype=np.float32)
    if bias is None:
        return z.copy()
    return (z + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)


def group_limit_mask(zb: np.ndarray, n_group: int, topk_group: int) -> np.ndarray:
    """Boolean [N, E]: experts inside the topk_group groups a token may use.

    [WEP] "Group-limited routing": experts are split into groups; the router
    first picks some groups, then the top-k experts inside the allowed groups.
    Readings: groups are contiguous blocks of E/n_group experts; a group's
    score is the largest logit inside it; ties between groups go to the lower
    group id.
    """
    N, E = zb.shape
    G = E // n_group
    score = zb.reshape(N, n_group, G).max(axis=2)
    # stable sort on the negated score: larger score first, equal scores by group id
    chosen = np.argsort(-score, axis=1, kind="stable")[:, :topk_group]
    group_ok = np.zeros((N, n_group), dtype=bool)
    np.put_along_axis(group_ok, chosen, True, axis=1)
    return np.repeat(group_ok, G, axis=1)


def topk_select(zb: np.ndarray, k: int, allowed: Optional[np.ndarray] = None) -> np.ndarray:
    """I_t as an ordered list: the k largest allowed logits of each token.

    [EPX] 2: the router picks an index set I_t with |I_t| = k.  Readings: slot
    j holds the j-th largest logit; equal logits go to the lower expert index.
    Selecting on logits equals selecting on softmax probabilities (softmax is
    monotone), so no exponential enters the indices.
    """
    key = zb.astype(np.float32)
    if allowed is not None:
        key = np.where(allowed, key, np.float32(-np.inf))
    # stable sort on the negated logit: larger logit first, equal logits by expert index
    # (numpy orders -0.0 and +0.0 as equal)
    return np.argsort(-key, axis=1, kind="stable")[:, :k].astype(np.int32)


def renormalized_gates(zb: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """g_{t,j} = softmax over the selected logits only, in float64.

    [EPX] 2 (gates g_{t,e} for e in I_t) and [DGG] 4.2 ("renormalize"): the
    softmax over all experts, restricted to I_t and renormalised to sum 1,
    which equals exp(z'_{t,j} - m_t) / sum_j' exp(z'_{t,j'} - m_t).
    """
    sel = np.take_along_axis(zb.astype(np.float64), idx.astype(np.int64), axis=1)
    m = sel.max(axis=1, keepdims=True)
    w = np.exp(sel - m)
    return w / w.sum(axis=1, keepdims=True)


def route(z: np.ndarray, k: int, bias: Optional[np.ndarray] = None, n_group: int = 0,
          topk_group: int = 0):
    """Router step of the layer: (topk_idx [N,k] int32, gates [N,k] float64).

    [FSDP] naive forward, steps 1-2 (scores, expert choice); [DGG] 4.2
    (router_topk with correction bias and grouped top-k, renormalised).
    """
    zb = biased_logits(z, bias)
    allowed = group_limit_mask(zb, n_group, topk_group) if n_group > 0 else None
    idx = topk_select(zb, k, allowed)
    return idx, renormalized_gates(zb, idx)


# --------------------------------------------------------------------------------------
# dispatch layout: n_e, offsets and the three index maps
# --------------------------------------------------------------------------------------

def dispatch_layout(topk_idx: np.ndarray, E: int):
    """(n_e [E], offsets [E+1], send_pos [N*k], src_slot [N*k]) as int64.

    [EPX] 2: n_e = |{(t,e): e in I_t}|.  [EPX] 3: each source buckets its
    tokens by expert before the exchange.  [EPX] 6: the layout keeps three
    maps -- token to send position, send position to expert-local position,
    return position to token.  On one GPU the send position is the row of the
    expert-ordered buffer; the expert-local position is row - offsets[e]; the
    return map is src_slot.
    Readings: rows of one expert keep ascending token order;
    slot t*k+j names the pair (token t, its j-th expert).
        offsets[e]          = sum_{e' < e} n_e'
        send_pos[t*k+j]     = offsets[e] + |{t' < t : e in I_t'}|,  e = I_t[j]
        src_slot[send_pos[s]] = s
    """
    flat = np.asarray(topk_idx, dtype=np.int64).reshape(-1)
    n_e = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(n_e)
    # a stable sort of the slots by expert id lists, for every expert, its slots in
    # ascending t*k+j order -- i.e. ascending token order, since a token names an
    # expert at most once; the position in that list is the row
    src_slot = np.argsort(flat, kind="stable").astype(np.int64)
    send_pos = np.empty_like(src_slot)
    send_pos[src_slot] = np.arange(flat.size, dtype=np.int64)
    return n_e, offsets, send_pos, src_slot


def permute(x: np.ndarray, send_pos: np.ndarray, k: int) -> np.ndarray:
    """x_perm[send_pos[t*k+j]] = x[t]: the on-device stand-in of the dispatch exchange.

    [EPX] 3: tokens are bucketed by their target expert and laid out so each
    expert's rows are contiguous for the grouped GEMM; [DGG] 4 (permute by
    expert before the expert GEMM).
    """
    out = np.empty((x.shape[0] * k,) + x.shape[1:], dtype=x.dtype)
    out[np.asarray(send_pos)] = np.repeat(x, k, axis=0)  # repeated row t*k+j is x[t]
    return out


# --------------------------------------------------------------------------------------
# fp8 e4m3 codec with per-128-column fp32 scales
# --------------------------------------------------------------------------------------

def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each OCP e4m3fn byte (1 sign, 4 exponent bits with bias 7, 3 mantissa bits).

    exponent field 0 -> subnormal m/8 * 2^-6; 0x7F / 0xFF -> NaN; no infinities.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return s * mag


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Nearest e4m3fn code to each (finite) value, ties to even, saturating at +-448.

    The spacing of representable values is 2^(E-3) in the binade [2^E, 2^(E+1))
    for E >= -6, and 2^-9 below 2^-6 (subnormals).  The magnitude is rounded
    to that grid with round-half-to-even (np.rint), which is exact in float64.
    """
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    _, ex = np.frexp(a)                       # a = f * 2^ex, f in [0.5, 1)
    E = np.maximum(ex - 1, -6)                # binade exponent, subnormals share E = -6
    step = np.exp2(E.astype(np.float64) - 3)
    q = np.rint(a / step) * step              # rounded magnitude (may carry into next binade)
    q = np.minimum(q, E4M3_MAX)
    _, qx = np.frexp(q)
    qE = qx - 1
    sub = q < 2.0 ** -6
    e_field = np.where(sub, 0, qE + 7)
    m_field = np.where(sub, np.rint(q / 2.0 ** -9), np.rint(q / np.exp2(qE.astype(np.float64) - 3)) - 8)
    m_field = np.where(q == 0, 0, m_field)
    code = (e_field.astype(np.int64) << 3) | m_field.astype(np.int64)
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)


def quantize_blocks(x: np.ndarray, block: int = 128):
    """Per (row, 128-column block) fp8 quantization: (codes uint8 [R,C], scales fp32 [R,C/block]).

    [EPX] 6 and [DEP] 7: an fp8 payload carries fp32 scales that share the
    token's index.  Readings (the pages give no scale rule or rounding mode):
        s = fp32(amax / 448)  (IEEE fp32 division; s = 1 when amax = 0)
        q = e4m3_rne_saturating(fp32(x / s))
    so the block's largest magnitude maps to +-448.
    """
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    if C % block:
        raise ValueError("columns must be a multiple of the block")
    xb = x.reshape(R, C // block, block)
    amax = np.abs(xb).max(axis=2)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    v = (xb / s[:, :, None]).astype(np.float32)
    return e4m3_encode(v).reshape(R, C), s


def dequantize_blocks(codes: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    """codes * scale per block, in float64 (exact: 4-bit by 24-bit significands)."""
    R, C = codes.shape
    vals = e4m3_decode(codes).reshape(R, C // block, block)
    return (vals * np.asarray(scales, dtype=np.float64)[:, :, None]).reshape(R, C)


# --------------------------------------------------------------------------------------
# expert SwiGLU FFN and the grouped form
# --------------------------------------------------------------------------------------

def silu(a: np.ndarray) -> np.ndarray:
    """silu(a) = a * sigmoid(a) = a / (1 + e^-a)."""
    return a / (1.0 + np.exp(-a))


def expert_ffn(a: np.ndarray, w13: np.ndarray, w2: np.ndarray):
    """One expert on rows a [n, H]: h = silu(a W_g^T) * (a W_u^T); out = h W_d^T (float64).

    [DGG] 4.1: an expert is FC1 -> activation -> FC2.  SwiGLU (the workloads'
    expert type) gates the activation: the first I rows of w13 [2I, H] are
    W_gate, the last I rows W_up; w2 [H, I] is W_down.
    """
    a = np.asarray(a, dtype=np.float64)
    w13 = np.asarray(w13, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    I = w13.shape[0] // 2
    gate = a @ w13[:I].T
    up = a @ w13[I:].T
    h = silu(gate) * up
    return h, h @ w2.T


WeightSource = Union[np.ndarray, Callable[[int], np.ndarray]]


def _weight(src: WeightSource, e: int) -> np.ndarray:
    return src(e) if callable(src) else src[e]


def grouped_ffn(a_perm: np.ndarray, offsets: Sequence[int], w13: WeightSource, w2: WeightSource):
    """Expert e applied to its rows [offsets[e], offsets[e+1]) of the expert-ordered buffer.

    [DGG] 2: the grouped GEMM batches many expert GEMMs with differing row
    counts and does not change the MoE mathematics -- so it is written here as
    one dense expert FFN per non-empty segment.  ``w13``/``w2`` are arrays
    indexed by expert or callables e -> weights (float64 values).
    """
    rows = a_perm.shape[0]
    E = len(offsets) - 1
    h = None
    out = None
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        he, oe = expert_ffn(a_perm[lo:hi], _weight(w13, e), _weight(w2, e))
        if h is None:
            h = np.zeros((rows, he.shape[1]))
            out = np.zeros((rows, oe.shape[1]))
        h[lo:hi] = he
        out[lo:hi] = oe
    if h is None:
        h, out = np.zeros((rows, 0)), np.zeros((rows, 0))
    return h, out


def combine(expert_out: np.ndarray, send_pos: np.ndarray, gates: np.ndarray, k: int,
            shared_out: Optional[np.ndarray] = None) -> np.ndarray:
    """y_t = sum_{j<k} g_{t,j} * expert_out[send_pos[t*k+j]]  (+ shared_out_t), float64.

    [EPX] 2: y_t = sum_{e in I_t} g_{t,e} Expert_e(x_t), with an optional shared
    branch added; [EPX] 3: the source sums the returned rows with the gates
    in original token order.  Readings: j ascending, the shared expert added
    last, gate 1.
    """
    N = gates.shape[0]
    sp = np.asarray(send_pos).reshape(N, k)
    g = np.asarray(gates, dtype=np.float64)
    y = np.zeros((N, expert_out.shape[1]))
    for j in range(k):
        y += g[:, j:j + 1] * np.asarray(expert_out[sp[:, j]], dtype=np.float64)
    if shared_out is not None:
        y += np.asarray(shared_out, dtype=np.float64)
    return y


def imbalance(n_e: np.ndarray) -> float:
    """max_e n_e / mean_e n_e  ([EPX] 4, applied over experts instead of ranks)."""
    n_e = np.asarray(n_e, dtype=np.float64)
    return float(n_e.max() / n_e.mean()) if n_e.sum() > 0 else 0.0


# --------------------------------------------------------------------------------------
# the whole layer
# --------------------------------------------------------------------------------------

def moe_layer(x: np.ndarray, z: np.ndarray, k: int, w13: WeightSource, w2: WeightSource,
              bias: Optional[np.ndarray] = None, n_group: int = 0, topk_group: int = 0,
              fp8: bool = False, w13_scale: Optional[WeightSource] = None,
              w2_scale: Optional[WeightSource] = None, shared_w13: Optional[np.ndarray] = None,
              shared_w2: Optional[np.ndarray] = None) -> dict:
    """route -> dispatch layout -> permute -> grouped SwiGLU FFN -> combine (+ shared expert).

    [DGG] 4 (permute by expert, grouped GEMM over tokens-per-expert, unpermute
    and weighted sum) and [FSDP] naive forward steps 1-5.  With ``fp8`` the
    payload is quantized per token and per 128 columns before the permutation
    and its scales travel with it ([EPX] 6); ``w13``/``w2`` then hold e4m3
    codes and ``w13_scale``/``w2_scale`` their scales.  Returns every
    intermediate.
    """
    x = np.asarray(x)
    N = x.shape[0]
    idx, gates = route(z, k, bias, n_group, topk_group)
    E = z.shape[1]
    n_e, offsets, send_pos, src_slot = dispatch_layout(idx, E)
    res = dict(topk_idx=idx, gates=gates, n_e=n_e, offsets=offsets, send_pos=send_pos,
               src_slot=src_slot)
    if fp8:
        codes, scales = quantize_blocks(x)
        res["x_perm_codes"] = permute(codes, send_pos, k)
        res["x_perm_scales"] = permute(scales, send_pos, k)
        a = dequantize_blocks(res["x_perm_codes"], res["x_perm_scales"])

        def deq13(e):
            return dequantize_blocks(_weight(w13, e), _weight(w13_scale, e))

        def deq2(e):
            return dequantize_blocks(_weight(w2, e), _weight(w2_scale, e))
        h, out = grouped_ffn(a, offsets, deq13, deq2)
    else:
        res["x_perm"] = permute(x, send_pos, k)
        h, out = grouped_ffn(res["x_perm"].astype(np.float64), offsets, w13, w2)
    res["h"], res["expert_out"] = h, out
    shared = None
    if shared_w13 is not None:
        _, shared = expert_ffn(x.astype(np.float64), shared_w13, shared_w2)
        res["shared_out"] = shared
    res["y"] = combine(out, send_pos, gates, k, shared)
    res["imbalance"] = imbalance(n_e)
    return res


# --------------------------------------------------------------------------------------
# backward: the gradients of the layer (training)
# --------------------------------------------------------------------------------------
# "DeepSeek MoE: EP and FSDP guide": the backward of the EP layer mirrors the forward
# (the same all-to-alls in reverse), the backward of dispatch being combine, and each
# expert keeps its own weight gradients.  Top-k selection is piecewise constant: the
# gradients reach the router only through the gates.

def combine_backward(dy: np.ndarray, send_pos: np.ndarray, gates: np.ndarray, expert_out: np.ndarray,
                     k: int):
    """Gradients of y_t = sum_j g_{t,j} o_{send_pos[t*k+j]}: (d_expert_out [rows, H], dg [N, k]).

    d o_row = g_{t,j} dy_t for row = send_pos[t*k+j] (dy dispatched to the slots and
    scaled by the gates); dg_{t,j} = <dy_t, o_row>.  Rows no slot names get 0.
    """
    N = gates.shape[0]
    sp = np.asarray(send_pos).reshape(N, k)
    dy = np.asarray(dy, dtype=np.float64)
    g = np.asarray(gates, dtype=np.float64)
    eo = np.asarray(expert_out, dtype=np.float64)
    d_eo = np.zeros_like(eo)
    dg = np.zeros((N, k))
    for j in range(k):
        d_eo[sp[:, j]] = g[:, j:j + 1] * dy
        dg[:, j] = (dy * eo[sp[:, j]]).sum(axis=1)
    return d_eo, dg


def dispatch_backward(d_perm: np.ndarray, send_pos: np.ndarray, N: int, k: int) -> np.ndarray:
    """Backward of the dispatch (permute): dx_t = sum_j d_perm[send_pos[t*k+j]], i.e. a combine
    with weight 1 ("DeepSeek MoE: EP and FSDP guide": dispatch's backward is combine)."""
    return combine(d_perm, send_pos, np.ones((N, k)), k)


def swiglu_backward(gate: np.ndarray, up: np.ndarray, dh: np.ndarray):
    """h = silu(a) * u  =>  da = dh * u * silu'(a), du = dh * silu(a), with
    silu'(a) = s(a) (1 + a (1 - s(a))), s the logistic function (float64)."""
    a = np.asarray(gate, dtype=np.float64)
    u = np.asarray(up, dtype=np.float64)
    dh = np.asarray(dh, dtype=np.float64)
    s = 1.0 / (1.0 + np.exp(-a))
    return dh * u * s * (1.0 + a * (1.0 - s)), dh * a * s


def expert_ffn_backward(a: np.ndarray, w13: np.ndarray, w2: np.ndarray, d_out: np.ndarray) -> dict:
    """Backward of expert_ffn on rows a [n, H] given d_out [n, H] (float64).

    dh = d_out W_d; dW_d = d_out^T h; (da, du) from swiglu_backward; d_a =
    [da, du] w13 (W_gate and W_up stacked as in w13); dW13 = [da, du]^T a.
    Returns d_in [n, H], dw13 [2I, H], dw2 [H, I] and the intermediates
    (gate and up pre-activations, h, dh, d_au = [da, du] [n, 2I]).
    """
    a = np.asarray(a, dtype=np.float64)
    w13 = np.asarray(w13, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    d_out = np.asarray(d_out, dtype=np.float64)
    I = w13.shape[0] // 2
    gate = a @ w13[:I].T
    up = a @ w13[I:].T
    h = silu(gate) * up
    dh = d_out @ w2
    da, du = swiglu_backward(gate, up, dh)
    d_au = np.concatenate([da, du], axis=1)
    return dict(d_in=d_au @ w13, dw13=d_au.T @ a, dw2=d_out.T @ h, gate=gate, up=up, h=h, dh=dh, d_au=d_au)


def gates_backward(gates: np.ndarray, dg: np.ndarray) -> np.ndarray:
    """Backward of the renormalised softmax over the selected logits: for g = softmax(z'_sel),
    dz'_j = g_j (dg_j - sum_i g_i dg_i) on the k selected experts (0 elsewhere)."""
    g = np.asarray(gates, dtype=np.float64)
    dg = np.asarray(dg, dtype=np.float64)
    return g * (dg - (g * dg).sum(axis=1, keepdims=True))


def router_backward(x: np.ndarray, w_r: np.ndarray, topk_idx: np.ndarray, dz_sel: np.ndarray):
    """Backward of z = x W_r^T when only the selected logits carry gradient dz_sel [N, k]:
    dx_t = sum_j dz_sel[t, j] W_r[idx[t, j]] and dW_r[e] = sum over (t, j) with idx = e of
    dz_sel[t, j] x_t.  (The correction bias enters z' additively: dz = dz'.)"""
    x = np.asarray(x, dtype=np.float64)
    w_r = np.asarray(w_r, dtype=np.float64)
    idx = np.asarray(topk_idx).astype(np.int64)
    dz = np.asarray(dz_sel, dtype=np.float64)
    dx = np.zeros_like(x)
    dw = np.zeros_like(w_r)
    for j in range(idx.shape[1]):
        dx += dz[:, j:j + 1] * w_r[idx[:, j]]
        np.add.at(dw, idx[:, j], dz[:, j:j + 1] * x)
    return dx, dw


def moe_layer_backward(x: np.ndarray, z: np.ndarray, k: int, w13: WeightSource, w2: WeightSource,
                       dy: np.ndarray, bias: Optional[np.ndarray] = None, n_group: int = 0,
                       topk_group: int = 0, shared_w13: Optional[np.ndarray] = None,
                       shared_w2: Optional[np.ndarray] = None, w_r: Optional[np.ndarray] = None) -> dict:
    """Gradients of moe_layer (bf16/fp32 layers) for the upstream gradient dy [N, H].

    Routes and gates are those of moe_layer on z; the gradient flows through the
    gates (gates_backward) into the selected logits and, given the router weight
    W_r (z = x W_r^T), into x and W_r.  Returns dx [N, H], dw13 / dw2 (dicts
    expert -> gradient, for the experts with rows), the shared expert's dw13 / dw2,
    dw_r, and the intermediates of every step (d_expert_out, dg, dz_sel, dh, d_au,
    d_perm, the recomputed gate/up pre-activations and h).
    """
    fwd = moe_layer(x, z, k, w13, w2, bias=bias, n_group=n_group, topk_group=topk_group,
                    shared_w13=shared_w13, shared_w2=shared_w2)
    x64 = np.asarray(x, dtype=np.float64)
    N, H = x64.shape
    offsets, send_pos = fwd["offsets"], fwd["send_pos"]
    rows = int(offsets[-1])
    d_eo, dg = combine_backward(dy, send_pos, fwd["gates"], fwd["expert_out"], k)
    x_perm = fwd["x_perm"].astype(np.float64)
    d_perm = np.zeros((rows, H))
    res = dict(fwd=fwd, d_expert_out=d_eo, dg=dg, dw13={}, dw2={})
    parts = {n: [] for n in ("gate", "up", "h", "dh", "d_au")}
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        b = expert_ffn_backward(x_perm[lo:hi], _weight(w13, e), _weight(w2, e), d_eo[lo:hi])
        d_perm[lo:hi] = b["d_in"]
        res["dw13"][e], res["dw2"][e] = b["dw13"], b["dw2"]
        for n in parts:
            parts[n].append(b[n])
    for n, v in parts.items():
        res[n] = np.concatenate(v) if v else np.zeros((0, 0))
    res["d_perm"] = d_perm
    dx = dispatch_backward(d_perm, send_pos, N, k)
    if shared_w13 is not None:
        b = expert_ffn_backward(x64, shared_w13, shared_w2, dy)
        dx = dx + b["d_in"]
        res["shared"] = b
        res["shared_dw13"], res["shared_dw2"] = b["dw13"], b["dw2"]
    res["dz_sel"] = gates_backward(fwd["gates"], dg)
    if w_r is not None:
        dx_r, res["dw_r"] = router_backward(x64, w_r, fwd["topk_idx"], res["dz_sel"])
        dx = dx + dx_r
    res["dx"] = dx
    return res
