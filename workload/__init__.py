"""Seeded synthetic inputs for the sparse-MoE layer workloads.

Both the GPU path and the CPU oracle consume these tensors; this module holds
no step of the layer itself (no top-k, gating, layout, permutation, expert FFN,
combine or fp8 coding).  It only produces:

* normally distributed values N(0, 0.02^2) (the pages' workloads draw hidden
  states and weights this way), cast to the workload's storage dtype;
* the router weight W_r [E, H] (one row per expert) in the storage dtype;
* the synthetic Zipf skew expressed as a per-expert additive logit bias.

Every random value is a pure function of ``(seed, tensor id, sub-stream,
element index)``: a 32-bit integer hash picks one of 65536 precomputed fp32
normal quantiles.  Only integer arithmetic and a table lookup are involved,
so a tensor generated on the CPU and the same tensor generated on the GPU
are bit-identical; large weights can therefore be generated directly in HBM
and any slice regenerated on the host.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np
import torch

_M32 = 0xFFFFFFFF
_TABLE_BITS = 16
WEIGHT_STD = 0.02

# tensor ids of the independent streams
T_X, T_WR, T_W13, T_W2, T_SW13, T_SW2, T_PERM, T_EO, T_GATE, T_IDX = range(10)


@dataclass(frozen=True)
class MoEConfig:
    """One synthetic MoE-layer workload (sizes in the pages' notation).

    N tokens, hidden size H, E routed experts, top-k, expert intermediate
    size I.  ``dtype`` is the storage / compute type of the layer:
    'f32', 'bf16', or 'fp8' (bf16 hidden states and weights quantized to
    OCP e4m3 with per-128-column fp32 scales by each side's own codec).
    """
    name: str
    N: int
    H: int
    E: int
    k: int
    I: int
    dtype: str
    n_group: int = 0
    topk_group: int = 0
    shared: bool = False
    zipf_s: float = 0.0
    seed: int = 0

    @property
    def rows(self) -> int:
        return self.N * self.k

    def scaled(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


CONFIGS: Dict[str, MoEConfig] = {
    # tiny fp32 layer, the oracle finishes it in well under a second
    "tiny_f32": MoEConfig("tiny_f32", N=256, H=128, E=8, k=2, I=256, dtype="f32"),
    # Mixtral-shaped bf16 layer
    "mixtral_bf16": MoEConfig("mixtral_bf16", N=4096, H=4096, E=8, k=2, I=14336, dtype="bf16"),
    # DeepSeek-V3-shaped bf16 layer: 256 experts in 8 groups, top-4 groups, top-8, one shared expert
    "dsv3_bf16": MoEConfig("dsv3_bf16", N=8192, H=7168, E=256, k=8, I=2048, dtype="bf16",
                           n_group=8, topk_group=4, shared=True),
    # same shapes with a Zipf(1.2) router bias: a few hot experts take most rows
    "dsv3_zipf_bf16": MoEConfig("dsv3_zipf_bf16", N=8192, H=7168, E=256, k=8, I=2048, dtype="bf16",
                                n_group=8, topk_group=4, shared=True, zipf_s=1.2),
    # decode-shaped fp8 layer
    "decode_fp8": MoEConfig("decode_fp8", N=128, H=7168, E=256, k=8, I=2048, dtype="fp8"),
    # the DeepSeek-V3-shaped layer in fp8 at a prefill batch (measured on request: bench.py
    # --config dsv3_fp8; not one of the default workloads)
    "dsv3_fp8": MoEConfig("dsv3_fp8", N=8192, H=7168, E=256, k=8, I=2048, dtype="fp8",
                          n_group=8, topk_group=4, shared=True),
}
CONFIG_ORDER = ["tiny_f32", "mixtral_bf16", "dsv3_bf16", "dsv3_zipf_bf16", "decode_fp8"]


# --------------------------------------------------------------------------------------
# counter-based generator
# --------------------------------------------------------------------------------------

def _mix32_int(x: int) -> int:
    """32-bit avalanche mix on a Python int (used to derive stream keys)."""
    x &= _M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & _M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & _M32
    x ^= x >> 16
    return x


def stream_key(seed: int, tensor_id: int, sub: int = 0) -> int:
    k = _mix32_int(seed * 0x9E3779B1 + 0x632BE5AB)
    k = _mix32_int(k ^ (tensor_id * 0x85EBCA77))
    k = _mix32_int(k ^ (sub * 0xC2B2AE3D) ^ 0x27D4EB2F)
    return k


def _mulmod32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2^32 for int64 tensors holding values in [0, 2^32), without overflow."""
    lo = x & 0xFFFF
    hi = x >> 16
    return (lo * c + (((hi * c) & 0xFFFF) << 16)) & _M32


def _mix32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mulmod32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mulmod32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _mix32_np(x: np.ndarray) -> np.ndarray:
    """Same mix as ``_mix32`` on uint32 arrays (numpy's uint32 arithmetic wraps mod 2^32)."""
    x = x ^ (x >> np.uint32(16))
    x = x * np.uint32(0x7FEB352D)
    x = x ^ (x >> np.uint32(15))
    x = x * np.uint32(0x846CA68B)
    x = x ^ (x >> np.uint32(16))
    return x


def uniform_bits(numel: int, key: int, device, start: int = 0) -> torch.Tensor:
    """32 random bits (int64 in [0, 2^32)) for element indices start .. start+numel-1.

    On the CPU the hash runs on numpy uint32 arrays; elsewhere on torch int64
    tensors with an overflow-free modular multiply.  Both compute the same
    function of the element index.
    """
    if start + numel > (1 << 32):
        raise ValueError("a stream holds at most 2^32 elements")
    k1 = key & _M32
    k2 = (key * 0x9E3779B1) & _M32
    if torch.device(device).type == "cpu":
        i = np.arange(start, start + numel, dtype=np.uint64).astype(np.uint32)
        with np.errstate(over="ignore"):
            h = _mix32_np(i ^ np.uint32(k1))
            h = _mix32_np(h ^ np.uint32(k2))
        return torch.from_numpy(h.astype(np.int64))
    return uniform_bits_torch(numel, key, device, start)


def uniform_bits_torch(numel: int, key: int, device, start: int = 0) -> torch.Tensor:
    """The torch int64 implementation of ``uniform_bits`` (any device)."""
    i = torch.arange(start, start + numel, dtype=torch.int64, device=device)
    h = _mix32(i ^ (key & _M32))
    h = _mix32(h ^ ((key * 0x9E3779B1) & _M32))
    return h


_TABLES: Dict[tuple, torch.Tensor] = {}


def normal_table(std: float = WEIGHT_STD) -> torch.Tensor:
    """2^16 fp32 quantiles of N(0, std^2): entry j = std * Phi^-1((j + 1/2) / 2^16).

    Built in float64 (scipy's ndtri), mirrored so the table is exactly
    symmetric, then rounded once to fp32.
    """
    key = ("cpu", std)
    if key not in _TABLES:
        from scipy.special import ndtri
        n = 1 << _TABLE_BITS
        half = ndtri((np.arange(n // 2, dtype=np.float64) + 0.5) / n) * std  # negative half
        full = np.concatenate([half, -half[::-1]])
        _TABLES[key] = torch.from_numpy(full.astype(np.float32))
    return _TABLES[key]


def _table_on(device, std: float) -> torch.Tensor:
    dev = torch.device(device)
    key = (str(dev), std)
    if key not in _TABLES:
        _TABLES[key] = normal_table(std).to(dev)
    return _TABLES[key]


def normal(shape, key: int, device="cpu", dtype=torch.float32, std: float = WEIGHT_STD,
           start: int = 0) -> torch.Tensor:
    """Seeded N(0, std^2) tensor of ``shape``; ``start`` offsets the element counter."""
    numel = int(np.prod(shape)) if len(shape) else 1
    idx = uniform_bits(numel, key, device, start) >> (32 - _TABLE_BITS)
    vals = _table_on(device, std)[idx]
    return vals.reshape(shape).to(dtype)


def random_permutation(n: int, key: int) -> np.ndarray:
    """Seeded permutation of range(n) (argsort of hashed keys, ties broken by position)."""
    h = uniform_bits(n, key, "cpu").numpy()
    return np.lexsort((np.arange(n), h))


# --------------------------------------------------------------------------------------
# workload tensors
# --------------------------------------------------------------------------------------

def storage_dtype(cfg: MoEConfig) -> torch.dtype:
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def hidden_states(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    """x [N, H] in the storage dtype."""
    return normal((cfg.N, cfg.H), stream_key(cfg.seed, T_X), device, storage_dtype(cfg))


def router_weight(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    """W_r [E, H] in the storage dtype: row e holds expert e's H router weights."""
    return normal((cfg.E, cfg.H), stream_key(cfg.seed, T_WR), device, storage_dtype(cfg))


def zipf_bias(cfg: MoEConfig) -> Optional[torch.Tensor]:
    """Per-expert additive logit bias b_e = sigma_z * ln p_{pi(e)}, fp32 [E], or None.

    p_r = r^-s / sum_{r'<=E} r'^-s (Zipf law over expert ranks r = 1..E), pi a
    seeded permutation of the experts, sigma_z = 0.02^2 * sqrt(H) the standard
    deviation of a logit when x and W_r are N(0, 0.02^2): the skew is measured
    in units of the logits' own spread, so hot experts take most rows without
    every token collapsing onto the same k experts.
    """
    if cfg.zipf_s <= 0.0:
        return None
    r = np.arange(1, cfg.E + 1, dtype=np.float64)
    p = r ** (-cfg.zipf_s)
    p /= p.sum()
    perm = random_permutation(cfg.E, stream_key(cfg.seed, T_PERM))
    sigma_z = WEIGHT_STD * WEIGHT_STD * math.sqrt(cfg.H)
    b = sigma_z * np.log(p[perm])
    return torch.from_numpy(b.astype(np.float32))


def expert_w13(cfg: MoEConfig, e: int, device="cpu", dtype=None, shared: bool = False) -> torch.Tensor:
    """Expert e's stacked [W_gate; W_up] as [2I, H] (rows 0..I-1 gate, I..2I-1 up)."""
    tid = T_SW13 if shared else T_W13
    return normal((2 * cfg.I, cfg.H), stream_key(cfg.seed, tid, e), device,
                  dtype or storage_dtype(cfg))


def expert_w2(cfg: MoEConfig, e: int, device="cpu", dtype=None, shared: bool = False) -> torch.Tensor:
    """Expert e's down projection W_down as [H, I]."""
    tid = T_SW2 if shared else T_W2
    return normal((cfg.H, cfg.I), stream_key(cfg.seed, tid, e), device,
                  dtype or storage_dtype(cfg))


def _normal_streams(keys, shape, device, dtype, std: float = WEIGHT_STD) -> torch.Tensor:
    """[len(keys), *shape]: stream b is exactly ``normal(shape, keys[b])``, made in one pass."""
    numel = int(np.prod(shape))
    dev = torch.device(device)
    k1 = torch.tensor([k & _M32 for k in keys], dtype=torch.int64, device=dev)[:, None]
    k2 = torch.tensor([(k * 0x9E3779B1) & _M32 for k in keys], dtype=torch.int64, device=dev)[:, None]
    i = torch.arange(numel, dtype=torch.int64, device=dev)[None, :]
    h = _mix32(_mix32(i ^ k1) ^ k2)
    vals = _table_on(dev, std)[h >> (32 - _TABLE_BITS)]
    return vals.reshape((len(keys),) + tuple(shape)).to(dtype)


def all_expert_weights(cfg: MoEConfig, device="cpu", shared: bool = False):
    """(w13 [E, 2I, H], w2 [E, H, I]) in the storage dtype.

    Expert e's matrices are the streams ``expert_w13(cfg, e)`` / ``expert_w2(cfg, e)``;
    off the CPU several experts are generated per pass (about 2^27 elements at a time),
    which gives the same values with a few hundred launches instead of tens of thousands.
    """
    E = 1 if shared else cfg.E
    dt = storage_dtype(cfg)
    w13 = torch.empty((E, 2 * cfg.I, cfg.H), dtype=dt, device=device)
    w2 = torch.empty((E, cfg.H, cfg.I), dtype=dt, device=device)
    if torch.device(device).type == "cpu":
        for e in range(E):
            w13[e] = expert_w13(cfg, e, device, dt, shared)
            w2[e] = expert_w2(cfg, e, device, dt, shared)
        return w13, w2
    t13, t2 = (T_SW13, T_SW2) if shared else (T_W13, T_W2)
    per = max(1, (1 << 27) // (2 * cfg.I * cfg.H))
    for e0 in range(0, E, per):
        es = list(range(e0, min(E, e0 + per)))
        w13[e0:e0 + len(es)] = _normal_streams([stream_key(cfg.seed, t13, e) for e in es],
                                               (2 * cfg.I, cfg.H), device, dt)
        w2[e0:e0 + len(es)] = _normal_streams([stream_key(cfg.seed, t2, e) for e in es],
                                              (cfg.H, cfg.I), device, dt)
    return w13, w2


def synthetic_rows(rows: int, cols: int, key_sub: int, cfg: MoEConfig, device="cpu",
                   dtype=None) -> torch.Tensor:
    """An arbitrary [rows, cols] N(0, 0.02^2) tensor (e.g. stand-in expert outputs)."""
    return normal((rows, cols), stream_key(cfg.seed, T_EO, key_sub), device,
                  dtype or storage_dtype(cfg))


def fixed_route(N: int, E: int, k: int, kind: str, seed: int = 0) -> torch.Tensor:
    """Hand-made routes [N, k] int32 that bypass the router (distinct experts per token).

    'round_robin': expert (t*k + j) mod E  -> every expert gets N*k/E rows when E | N*k
    'hot':         experts 0..k-1 for every token -> n_e = N for e < k, 0 otherwise
    'random':      k distinct experts per token drawn from the seeded stream
    """
    if kind == "round_robin":
        t = torch.arange(N, dtype=torch.int64)[:, None]
        j = torch.arange(k, dtype=torch.int64)[None, :]
        return ((t * k + j) % E).to(torch.int32)
    if kind == "hot":
        return torch.arange(k, dtype=torch.int32)[None, :].repeat(N, 1)
    if kind == "random":
        bits = uniform_bits(N * E, stream_key(seed, T_IDX, E * 1000 + k), "cpu").reshape(N, E)
        order = torch.argsort(bits, dim=1, stable=True)
        return order[:, :k].to(torch.int32).contiguous()
    raise ValueError(kind)


def counted_route(n_e, k: int, seed: int = 0) -> torch.Tensor:
    """Routes [N, k] int32 in which expert e appears exactly n_e[e] times (distinct experts
    per token); N = sum(n_e) / k, and every n_e[e] must be at most N.

    The expert ids, listed in runs of n_e[e], are read column-wise: slot j of token t takes
    entry j * N + t, so a token's k entries are N apart and fall in k different runs.  The
    tokens are then shuffled by a seeded permutation.
    """
    n_e = [int(c) for c in n_e]
    total = sum(n_e)
    if total % k or any(c < 0 for c in n_e):
        raise ValueError("sum(n_e) must be a multiple of k")
    N = total // k
    if any(c > N for c in n_e):
        raise ValueError("an expert cannot take more rows than there are tokens")
    ids = np.repeat(np.arange(len(n_e), dtype=np.int32), n_e)
    idx = ids.reshape(k, N).T
    return torch.from_numpy(np.ascontiguousarray(idx[random_permutation(N, stream_key(seed, T_IDX, 7))]))


def random_gates(N: int, k: int, seed: int = 0) -> torch.Tensor:
    """Positive fp32 gates [N, k] (uniform in (0, 1]) for steps tested apart from the router."""
    bits = uniform_bits(N * k, stream_key(seed, T_GATE, k), "cpu")
    return ((bits >> 8).to(torch.float32) + 1.0).mul_(1.0 / (1 << 24)).reshape(N, k)


def make_layer_inputs(cfg: MoEConfig, device="cpu", weights: bool = True) -> dict:
    """All inputs of one layer call: x, W_r, bias, routed and shared expert weights.

    x, W_r and the expert weights are generated on ``device``; the bias is
    computed on the host and moved to ``device``.
    """
    x = hidden_states(cfg, device)
    w_r = router_weight(cfg, device)
    b = zipf_bias(cfg)
    out = {"x": x, "w_r": w_r, "bias": None if b is None else b.to(device), "bias_cpu": b}
    if weights:
        out["w13"], out["w2"] = all_expert_weights(cfg, device)
        if cfg.shared:
            out["sw13"], out["sw2"] = all_expert_weights(cfg, device, shared=True)
    return out
