"""Helpers shared by the GPU parity tests (comparison metrics and oracle adapters)."""
import numpy as np
import torch


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def token_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of ||got_t - ref_t||_inf / ||ref_t||_inf (rows with a zero reference skipped)."""
    num = np.abs(np.asarray(got, np.float64) - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    ok = den > 0
    if not ok.any():
        return float(num.max()) if num.size else 0.0
    return float((num[ok] / den[ok]).max())


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (round to nearest even), returned as float64."""
    return torch.from_numpy(np.asarray(a, np.float64)).to(torch.float32).to(torch.bfloat16).to(
        torch.float64).numpy()


def bf16_ulp(a: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |a| (8 significant bits)."""
    a = np.abs(np.asarray(a, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def sync():
    torch.cuda.synchronize()


def say(msg: str):
    print(msg, flush=True)


def with_logits(inp: dict) -> dict:
    """Adds the oracle's router logits z = x W_r^T (host fp32 'z_cpu' and its device copy 'z')
    to a layer's inputs, for the tests that start the path at z."""
    from oracle import moe_oracle as oracle
    z = torch.from_numpy(oracle.router_logits(f64(inp["x"]), f64(inp["w_r"])))
    inp["z_cpu"] = z
    inp["z"] = z.to(inp["x"].device)
    return inp


U32 = 2.0 ** -24


def router_bound(x64, w64, H):
    """Bound on |z_gpu - z| for the fp32 sum of H products in any order: each of the at
    most H + 16 additions (16: the most partial sums the K split adds) rounds once, by at
    most 2^-24 of a partial sum no larger than sum_h |x_h w_h| (bf16 products are exact in
    fp32; fp32 operands multiply inside an FMA).  Doubled for the second-order terms."""
    return 2.0 * (H + 16) * U32 * (np.abs(x64) @ np.abs(w64).T)


def decision_margin(zb, k, n_group, topk_group):
    """Per token, the smallest gap between biased logits that the route's decisions compare:
    the kept and the first dropped group score, and consecutive logits among the k + 1
    largest allowed ones (slot order and the last kept expert).  Logits that move by less
    than half of it cannot change the route."""
    zb = np.asarray(zb, np.float64)
    N, E = zb.shape
    out = np.full(N, np.inf)
    for t in range(N):
        row = zb[t]
        allowed = np.ones(E, bool)
        if n_group:
            G = E // n_group
            gs = row.reshape(n_group, G).max(axis=1)
            order = np.argsort(-gs, kind="stable")
            if topk_group < n_group:
                out[t] = gs[order[topk_group - 1]] - gs[order[topk_group]]
            allowed[:] = False
            for g in order[:topk_group]:
                allowed[g * G:(g + 1) * G] = True
        s = np.sort(row[allowed])[::-1][:k + 1]
        if s.size > 1:
            out[t] = min(out[t], np.diff(-s).min())
    return out
