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
