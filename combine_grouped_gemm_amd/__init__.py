"""Python binding of libmoe: argument marshalling only.

Each function passes torch tensors' device pointers and the current HIP stream
to the C entry point of the same name (include/moe.h) and raises MoEError on a
non-OK status.  Output tensors and workspaces are allocated with torch, which
serves here only as the device-memory and stream provider; every step of the
layer runs in libmoe's HIP kernels.  There is no fallback: if libmoe.so is
missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch

__all__ = [
    "MoEError", "lib", "library_path", "declared_symbols",
    "MOE_F32", "MOE_BF16", "MOE_FP8_E4M3",
    "MOE_OP_DISPATCH_LAYOUT", "MOE_OP_GROUPED_FFN", "MOE_OP_EXPERT_GEMM", "MOE_OP_ROUTER", "MOE_OP_EXPERT_DGRAD",
    "MOE_LAYOUT_SCRATCH_BYTES", "moe_router_logits", "moe_route", "moe_dispatch_layout",
    "moe_dispatch_layout_noalloc", "moe_permute", "moe_quantize_fp8", "moe_dequantize_fp8", "moe_expert_gate_up",
    "moe_expert_gate_up_gathered", "moe_expert_gate_up_gathered_shared", "moe_expert_down",
    "moe_expert_down_shared", "moe_expert_gate_up_gathered_shared_e4m3", "moe_expert_down_shared_e4m3",
    "moe_grouped_ffn", "moe_combine", "moe_workspace_bytes", "moe_status_str",
    "moe_version", "moe_combine_backward", "moe_expert_gate_up_preact", "moe_swiglu_backward", "moe_expert_dgrad",
    "moe_expert_wgrad", "moe_router_backward", "moe_router_input_grad", "moe_stream_probe",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_HEADER = os.path.join(os.path.dirname(_HERE), "include", "moe.h")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = range(3)
MOE_OP_DISPATCH_LAYOUT, MOE_OP_GROUPED_FFN, MOE_OP_EXPERT_GEMM, MOE_OP_ROUTER, MOE_OP_EXPERT_DGRAD = range(5)
MOE_LAYOUT_SCRATCH_BYTES = 4 << 20   # the fixed count table of moe_dispatch_layout_noalloc


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {moe_status_str(status)} (status {status})")


def library_path() -> str:
    return os.path.join(_HERE, "libmoe.so")


_LIB: Optional[ctypes.CDLL] = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGS = {
    "moe_router_logits": [_P, _I, _I, _I, _P, _I, _P, _P, _SZ, _P],
    "moe_route": [_P, _I, _I, _I, _P, _I, _I, _P, _P, _P],
    "moe_dispatch_layout": [_P, _I, _I, _I, _P, _P, _P, _P, _P, _SZ, _P],
    "moe_dispatch_layout_noalloc": [_P, _I, _I, _I, _P, _P, _P, _P, _P],
    "moe_permute": [_P, _I, _I, _I, _I, _P, _P, _I, _P, _P],
    "moe_quantize_fp8": [_P, _I, ctypes.c_int64, _I, _P, _P, _P],
    "moe_dequantize_fp8": [_P, _P, ctypes.c_int64, _I, _P, _P],
    "moe_grouped_ffn": [_P, _P, _I, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P, _SZ, _P],
    "moe_expert_gate_up": [_P, _P, _I, _P, _I, _I, _I, _I, _P, _P, _P, _P, _SZ, _P],
    "moe_expert_gate_up_gathered": [_P, _I, _I, _P, _I, _P, _I, _I, _I, _I, _P, _P, _P, _SZ, _P],
    "moe_expert_down": [_P, _I, _P, _I, _I, _I, _I, _P, _I, _P, _P, _I, _P, _SZ, _P],
    "moe_expert_gate_up_gathered_shared": [_P, _I, _I, _P, _I, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _SZ, _P],
    "moe_expert_down_shared": [_P, _I, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P, _SZ, _P],
    "moe_expert_gate_up_gathered_shared_e4m3": [_P, _I, _P, _I, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _SZ,
                                                _P],
    "moe_expert_down_shared_e4m3": [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "moe_combine": [_P, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P],
    "moe_workspace_bytes": [_I, _I, _I, _I, _I, _I, _I],
    "moe_combine_backward": [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P],
    "moe_expert_gate_up_preact": [_P, _I, _I, _P, _I, _P, _I, _I, _I, _I, _P, _P, _P, _SZ, _P],
    "moe_swiglu_backward": [_P, _P, _I, _I, _P, _P, _P],
    "moe_expert_dgrad": [_P, _P, _I, _I, _I, _I, _P, _P, _P, _SZ, _P],
    "moe_expert_wgrad": [_P, _I, _P, _I, _P, _I, _I, _P, _I, _I, _P, _I, _P],
    "moe_router_backward": [_P, _P, _I, _I, _P, _P, _I, _I, _P, _I, _I, _P, _P, _I, _P],
    "moe_stream_probe": [_P, _SZ, _I, _P, _P],
    "moe_router_input_grad": [_P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P],
    "moe_status_str": [_I],
    "moe_version": [],
}


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                               "(python -m combine_grouped_gemm_amd.build)")
        L = ctypes.CDLL(path)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = _SZ if name == "moe_workspace_bytes" else (
                ctypes.c_char_p if name in ("moe_status_str", "moe_version") else _I)
        _LIB = L
    return _LIB


def declared_symbols() -> list:
    """Names of the functions include/moe.h declares."""
    text = open(_HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def moe_status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def moe_version() -> str:
    return lib().moe_version().decode()


def moe_workspace_bytes(op: int, N: int, H: int, I: int, E: int, k: int, a_dt: int) -> int:
    return int(lib().moe_workspace_bytes(op, N, H, I, E, k, a_dt))


# ------------------------------------------------------------------------------------------
# marshalling helpers
# ------------------------------------------------------------------------------------------

def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoEError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmoe takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libmoe takes contiguous tensors")
    return t.data_ptr()


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MOE_FP8_E4M3
    raise ValueError(f"unsupported dtype {t.dtype}")


def _torch_dt(dt: int) -> torch.dtype:
    return {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16, MOE_FP8_E4M3: torch.uint8}[dt]


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------------------------------
# entry points
# ------------------------------------------------------------------------------------------

def moe_router_logits(x: torch.Tensor, w_r: torch.Tensor, z: Optional[torch.Tensor] = None,
                      ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """z [N, E] fp32 = x [N, H] . w_r [E, H]^T (x and w_r of one dtype)."""
    N, H = x.shape
    E = w_r.shape[0]
    if w_r.shape[1] != H or w_r.dtype != x.dtype:
        raise ValueError("w_r must be [E, H] of x's dtype")
    if z is None:
        z = torch.empty((N, E), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = _workspace(moe_workspace_bytes(MOE_OP_ROUTER, N, H, 0, E, 0, _dt(x)), x.device)
    _check("moe_router_logits", lib().moe_router_logits(_ptr(x), _dt(x), N, H, _ptr(w_r), E, _ptr(z),
                                                        _ptr(ws), ws.numel(), _stream(x)))
    return z


def moe_route(z: torch.Tensor, k: int, bias: Optional[torch.Tensor] = None, n_group: int = 0,
              topk_group: int = 0, topk_idx: Optional[torch.Tensor] = None,
              topk_gate: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    N, E = z.shape
    if topk_idx is None:
        topk_idx = torch.empty((N, k), dtype=torch.int32, device=z.device)
    if topk_gate is None:
        topk_gate = torch.empty((N, k), dtype=torch.float32, device=z.device)
    _check("moe_route", lib().moe_route(_ptr(z), N, E, k, _ptr(bias), n_group, topk_group,
                                        _ptr(topk_idx), _ptr(topk_gate), _stream(z)))
    return topk_idx, topk_gate


def moe_dispatch_layout(topk_idx: torch.Tensor, E: int, out=None, ws: Optional[torch.Tensor] = None):
    """Returns (n_e [E], offsets [E+1], send_pos [N*k], src_slot [N*k]) int32."""
    N, k = topk_idx.shape
    dev = topk_idx.device
    if out is None:
        out = (torch.empty(E, dtype=torch.int32, device=dev),
               torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty(N * k, dtype=torch.int32, device=dev),
               torch.empty(N * k, dtype=torch.int32, device=dev))
    n_e, offsets, send_pos, src_slot = out
    if ws is None:
        ws = _workspace(moe_workspace_bytes(MOE_OP_DISPATCH_LAYOUT, N, 0, 0, E, k, 0), dev)
    _check("moe_dispatch_layout", lib().moe_dispatch_layout(
        _ptr(topk_idx), N, k, E, _ptr(n_e), _ptr(offsets), _ptr(send_pos), _ptr(src_slot),
        _ptr(ws), ws.numel(), _stream(topk_idx)))
    return n_e, offsets, send_pos, src_slot


def moe_dispatch_layout_noalloc(topk_idx: torch.Tensor, E: int, out=None):
    """moe_dispatch_layout without a workspace: the counts go to the library's fixed device
    scratch.  Returns (n_e, offsets, send_pos, src_slot) int32."""
    N, k = topk_idx.shape
    dev = topk_idx.device
    if out is None:
        out = (torch.empty(E, dtype=torch.int32, device=dev),
               torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty(N * k, dtype=torch.int32, device=dev),
               torch.empty(N * k, dtype=torch.int32, device=dev))
    n_e, offsets, send_pos, src_slot = out
    _check("moe_dispatch_layout_noalloc", lib().moe_dispatch_layout_noalloc(
        _ptr(topk_idx), N, k, E, _ptr(n_e), _ptr(offsets), _ptr(send_pos), _ptr(src_slot), _stream(topk_idx)))
    return n_e, offsets, send_pos, src_slot


def moe_permute(x: torch.Tensor, send_pos: torch.Tensor, k: int, perm_dt: Optional[int] = None,
                x_perm: Optional[torch.Tensor] = None, perm_scale: Optional[torch.Tensor] = None):
    """x_perm (and the fp8 block scales when perm_dt is MOE_FP8_E4M3)."""
    N, H = x.shape
    pdt = _dt(x) if perm_dt is None else perm_dt
    if x_perm is None:
        x_perm = torch.empty((N * k, H), dtype=_torch_dt(pdt), device=x.device)
    if pdt == MOE_FP8_E4M3 and perm_scale is None:
        perm_scale = torch.empty((N * k, H // 128), dtype=torch.float32, device=x.device)
    _check("moe_permute", lib().moe_permute(_ptr(x), _dt(x), N, H, k, _ptr(send_pos), _ptr(x_perm),
                                            pdt, _ptr(perm_scale), _stream(x)))
    return (x_perm, perm_scale) if pdt == MOE_FP8_E4M3 else x_perm


def moe_quantize_fp8(x: torch.Tensor, q: Optional[torch.Tensor] = None,
                     scale: Optional[torch.Tensor] = None):
    """(codes uint8 of x's shape, fp32 scales [..., cols / 128]) for the rows of x."""
    cols = x.shape[-1]
    rows = x.numel() // cols
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(tuple(x.shape[:-1]) + (cols // 128,), dtype=torch.float32, device=x.device)
    _check("moe_quantize_fp8", lib().moe_quantize_fp8(_ptr(x), _dt(x), rows, cols, _ptr(q),
                                                      _ptr(scale), _stream(x)))
    return q, scale


def moe_dequantize_fp8(q: torch.Tensor, scale: torch.Tensor, out: Optional[torch.Tensor] = None):
    """bf16 values (code times its block's scale, one rounding) of e4m3 codes q [..., cols]
    with scales [..., cols / 128]."""
    cols = q.shape[-1]
    rows = q.numel() // cols
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _check("moe_dequantize_fp8", lib().moe_dequantize_fp8(_ptr(q), _ptr(scale), rows, cols, _ptr(out),
                                                          _stream(q)))
    return out


def moe_expert_gate_up(a: torch.Tensor, offsets: torch.Tensor, w13: torch.Tensor,
                       a_scale: Optional[torch.Tensor] = None, w13_scale: Optional[torch.Tensor] = None,
                       h: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    rows, H = a.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    adt = _dt(a)
    if h is None:
        h = torch.empty((rows, I), dtype=torch.float32 if adt == MOE_F32 else torch.bfloat16,
                        device=a.device)
    if ws is None:
        ws = _workspace(moe_workspace_bytes(MOE_OP_EXPERT_GEMM, rows, H, I, E, 1, adt), a.device)
    _check("moe_expert_gate_up", lib().moe_expert_gate_up(
        _ptr(a), _ptr(a_scale), adt, _ptr(offsets), E, rows, H, I, _ptr(w13), _ptr(w13_scale),
        _ptr(h), _ptr(ws), ws.numel(), _stream(a)))
    return h


def moe_expert_gate_up_gathered(x: torch.Tensor, src_slot: torch.Tensor, k: int, offsets: torch.Tensor,
                                w13: torch.Tensor, rows: Optional[int] = None, h: Optional[torch.Tensor] = None,
                                ws: Optional[torch.Tensor] = None):
    """Gate/up GEMM whose row r reads token src_slot[r] // k of x (no permuted copy)."""
    N, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    if rows is None:
        rows = src_slot.numel()
    if h is None:
        h = torch.empty((rows, I), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = _workspace(moe_workspace_bytes(MOE_OP_EXPERT_GEMM, rows, H, I, E, 1, MOE_BF16), x.device)
    _check("moe_expert_gate_up_gathered", lib().moe_expert_gate_up_gathered(
        _ptr(x), _dt(x), N, _ptr(src_slot), k, _ptr(offsets), E, rows, H, I, _ptr(w13), _ptr(h),
        _ptr(ws), ws.numel(), _stream(x)))
    return h


def moe_expert_gate_up_gathered_shared(x: torch.Tensor, src_slot: torch.Tensor, k: int, offsets: torch.Tensor,
                                       w13: torch.Tensor, shared_w13: torch.Tensor, rows: Optional[int] = None,
                                       h: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                                       au: Optional[torch.Tensor] = None):
    """Routed gate/up (rows gathered from x) plus the shared expert on all N tokens in one
    launch: h [rows + N, I], the shared expert's rows last (and the pre-activations into au
    [rows + N, 2I] when given)."""
    N, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    if rows is None:
        rows = src_slot.numel()
    if h is None:
        h = torch.empty((rows + N, I), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = _workspace(moe_workspace_bytes(MOE_OP_EXPERT_GEMM, rows + N, H, I, E + 1, 1, MOE_BF16), x.device)
    _check("moe_expert_gate_up_gathered_shared", lib().moe_expert_gate_up_gathered_shared(
        _ptr(x), _dt(x), N, _ptr(src_slot), k, _ptr(offsets), E, rows, H, I, _ptr(w13), _ptr(shared_w13),
        _ptr(h), _ptr(au), _ptr(ws), ws.numel(), _stream(x)))
    return h


def moe_expert_down_shared(h: torch.Tensor, offsets: torch.Tensor, w2: torch.Tensor, shared_w2: torch.Tensor,
                           rows: int, out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                           src_slot: Optional[torch.Tensor] = None, topk_gate: Optional[torch.Tensor] = None):
    """Routed down GEMM over rows [0, rows) of h plus the shared expert's down over the rest:
    out [h rows, H], the shared expert's rows last.  With src_slot and topk_gate, routed row r
    is multiplied by its gate topk_gate.flat[src_slot[r]] in the epilogue."""
    total, I = h.shape
    E, H, _ = w2.shape
    n_shared = total - rows
    if out is None:
        out = torch.empty((total, H), dtype=h.dtype, device=h.device)
    if ws is None:
        ws = _workspace(moe_workspace_bytes(MOE_OP_EXPERT_GEMM, total, H, I, E + 1, 1, MOE_BF16), h.device)
    _check("moe_expert_down_shared", lib().moe_expert_down_shared(
        _ptr(h), _dt(h), _ptr(offsets), E, rows, n_shared, I, H, _ptr(w2), _ptr(shared_w2), _ptr(src_slot),
        _ptr(topk_gate), _ptr(out), _dt(out), _ptr(ws), ws.numel(), _stream(h)))
    return out


def moe_expert_gate_up_gathered_shared_e4m3(x: torch.Tensor, src_slot: torch.Tensor, k: int, offsets: torch.Tensor,
                                            w13: torch.Tensor, w13_scale: torch.Tensor, shared_w13: torch.Tensor,
                                            shared_w13_scale: torch.Tensor, rows: Optional[int] = None,
                                            h: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """moe_expert_gate_up_gathered_shared on e4m3 weights (codes and block scales); x [N, H]
    bf16 holds the tokens' fp8 payload values."""
    N, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    if rows is None:
        rows = src_slot.numel()
    if h is None:
        h = torch.empty((rows + N, I), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = _workspace(moe_workspace_bytes(MOE_OP_EXPERT_GEMM, rows + N, H, I, E + 1, 1, MOE_BF16), x.device)
    _check("moe_expert_gate_up_gathered_shared_e4m3", lib().moe_expert_gate_up_gathered_shared_e4m3(
        _ptr(x), N, _ptr(src_slot), k, _ptr(offsets), E, rows, H, I, _ptr(w13), _ptr(w13_scale), _ptr(shared_w13),
        _ptr(shared_w13_scale), _ptr(h), _ptr(ws), ws.numel(), _stream(x)))
    return h


def moe_expert_down_shared_e4m3(h: torch.Tensor, offsets: torch.Tensor, w2: torch.Tensor, w2_scale: torch.Tensor,
                                shared_w2: torch.Tensor, shared_w2_scale: torch.Tensor, rows: int,
                                out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """moe_expert_down_shared on e4m3 weights (codes and block scales)."""
    total, I = h.shape
    E, H, _ = w2.shape
    if out is None:
        out = torch.empty((total, H), dtype=torch.bfloat16, device=h.device)
    if ws is None:
        ws = _workspace(moe_workspace_bytes(MOE_OP_EXPERT_GEMM, total, H, I, E + 1, 1, MOE_BF16), h.device)
    _check("moe_expert_down_shared_e4m3", lib().moe_expert_down_shared_e4m3(
        _ptr(h), _ptr(offsets), E, rows, total - rows, I, H, _ptr(w2), _ptr(w2_scale), _ptr(shared_w2),
        _ptr(shared_w2_scale), _ptr(out), _ptr(ws), ws.numel(), _stream(h)))
    return out


def moe_expert_down(h: torch.Tensor, offsets: torch.Tensor, w2: torch.Tensor,
                    w2_scale: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None):
    rows, I = h.shape
    E, H, _ = w2.shape
    hdt = _dt(h)
    if out is None:
        out = torch.empty((rows, H), dtype=h.dtype, device=h.device)
    if ws is None:
        ws = _workspace(moe_workspace_bytes(MOE_OP_EXPERT_GEMM, rows, H, I, E, 1, hdt), h.device)
    _check("moe_expert_down", lib().moe_expert_down(
        _ptr(h), hdt, _ptr(offsets), E, rows, I, H, _ptr(w2), _dt(w2), _ptr(w2_scale), _ptr(out),
        _dt(out), _ptr(ws), ws.numel(), _stream(h)))
    return out


def moe_grouped_ffn(a: torch.Tensor, offsets: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor,
                    a_scale: Optional[torch.Tensor] = None, w13_scale: Optional[torch.Tensor] = None,
                    w2_scale: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None):
    rows, H = a.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    adt = _dt(a)
    odt = MOE_F32 if adt == MOE_F32 else MOE_BF16
    if out is None:
        out = torch.empty((rows, H), dtype=_torch_dt(odt), device=a.device)
    if ws is None:
        ws = _workspace(moe_workspace_bytes(MOE_OP_GROUPED_FFN, rows, H, I, E, 1, adt), a.device)
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(
        _ptr(a), _ptr(a_scale), adt, _ptr(offsets), E, rows, H, I, _ptr(w13), _ptr(w13_scale),
        _ptr(w2), _ptr(w2_scale), _ptr(out), odt, _ptr(ws), ws.numel(), _stream(a)))
    return out


def moe_combine(expert_out: torch.Tensor, send_pos: torch.Tensor, topk_gate: Optional[torch.Tensor],
                shared_out: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                y_dtype: Optional[torch.dtype] = None, k: Optional[int] = None):
    """topk_gate None: the expert outputs already carry their gates (pass k)."""
    if topk_gate is not None:
        N, k = topk_gate.shape
    else:
        N = send_pos.numel() // k
    H = expert_out.shape[1]
    if y is None:
        y = torch.empty((N, H), dtype=y_dtype or expert_out.dtype, device=expert_out.device)
    _check("moe_combine", lib().moe_combine(
        _ptr(expert_out), _dt(expert_out), N, H, k, _ptr(send_pos), _ptr(topk_gate),
        _ptr(shared_out), _ptr(y), _dt(y), _stream(expert_out)))
    return y


# ------------------------------------------------------------------------------------------
# backward pass
# ------------------------------------------------------------------------------------------

def moe_combine_backward(dy: torch.Tensor, send_pos: torch.Tensor, topk_gate: torch.Tensor,
                         expert_out: torch.Tensor, d_expert_out: Optional[torch.Tensor] = None,
                         d_gate: Optional[torch.Tensor] = None):
    """(d_expert_out [rows, H] in dy's dtype, d_gate [N, k] fp32) of moe_combine's weighted sum."""
    N, H = dy.shape
    k = topk_gate.shape[1]
    if d_expert_out is None:
        d_expert_out = torch.empty_like(expert_out, dtype=dy.dtype)
    if d_gate is None:
        d_gate = torch.empty((N, k), dtype=torch.float32, device=dy.device)
    if expert_out.dtype != dy.dtype or d_expert_out.dtype != dy.dtype:
        raise ValueError("dy, expert_out and d_expert_out share one dtype")
    _check("moe_combine_backward", lib().moe_combine_backward(
        _ptr(dy), _dt(dy), N, H, k, _ptr(send_pos), _ptr(topk_gate), _ptr(expert_out), _ptr(d_expert_out),
        _ptr(d_gate), _stream(dy)))
    return d_expert_out, d_gate


def moe_expert_gate_up_preact(x: torch.Tensor, offsets: torch.Tensor, w13: torch.Tensor, rows: Optional[int] = None,
                              src_slot: Optional[torch.Tensor] = None, k: int = 1, au: Optional[torch.Tensor] = None,
                              ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """au [rows, 2I] bf16 = a W13_e^T per segment; a = x[src_slot[r] // k] (src_slot given) or x's rows."""
    N, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    if rows is None:
        rows = src_slot.numel() if src_slot is not None else N
    if au is None:
        au = torch.empty((rows, 2 * I), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = _workspace(moe_workspace_bytes(MOE_OP_EXPERT_GEMM, rows, H, I, E, 1, MOE_BF16), x.device)
    _check("moe_expert_gate_up_preact", lib().moe_expert_gate_up_preact(
        _ptr(x), _dt(x), N, _ptr(src_slot), k, _ptr(offsets), E, rows, H, I, _ptr(w13), _ptr(au), _ptr(ws),
        ws.numel(), _stream(x)))
    return au


def moe_swiglu_backward(au: torch.Tensor, dh: torch.Tensor, d_au: Optional[torch.Tensor] = None,
                        h: Optional[torch.Tensor] = None, want_h: bool = True):
    """(d_au [rows, 2I], h [rows, I] or None) from the pre-activations au and dh (bf16)."""
    rows, I = dh.shape
    if d_au is None:
        d_au = torch.empty((rows, 2 * I), dtype=torch.bfloat16, device=dh.device)
    if h is None and want_h:
        h = torch.empty((rows, I), dtype=torch.bfloat16, device=dh.device)
    _check("moe_swiglu_backward", lib().moe_swiglu_backward(_ptr(au), _ptr(dh), rows, I, _ptr(d_au), _ptr(h),
                                                            _stream(dh)))
    return d_au, h


def moe_expert_dgrad(dC: torch.Tensor, offsets: torch.Tensor, w: torch.Tensor, out: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out [rows, N] bf16 = dC[r] W_e per segment, W [E, K, N] as stored."""
    rows, K = dC.shape
    E, K2, N = w.shape
    if K2 != K:
        raise ValueError("dC's columns must match the weight's K")
    if out is None:
        out = torch.empty((rows, N), dtype=torch.bfloat16, device=dC.device)
    if ws is None:
        ws = _workspace(moe_workspace_bytes(MOE_OP_EXPERT_DGRAD, rows, 0, 0, E, 0, 0), dC.device)
    _check("moe_expert_dgrad", lib().moe_expert_dgrad(_ptr(dC), _ptr(offsets), E, rows, K, N, _ptr(w), _ptr(out),
                                                      _ptr(ws), ws.numel(), _stream(dC)))
    return out


def moe_expert_wgrad(a: torch.Tensor, b: torch.Tensor, offsets: torch.Tensor, b_rows: Optional[torch.Tensor] = None,
                     b_div: int = 1, dw: Optional[torch.Tensor] = None, dw_dtype: torch.dtype = torch.float32,
                     rows: Optional[int] = None) -> torch.Tensor:
    """dW [E, M, N] = A_e^T B_e over each segment's rows (B's row r = b[b_rows[r] // b_div] if given)."""
    E = offsets.numel() - 1
    M = a.shape[1]
    N = b.shape[1]
    if rows is None:
        rows = a.shape[0]
    if dw is None:
        dw = torch.empty((E, M, N), dtype=dw_dtype, device=a.device)
    _check("moe_expert_wgrad", lib().moe_expert_wgrad(
        _ptr(a), M, _ptr(b), N, _ptr(b_rows), b_div, b.shape[0], _ptr(offsets), E, rows, _ptr(dw), _dt(dw),
        _stream(a)))
    return dw


def moe_router_backward(topk_gate: torch.Tensor, d_gate: torch.Tensor, offsets: torch.Tensor,
                        src_slot: torch.Tensor, x: torch.Tensor, dz: Optional[torch.Tensor] = None,
                        dw_r: Optional[torch.Tensor] = None, dw_dtype: torch.dtype = torch.float32):
    """(dz [N, k] fp32 on the selected logits, dW_r [E, H])."""
    N, k = topk_gate.shape
    E = offsets.numel() - 1
    H = x.shape[1]
    rows = src_slot.numel()
    if dz is None:
        dz = torch.empty((N, k), dtype=torch.float32, device=x.device)
    if dw_r is None:
        dw_r = torch.empty((E, H), dtype=dw_dtype, device=x.device)
    _check("moe_router_backward", lib().moe_router_backward(
        _ptr(topk_gate), _ptr(d_gate), N, k, _ptr(offsets), _ptr(src_slot), E, rows, _ptr(x), _dt(x), H, _ptr(dz),
        _ptr(dw_r), _dt(dw_r), _stream(x)))
    return dz, dw_r


def moe_router_input_grad(w_r: torch.Tensor, topk_idx: torch.Tensor, dz: torch.Tensor,
                          rest: Optional[torch.Tensor] = None, dx: Optional[torch.Tensor] = None):
    """dx [N, H] = sum_j dz[t, j] W_r[topk_idx[t, j]] (+ rest): the router's input gradient."""
    E, H = w_r.shape
    N, k = topk_idx.shape
    if dx is None:
        dx = torch.empty((N, H), dtype=w_r.dtype, device=w_r.device)
    _check("moe_router_input_grad", lib().moe_router_input_grad(
        _ptr(w_r), _dt(w_r), N, E, H, k, _ptr(topk_idx), _ptr(dz), _ptr(rest), _ptr(dx), _dt(dx), _stream(w_r)))
    return dx


def moe_stream_probe(src: torch.Tensor, ratio: int, dst: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Read-mostly streaming probe: src holds ratio * n 16-byte words, dst n words (uint8
    tensors); dst[i] = the integer sum of src[j * n + i] over j."""
    nbytes = src.numel() * src.element_size()
    if nbytes % (16 * ratio):
        raise ValueError("src must hold ratio * n 16-byte words")
    n16 = nbytes // (16 * ratio)
    if dst is None:
        dst = torch.empty(n16 * 16, dtype=torch.uint8, device=src.device)
    _check("moe_stream_probe", lib().moe_stream_probe(_ptr(src), n16, ratio, _ptr(dst), _stream(src)))
    return dst
