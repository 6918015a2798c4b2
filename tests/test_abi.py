"""The C ABI on the CPU: the library loads, exports every declared symbol, and rejects
invalid arguments on the host before anything is enqueued (no GPU needed)."""
import ctypes

import pytest

import combine_grouped_gemm_amd as moe
from combine_grouped_gemm_amd import (MOE_BF16, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED,
                                      MOE_ERR_WORKSPACE, MOE_F32, MOE_FP8_E4M3, MOE_OK)

FAKE = 4096  # a non-null, 16-byte aligned host integer: never dereferenced on these paths


@pytest.fixture(scope="module")
def L():
    return moe.lib()


def test_exports_every_declared_symbol(L):
    names = moe.declared_symbols()
    assert {"moe_route", "moe_dispatch_layout", "moe_permute", "moe_grouped_ffn", "moe_combine",
            "moe_workspace_bytes", "moe_status_str"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
        assert ctypes.cast(getattr(L, n), ctypes.c_void_p).value


def test_status_strings_and_version():
    assert moe.moe_status_str(MOE_OK) == "ok"
    assert "workspace" in moe.moe_status_str(MOE_ERR_WORKSPACE)
    assert moe.moe_version().count(".") == 2


def test_router_validation_and_workspace(L):
    ws_b = lambda N, H, E, dt: moe.moe_workspace_bytes(moe.MOE_OP_ROUTER, N, H, 0, E, 0, dt)
    # DeepSeek-V3 shape: 32 tiles of 256 x 256, K in 8 parts (one per XCD) of fp32 partial sums
    assert ws_b(8192, 7168, 256, MOE_BF16) == 8 * 8192 * 256 * 4
    # decode batch: one tile, K in 14 parts (the most parts, up to 16, dividing 56 blocks of 128)
    assert ws_b(128, 7168, 256, MOE_BF16) == 14 * 128 * 256 * 4
    # enough tiles for every CU: no parts; fp32 operands and E % 4 != 0: the plain kernel
    assert ws_b(65536, 7168, 256, MOE_BF16) == 0
    assert ws_b(256, 128, 8, MOE_F32) == 0
    assert ws_b(512, 1024, 6, MOE_BF16) == 0
    ws = ws_b(8192, 7168, 256, MOE_BF16)
    f = L.moe_router_logits
    assert f(FAKE, MOE_BF16, -1, 7168, FAKE, 256, FAKE, FAKE, ws, None) == MOE_ERR_INVALID_ARG
    assert f(FAKE, MOE_BF16, 8192, 7168, FAKE, 0, FAKE, FAKE, ws, None) == MOE_ERR_INVALID_ARG
    assert f(FAKE, MOE_BF16, 8192, 0, FAKE, 256, FAKE, FAKE, ws, None) == MOE_ERR_INVALID_ARG
    assert f(FAKE, MOE_FP8_E4M3, 8192, 7168, FAKE, 256, FAKE, FAKE, ws, None) == MOE_ERR_UNSUPPORTED
    assert f(FAKE, MOE_BF16, 8192, 7168, FAKE, 2048, FAKE, FAKE, ws, None) == MOE_ERR_UNSUPPORTED
    assert f(FAKE, MOE_BF16, 8192, 7168, None, 256, FAKE, FAKE, ws, None) == MOE_ERR_INVALID_ARG
    assert f(FAKE, MOE_BF16, 8192, 7168, FAKE, 256, None, FAKE, ws, None) == MOE_ERR_INVALID_ARG
    assert f(FAKE, MOE_BF16, 8192, 7168, FAKE, 256, FAKE, FAKE, ws - 1, None) == MOE_ERR_WORKSPACE
    assert f(FAKE, MOE_BF16, 8192, 7168, FAKE, 256, FAKE, None, ws, None) == MOE_ERR_WORKSPACE
    assert f(FAKE + 8, MOE_BF16, 8192, 7168, FAKE, 256, FAKE, FAKE, ws, None) == MOE_ERR_INVALID_ARG
    assert f(FAKE, MOE_BF16, 8192, 7168, FAKE, 256, FAKE + 4, FAKE, ws, None) == MOE_ERR_INVALID_ARG
    assert f(None, MOE_BF16, 0, 7168, None, 256, None, None, 0, None) == MOE_OK


def test_route_validation(L):
    r = lambda *a: L.moe_route(*a)
    assert r(FAKE, 4, 8, 9, None, 0, 0, FAKE, FAKE, None) == MOE_ERR_INVALID_ARG      # k > E
    assert r(FAKE, 4, 8, 0, None, 0, 0, FAKE, FAKE, None) == MOE_ERR_INVALID_ARG      # k = 0
    assert r(FAKE, 4, 2048, 8, None, 0, 0, FAKE, FAKE, None) == MOE_ERR_UNSUPPORTED   # E > 1024
    assert r(FAKE, 4, 64, 33, None, 0, 0, FAKE, FAKE, None) == MOE_ERR_UNSUPPORTED    # k > 32
    assert r(FAKE, 4, 10, 2, None, 4, 2, FAKE, FAKE, None) == MOE_ERR_INVALID_ARG     # E % n_group
    assert r(FAKE, 4, 16, 8, None, 8, 2, FAKE, FAKE, None) == MOE_ERR_INVALID_ARG     # k > 2 groups * 2
    assert r(FAKE, 4, 16, 2, None, 8, 9, FAKE, FAKE, None) == MOE_ERR_INVALID_ARG     # topk_group > n_group
    assert r(FAKE, 4, 16, 2, None, 0, 2, FAKE, FAKE, None) == MOE_ERR_INVALID_ARG     # topk_group w/o groups
    assert r(None, 4, 16, 2, None, 0, 0, FAKE, FAKE, None) == MOE_ERR_INVALID_ARG     # null z
    assert r(None, 0, 16, 2, None, 0, 0, None, None, None) == MOE_OK                  # N = 0: no-op


def test_layout_validation_and_workspace(L):
    ws = moe.moe_workspace_bytes(moe.MOE_OP_DISPATCH_LAYOUT, 8192, 0, 0, 256, 8, 0)
    assert ws >= 64 * 256 * 4 and ws % 256 == 0
    f = L.moe_dispatch_layout
    assert f(FAKE, 8192, 8, 256, FAKE, FAKE, FAKE, FAKE, FAKE, ws - 1, None) == MOE_ERR_WORKSPACE
    assert f(FAKE, 8192, 8, 256, FAKE, FAKE, FAKE, FAKE, None, ws, None) == MOE_ERR_WORKSPACE
    assert f(FAKE, 8192, 0, 256, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == MOE_ERR_INVALID_ARG
    assert f(None, 0, 8, 256, None, None, None, None, None, 0, None) == MOE_OK


def test_permute_validation(L):
    f = L.moe_permute
    assert f(FAKE, MOE_BF16, 4, 100, 2, FAKE, FAKE, MOE_BF16, None, None) == MOE_ERR_UNSUPPORTED  # 200 B rows
    assert f(FAKE, MOE_BF16, 4, 192, 2, FAKE, FAKE, MOE_FP8_E4M3, FAKE, None) == MOE_ERR_UNSUPPORTED  # H % 128
    assert f(FAKE, MOE_BF16, 4, 256, 2, FAKE, FAKE, MOE_FP8_E4M3, None, None) == MOE_ERR_INVALID_ARG  # no scales
    assert f(FAKE, MOE_BF16, 4, 256, 2, FAKE, FAKE, MOE_F32, None, None) == MOE_ERR_UNSUPPORTED     # bf16 -> f32
    assert f(FAKE + 8, MOE_BF16, 4, 256, 2, FAKE, FAKE, MOE_BF16, None, None) == MOE_ERR_INVALID_ARG  # misaligned
    assert f(None, MOE_BF16, 0, 256, 2, None, None, MOE_BF16, None, None) == MOE_OK


def test_ffn_validation_and_workspace(L):
    rows, H, I, E = 65536, 7168, 2048, 256
    ws = moe.moe_workspace_bytes(moe.MOE_OP_GROUPED_FFN, rows, H, I, E, 1, MOE_BF16)
    sched = moe.moe_workspace_bytes(moe.MOE_OP_EXPERT_GEMM, rows, H, I, E, 1, MOE_BF16)
    assert ws == sched + rows * I * 2
    f = L.moe_grouped_ffn
    args = lambda **kw: dict(dict(a=FAKE, a_scale=None, a_dt=MOE_BF16, offsets=FAKE, E=E, rows=rows,
                                  H=H, I=I, w13=FAKE, w13_scale=None, w2=FAKE, w2_scale=None,
                                  out=FAKE, out_dt=MOE_BF16, ws=FAKE, ws_bytes=ws, s=None), **kw)
    call = lambda **kw: f(*args(**kw).values())
    assert call(ws_bytes=ws - 1) == MOE_ERR_WORKSPACE
    assert call(H=7000) == MOE_ERR_UNSUPPORTED
    assert call(I=2000) == MOE_ERR_UNSUPPORTED
    assert call(E=0) == MOE_ERR_INVALID_ARG
    assert call(E=2048) == MOE_ERR_INVALID_ARG
    assert call(out_dt=MOE_F32) == MOE_ERR_UNSUPPORTED
    assert call(a_dt=MOE_FP8_E4M3, a_scale=None) == MOE_ERR_INVALID_ARG
    assert call(offsets=None) == MOE_ERR_INVALID_ARG
    assert call(rows=0, ws=None, ws_bytes=0) == MOE_OK


def test_gathered_gate_up_validation(L):
    rows, H, I, E, N, k = 65536, 7168, 2048, 256, 8192, 8
    sched = moe.moe_workspace_bytes(moe.MOE_OP_EXPERT_GEMM, rows, H, I, E, 1, MOE_BF16)
    f = L.moe_expert_gate_up_gathered
    args = lambda **kw: dict(dict(x=FAKE, x_dt=MOE_BF16, N=N, src_slot=FAKE, k=k, offsets=FAKE, E=E,
                                  rows=rows, H=H, I=I, w13=FAKE, h=FAKE, ws=FAKE, ws_bytes=sched, s=None), **kw)
    call = lambda **kw: f(*args(**kw).values())
    assert call(x_dt=MOE_FP8_E4M3) == MOE_ERR_UNSUPPORTED
    assert call(x_dt=MOE_F32) == MOE_ERR_UNSUPPORTED
    assert call(ws_bytes=sched - 1) == MOE_ERR_WORKSPACE
    assert call(k=0) == MOE_ERR_INVALID_ARG
    assert call(src_slot=None) == MOE_ERR_INVALID_ARG
    assert call(N=0) == MOE_ERR_INVALID_ARG
    assert call(N=300000) == MOE_ERR_UNSUPPORTED        # N * H * 2 >= 2^32
    assert call(H=7000) == MOE_ERR_UNSUPPORTED
    assert call(x=FAKE + 8) == MOE_ERR_INVALID_ARG
    assert call(rows=0, ws=None, ws_bytes=0) == MOE_OK


def test_combine_validation(L):
    f = L.moe_combine
    assert f(FAKE, MOE_BF16, 4, 100, 2, FAKE, FAKE, None, FAKE, MOE_BF16, None) == MOE_ERR_UNSUPPORTED
    assert f(FAKE, MOE_FP8_E4M3, 4, 128, 2, FAKE, FAKE, None, FAKE, MOE_BF16, None) == MOE_ERR_UNSUPPORTED
    assert f(FAKE, MOE_BF16, 4, 128, 0, FAKE, FAKE, None, FAKE, MOE_BF16, None) == MOE_ERR_INVALID_ARG
    assert f(None, MOE_BF16, 4, 128, 2, FAKE, FAKE, None, FAKE, MOE_BF16, None) == MOE_ERR_INVALID_ARG
    assert f(None, MOE_BF16, 0, 128, 2, None, None, None, None, MOE_BF16, None) == MOE_OK
    # topk_gate NULL is the gate-free sum (outputs that already carry their gates): accepted
    assert f(FAKE, MOE_BF16, 0, 128, 2, FAKE, None, None, FAKE, MOE_BF16, None) == MOE_OK
    assert f(FAKE, MOE_BF16, 4, 128, 2, None, None, None, FAKE, MOE_BF16, None) == MOE_ERR_INVALID_ARG


def test_no_cpu_fallback_in_binding():
    import inspect
    src = inspect.getsource(moe)
    assert "oracle" not in src.replace("no fallback", "")


def test_shared_segment_validation(L):
    """The fused routed + shared entry points: dtype, shape, workspace and pointer checks happen
    on the host, before anything is enqueued."""
    rows, H, I, E, N, k = 65536, 7168, 2048, 256, 8192, 8
    sched = moe.moe_workspace_bytes(moe.MOE_OP_EXPERT_GEMM, rows + N, H, I, E + 1, 1, MOE_BF16)
    assert sched > moe.moe_workspace_bytes(moe.MOE_OP_EXPERT_GEMM, rows, H, I, E, 1, MOE_BF16)
    f = L.moe_expert_gate_up_gathered_shared
    args = lambda **kw: dict(dict(x=FAKE, x_dt=MOE_BF16, N=N, src_slot=FAKE, k=k, offsets=FAKE, E=E,
                                  rows=rows, H=H, I=I, w13=FAKE, sw13=FAKE, h=FAKE, au=None, ws=FAKE, ws_bytes=sched,
                                  s=None), **kw)
    call = lambda **kw: f(*args(**kw).values())
    assert call(x_dt=MOE_F32) == MOE_ERR_UNSUPPORTED
    assert call(ws_bytes=sched - 1) == MOE_ERR_WORKSPACE
    assert call(sw13=None) == MOE_ERR_INVALID_ARG
    assert call(src_slot=None) == MOE_ERR_INVALID_ARG
    assert call(k=0) == MOE_ERR_INVALID_ARG
    assert call(au=FAKE + 8) == MOE_ERR_INVALID_ARG      # misaligned pre-activation output
    assert call(E=1024) == MOE_ERR_UNSUPPORTED            # E + 1 segments must fit the schedule
    assert call(I=2000) == MOE_ERR_UNSUPPORTED
    assert call(N=300000, ws_bytes=1 << 40) == MOE_ERR_UNSUPPORTED   # N * H * 2 >= 2^32
    assert call(sw13=FAKE + 8) == MOE_ERR_INVALID_ARG
    assert call(rows=0, N=0, ws=None, ws_bytes=0) == MOE_OK
    g = L.moe_expert_down_shared
    dargs = lambda **kw: dict(dict(h=FAKE, h_dt=MOE_BF16, offsets=FAKE, E=E, rows=rows, n=N, I=I, H=H,
                                   w2=FAKE, sw2=FAKE, slot=None, gate=None, out=FAKE, out_dt=MOE_BF16, ws=FAKE,
                                   ws_bytes=sched, s=None), **kw)
    dcall = lambda **kw: g(*dargs(**kw).values())
    assert dcall(h_dt=MOE_F32) == MOE_ERR_UNSUPPORTED
    assert dcall(out_dt=MOE_F32) == MOE_ERR_UNSUPPORTED
    assert dcall(ws_bytes=sched - 1) == MOE_ERR_WORKSPACE
    assert dcall(sw2=None) == MOE_ERR_INVALID_ARG
    assert dcall(n=-1) == MOE_ERR_INVALID_ARG
    assert dcall(H=7000) == MOE_ERR_UNSUPPORTED
    assert dcall(rows=0, n=0, ws=None, ws_bytes=0) == MOE_OK
    assert dcall(slot=FAKE) == MOE_ERR_INVALID_ARG     # gates need both the slot map and the gates
    assert dcall(gate=FAKE) == MOE_ERR_INVALID_ARG


def test_fp8_weight_entry_points_validation(L):
    """The e4m3-weight fused launches, the fp8 dequantizer and the fp8 gate/up workspace: every
    check happens on the host, before anything is enqueued."""
    rows, H, I, E, N, k = 65536, 7168, 2048, 256, 8192, 8
    sched = moe.moe_workspace_bytes(moe.MOE_OP_EXPERT_GEMM, rows + N, H, I, E + 1, 1, MOE_BF16)
    f = L.moe_expert_gate_up_gathered_shared_e4m3
    args = lambda **kw: dict(dict(x=FAKE, N=N, src_slot=FAKE, k=k, offsets=FAKE, E=E, rows=rows, H=H, I=I,
                                  w13=FAKE, w13_s=FAKE, sw13=FAKE, sw13_s=FAKE, h=FAKE, ws=FAKE, ws_bytes=sched,
                                  s=None), **kw)
    call = lambda **kw: f(*args(**kw).values())
    assert call(ws_bytes=sched - 1) == MOE_ERR_WORKSPACE
    assert call(w13_s=None) == MOE_ERR_INVALID_ARG
    assert call(sw13_s=None) == MOE_ERR_INVALID_ARG
    assert call(src_slot=None) == MOE_ERR_INVALID_ARG
    assert call(k=0) == MOE_ERR_INVALID_ARG
    assert call(I=2000) == MOE_ERR_UNSUPPORTED
    assert call(E=1024) == MOE_ERR_UNSUPPORTED
    assert call(N=300000, ws_bytes=1 << 40) == MOE_ERR_UNSUPPORTED   # N * H * 2 >= 2^32
    assert call(x=FAKE + 8) == MOE_ERR_INVALID_ARG
    assert call(rows=0, N=0, ws=None, ws_bytes=0) == MOE_OK
    g = L.moe_expert_down_shared_e4m3
    dargs = lambda **kw: dict(dict(h=FAKE, offsets=FAKE, E=E, rows=rows, n=N, I=I, H=H, w2=FAKE, w2_s=FAKE,
                                   sw2=FAKE, sw2_s=FAKE, out=FAKE, ws=FAKE, ws_bytes=sched, s=None), **kw)
    dcall = lambda **kw: g(*dargs(**kw).values())
    assert dcall(ws_bytes=sched - 1) == MOE_ERR_WORKSPACE
    assert dcall(w2_s=None) == MOE_ERR_INVALID_ARG
    assert dcall(sw2_s=None) == MOE_ERR_INVALID_ARG
    assert dcall(n=-1) == MOE_ERR_INVALID_ARG
    assert dcall(H=7000) == MOE_ERR_UNSUPPORTED
    assert dcall(rows=0, n=0, ws=None, ws_bytes=0) == MOE_OK
    d = L.moe_dequantize_fp8
    assert d(FAKE, FAKE, 4, 200, FAKE, None) == MOE_ERR_UNSUPPORTED        # cols % 128
    assert d(FAKE, FAKE, 1 << 31, 128, FAKE, None) == MOE_ERR_UNSUPPORTED  # rows * cols / 8 >= 2^31
    assert d(FAKE, None, 4, 128, FAKE, None) == MOE_ERR_INVALID_ARG
    assert d(FAKE, FAKE, 4, 128, FAKE + 8, None) == MOE_ERR_INVALID_ARG    # misaligned output
    assert d(FAKE, FAKE, -1, 128, FAKE, None) == MOE_ERR_INVALID_ARG
    assert d(None, None, 0, 128, None, None) == MOE_OK
    # the fp8 gate/up keeps a bf16 copy of its activations after the schedule
    gu = moe.moe_workspace_bytes(moe.MOE_OP_EXPERT_GEMM, rows, H, I, E, 1, MOE_FP8_E4M3)
    assert gu == moe.moe_workspace_bytes(moe.MOE_OP_EXPERT_GEMM, rows, H, I, E, 1, MOE_BF16) + rows * H * 2
    e = L.moe_expert_gate_up
    assert e(FAKE, FAKE, MOE_FP8_E4M3, FAKE, E, rows, H, I, FAKE, FAKE, FAKE, FAKE, gu - 1, None) == MOE_ERR_WORKSPACE
    assert moe.moe_workspace_bytes(moe.MOE_OP_GROUPED_FFN, rows, H, I, E, 1, MOE_FP8_E4M3) == gu + rows * I * 2


def test_backward_validation_and_workspace(L):
    ws = moe.moe_workspace_bytes(moe.MOE_OP_EXPERT_DGRAD, 65536, 0, 0, 256, 0, 0)
    # prefix [E+1] + one entry per 128-row tile (rows / 128 + E) + 8 counters, int32, 256-byte rounded
    assert ws == ((257 + 512 + 256 + 8) * 4 + 255) // 256 * 256
    f = L.moe_combine_backward
    assert f(FAKE, MOE_BF16, 4, 256, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == MOE_ERR_INVALID_ARG
    assert f(FAKE, MOE_FP8_E4M3, 4, 256, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None) == MOE_ERR_UNSUPPORTED
    assert f(FAKE, MOE_BF16, 4, 100, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None) == MOE_ERR_UNSUPPORTED
    assert f(FAKE, MOE_BF16, 4, 256, 2, FAKE, None, FAKE, FAKE, FAKE, None) == MOE_ERR_INVALID_ARG
    assert f(None, MOE_BF16, 0, 256, 2, None, None, None, None, None, None) == MOE_OK
    f = L.moe_expert_gate_up_preact
    gws = moe.moe_workspace_bytes(moe.MOE_OP_EXPERT_GEMM, 1024, 256, 128, 8, 1, MOE_BF16)
    assert f(FAKE, MOE_F32, 64, FAKE, 2, FAKE, 8, 128, 256, 128, FAKE, FAKE, FAKE, gws, None) == MOE_ERR_UNSUPPORTED
    assert f(FAKE, MOE_BF16, 64, FAKE, 2, FAKE, 8, 128, 200, 128, FAKE, FAKE, FAKE, gws, None) == MOE_ERR_UNSUPPORTED
    assert f(FAKE, MOE_BF16, 64, FAKE, 2, FAKE, 8, 128, 256, 128, FAKE, FAKE, FAKE, 0, None) == MOE_ERR_WORKSPACE
    assert f(FAKE, MOE_BF16, 64, FAKE, 0, FAKE, 8, 128, 256, 128, FAKE, FAKE, FAKE, gws, None) == MOE_ERR_INVALID_ARG
    assert f(None, MOE_BF16, 0, None, 1, FAKE, 8, 0, 256, 128, None, None, None, 0, None) == MOE_OK
    f = L.moe_swiglu_backward
    assert f(FAKE, FAKE, 4, 12, FAKE, None, None) == MOE_ERR_UNSUPPORTED
    assert f(FAKE, None, 4, 16, FAKE, None, None) == MOE_ERR_INVALID_ARG
    assert f(None, None, 0, 16, None, None, None) == MOE_OK
    f = L.moe_expert_dgrad
    dws = moe.moe_workspace_bytes(moe.MOE_OP_EXPERT_DGRAD, 1024, 0, 0, 8, 0, 0)
    assert f(FAKE, FAKE, 8, 1024, 100, 256, FAKE, FAKE, FAKE, dws, None) == MOE_ERR_UNSUPPORTED   # K % 32
    assert f(FAKE, FAKE, 8, 1024, 128, 200, FAKE, FAKE, FAKE, dws, None) == MOE_ERR_UNSUPPORTED   # N % 128
    assert f(FAKE, FAKE, 8, 1024, 128, 256, FAKE, FAKE, FAKE, dws - 1, None) == MOE_ERR_WORKSPACE
    assert f(FAKE, FAKE, 0, 1024, 128, 256, FAKE, FAKE, FAKE, dws, None) == MOE_ERR_INVALID_ARG
    assert f(FAKE, FAKE, 8, 1024, 128, 256, None, FAKE, FAKE, dws, None) == MOE_ERR_INVALID_ARG
    assert f(None, FAKE, 8, 0, 128, 256, None, None, None, 0, None) == MOE_OK
    f = L.moe_expert_wgrad
    assert f(FAKE, 200, FAKE, 256, None, 1, 0, FAKE, 8, 64, FAKE, MOE_F32, None) == MOE_ERR_UNSUPPORTED
    assert f(FAKE, 256, FAKE, 256, None, 1, 0, FAKE, 8, 64, FAKE, MOE_FP8_E4M3, None) == MOE_ERR_UNSUPPORTED
    assert f(FAKE, 256, FAKE, 256, FAKE, 0, 64, FAKE, 8, 64, FAKE, MOE_F32, None) == MOE_ERR_INVALID_ARG
    assert f(FAKE, 256, FAKE, 256, None, 1, 0, FAKE, 8, 64, None, MOE_F32, None) == MOE_ERR_INVALID_ARG
    assert f(FAKE, 256, FAKE, 256, None, 1, 0, None, 8, 64, FAKE, MOE_F32, None) == MOE_ERR_INVALID_ARG
    f = L.moe_router_backward
    assert f(FAKE, FAKE, 4, 2, FAKE, FAKE, 8, 8, FAKE, MOE_FP8_E4M3, 256, FAKE, FAKE, MOE_F32, None) == \
        MOE_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, 4, 2, FAKE, None, 8, 8, FAKE, MOE_BF16, 256, FAKE, FAKE, MOE_F32, None) == MOE_ERR_INVALID_ARG
    assert f(FAKE, FAKE, 4, 2, FAKE, FAKE, 8, 8, FAKE, MOE_BF16, 100, FAKE, FAKE, MOE_F32, None) == \
        MOE_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, 4, 2, None, FAKE, 8, 8, FAKE, MOE_BF16, 256, FAKE, FAKE, MOE_F32, None) == MOE_ERR_INVALID_ARG


def test_router_input_grad_validation(L):
    f = L.moe_router_input_grad
    ok = (FAKE, MOE_BF16, 8, 16, 256, 4, FAKE, FAKE, None, FAKE, MOE_BF16, None)
    assert f(*ok[:1], MOE_BF16, 0, 16, 256, 4, None, None, None, None, MOE_BF16, None) == MOE_OK   # N = 0
    assert f(FAKE, MOE_BF16, 8, 16, 256, 17, FAKE, FAKE, None, FAKE, MOE_BF16, None) == MOE_ERR_INVALID_ARG  # k > E
    assert f(FAKE, MOE_BF16, -1, 16, 256, 4, FAKE, FAKE, None, FAKE, MOE_BF16, None) == MOE_ERR_INVALID_ARG
    assert f(FAKE, MOE_FP8_E4M3, 8, 16, 256, 4, FAKE, FAKE, None, FAKE, MOE_BF16, None) == MOE_ERR_UNSUPPORTED
    assert f(FAKE, MOE_BF16, 8, 16, 260, 4, FAKE, FAKE, None, FAKE, MOE_BF16, None) == MOE_ERR_UNSUPPORTED  # H % 8
    assert f(FAKE, MOE_BF16, 8, 16, 256, 33, FAKE, FAKE, None, FAKE, MOE_BF16, None) in (MOE_ERR_UNSUPPORTED,
                                                                                          MOE_ERR_INVALID_ARG)
    assert f(None, MOE_BF16, 8, 16, 256, 4, FAKE, FAKE, None, FAKE, MOE_BF16, None) == MOE_ERR_INVALID_ARG
    assert f(FAKE, MOE_BF16, 8, 16, 256, 4, None, FAKE, None, FAKE, MOE_BF16, None) == MOE_ERR_INVALID_ARG
    assert f(FAKE + 8, MOE_BF16, 8, 16, 256, 4, FAKE, FAKE, None, FAKE, MOE_BF16, None) == MOE_ERR_INVALID_ARG
    assert f(FAKE, MOE_BF16, 8, 16, 256, 4, FAKE, FAKE, FAKE + 8, FAKE, MOE_BF16, None) == MOE_ERR_INVALID_ARG
