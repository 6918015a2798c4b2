// Host side of libmoe: argument validation, workspace sizing and kernel launches behind
// the C ABI declared in include/moe.h.  Every check runs before anything is enqueued, and
// no HIP call is made on an error path.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "moe.h"
#include "moe_launch.h"

namespace {

constexpr long long kMaxRowsPerLaunch = (1ll << 24);  // one 256-lane workgroup per row

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t dtype_bytes(int dt) {
  switch (dt) {
    case MOE_F32: return 4;
    case MOE_BF16: return 2;
    case MOE_FP8_E4M3: return 1;
    default: return 0;
  }
}

size_t round256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

size_t layout_ws(int N, int k, int E) {
  const long long nk = static_cast<long long>(N) * k;
  if (nk <= 0 || E <= 0) return 0;
  return round256(static_cast<size_t>(moe::layout_num_chunks(nk)) * E * sizeof(int32_t));
}

size_t h_bytes(int rows, int I, int a_dt) {
  return round256(static_cast<size_t>(rows) * I * (a_dt == MOE_F32 ? 4 : 2));
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Checks shared by the two expert GEMMs.
moe_status check_gemm(const int32_t* offsets, int E, int rows, int H, int I, void* ws,
                      size_t ws_bytes) {
  if (E < 1 || E > MOE_MAX_EXPERTS || rows < 0 || H <= 0 || I <= 0) return MOE_ERR_INVALID_ARG;
  if (offsets == nullptr) return MOE_ERR_INVALID_ARG;
  if (H % 128 != 0 || I % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows > 0 && (ws == nullptr || ws_bytes < moe::gemm_schedule_bytes(rows, E))) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_version(void) { return "0.1.0"; }

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

size_t moe_workspace_bytes(int op, int N, int H, int I, int E, int k, int a_dt) {
  if (N < 0 || E < 0) return 0;
  switch (op) {
    case MOE_OP_DISPATCH_LAYOUT:
      if (k < 1 || E < 1) return 0;
      return layout_ws(N, k, E);
    case MOE_OP_EXPERT_GEMM:
      if (E < 1 || N == 0) return 0;
      return moe::gemm_schedule_bytes(N, E) + (a_dt == MOE_FP8_E4M3 && H > 0 ? moe::gemm_a8_bytes(N, H) : 0);
    case MOE_OP_GROUPED_FFN:
      if (E < 1 || N == 0 || I <= 0 || H <= 0) return 0;
      return moe_workspace_bytes(MOE_OP_EXPERT_GEMM, N, H, I, E, k, a_dt) + h_bytes(N, I, a_dt);
    case MOE_OP_EXPERT_DGRAD:
      if (E < 1 || N == 0) return 0;
      return moe::bwd_dgrad_ws_bytes(N, E);
    case MOE_OP_ROUTER:
      if (E < 1 || N == 0 || H <= 0) return 0;
      return moe::router_ws_bytes(N, H, E, a_dt == MOE_BF16);
    default:
      return 0;
  }
}

moe_status moe_router_logits(const void* x, moe_dtype x_dt, int N, int H, const void* w_r, int E, float* z,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  if (N < 0 || H <= 0 || E < 1) return MOE_ERR_INVALID_ARG;
  if (x_dt != MOE_F32 && x_dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  if (N == 0) return MOE_OK;
  if (x == nullptr || w_r == nullptr || z == nullptr) return MOE_ERR_INVALID_ARG;
  const size_t need = moe::router_ws_bytes(N, H, E, x_dt == MOE_BF16);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(w_r) || !aligned16(z) || (need > 0 && !aligned16(ws))) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_router_logits(x, x_dt == MOE_BF16, N, H, w_r, E, z, ws, stream));
}

moe_status moe_route(const float* z, int N, int E, int k, const float* bias, int n_group,
                     int topk_group, int32_t* topk_idx, float* topk_gate, hipStream_t stream) {
  if (N < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if (n_group < 0 || topk_group < 0) return MOE_ERR_INVALID_ARG;
  if (n_group > 0) {
    if (n_group > MOE_MAX_GROUPS) return MOE_ERR_UNSUPPORTED;
    if (E % n_group != 0 || topk_group < 1 || topk_group > n_group) return MOE_ERR_INVALID_ARG;
    if (static_cast<long long>(topk_group) * (E / n_group) < k) return MOE_ERR_INVALID_ARG;
  } else if (topk_group != 0) {
    return MOE_ERR_INVALID_ARG;
  }
  if (static_cast<long long>(N) * k >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  if (N == 0) return MOE_OK;
  if (z == nullptr || topk_idx == nullptr || topk_gate == nullptr) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_route(z, N, E, k, bias, n_group, topk_group, topk_idx, topk_gate, stream));
}

moe_status moe_dispatch_layout(const int32_t* topk_idx, int N, int k, int E, int32_t* n_e,
                               int32_t* offsets, int32_t* send_pos, int32_t* src_slot, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  if (N < 0 || k < 1 || E < 1) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if (static_cast<long long>(N) * k >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  if (N == 0) return MOE_OK;
  if (topk_idx == nullptr || n_e == nullptr || offsets == nullptr || send_pos == nullptr ||
      src_slot == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (ws == nullptr || ws_bytes < layout_ws(N, k, E)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_dispatch_layout(topk_idx, N * k, E, n_e, offsets, send_pos, src_slot,
                                                reinterpret_cast<int32_t*>(ws), stream));
}

moe_status moe_dispatch_layout_noalloc(const int32_t* topk_idx, int N, int k, int E, int32_t* n_e,
                                       int32_t* offsets, int32_t* send_pos, int32_t* src_slot,
                                       hipStream_t stream) {
  if (N < 0 || k < 1 || E < 1) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if (static_cast<long long>(N) * k >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  if (N == 0) return MOE_OK;
  if (topk_idx == nullptr || n_e == nullptr || offsets == nullptr || send_pos == nullptr ||
      src_slot == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (layout_ws(N, k, E) > MOE_LAYOUT_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  int32_t* counts = nullptr;
  if (moe::layout_scratch(&counts) != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_dispatch_layout(topk_idx, N * k, E, n_e, offsets, send_pos, src_slot, counts,
                                                stream));
}

moe_status moe_permute(const void* x, moe_dtype x_dt, int N, int H, int k,
                       const int32_t* send_pos, void* x_perm, moe_dtype perm_dt, float* perm_scale,
                       hipStream_t stream) {
  if (N < 0 || H <= 0 || k < 1) return MOE_ERR_INVALID_ARG;
  if (x_dt != MOE_F32 && x_dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (perm_dt != x_dt && perm_dt != MOE_FP8_E4M3) return MOE_ERR_UNSUPPORTED;
  if (k > MOE_MAX_TOPK || N >= kMaxRowsPerLaunch) return MOE_ERR_UNSUPPORTED;
  if (static_cast<long long>(N) * k >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  const size_t row_bytes = static_cast<size_t>(H) * dtype_bytes(x_dt);
  if (row_bytes % 16 != 0) return MOE_ERR_UNSUPPORTED;
  if (perm_dt == MOE_FP8_E4M3 && H % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (N == 0) return MOE_OK;
  if (x == nullptr || send_pos == nullptr || x_perm == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_INVALID_ARG;
  if (perm_dt == MOE_FP8_E4M3) {
    if (perm_scale == nullptr) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_permute_fp8(x, x_dt == MOE_F32, N, H, k, send_pos,
                                              reinterpret_cast<uint8_t*>(x_perm), perm_scale, stream));
  }
  return hip_status(moe::launch_permute_copy(x, row_bytes, N, k, send_pos, x_perm, stream));
}

moe_status moe_quantize_fp8(const void* x, moe_dtype x_dt, int64_t rows, int cols, uint8_t* q,
                            float* scale, hipStream_t stream) {
  if (rows < 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
  if (x_dt != MOE_F32 && x_dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (cols % 128 != 0 || rows >= kMaxRowsPerLaunch) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (x == nullptr || q == nullptr || scale == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(q)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_permute_fp8(x, x_dt == MOE_F32, rows, cols, 1, nullptr, q, scale, stream));
}

moe_status moe_expert_gate_up(const void* a, const float* a_scale, moe_dtype a_dt,
                              const int32_t* offsets, int E, int rows, int H, int I,
                              const void* w13, const float* w13_scale, void* h, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  if (a_dt != MOE_F32 && a_dt != MOE_BF16 && a_dt != MOE_FP8_E4M3) return MOE_ERR_UNSUPPORTED;
  const moe_status st = check_gemm(offsets, E, rows, H, I, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if (rows == 0) return MOE_OK;
  if (a == nullptr || w13 == nullptr || h == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(w13)) return MOE_ERR_INVALID_ARG;
  if (a_dt == MOE_FP8_E4M3 && (a_scale == nullptr || w13_scale == nullptr)) return MOE_ERR_INVALID_ARG;
  // (fp8: room for the bf16 copy of a after the schedule)
  if (a_dt == MOE_FP8_E4M3 && ws_bytes < moe::gemm_schedule_bytes(rows, E) + moe::gemm_a8_bytes(rows, H))
    return MOE_ERR_WORKSPACE;
  const int ct = a_dt == MOE_F32 ? 0 : (a_dt == MOE_BF16 ? 1 : 2);
  return hip_status(moe::launch_grouped_gemm(ct, false, 0, a, a_scale, w13, w13_scale, h,
                                             a_dt == MOE_F32, offsets, E, rows, H, I, I,
                                             2ll * I, ws, stream));
}

moe_status moe_expert_gate_up_gathered(const void* x, moe_dtype x_dt, int N, const int32_t* src_slot,
                                       int k, const int32_t* offsets, int E, int rows, int H, int I,
                                       const void* w13, void* h, void* ws, size_t ws_bytes,
                                       hipStream_t stream) {
  if (x_dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  const moe_status st = check_gemm(offsets, E, rows, H, I, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if (N < 0 || k < 1 || k > MOE_MAX_TOPK) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (N == 0 || x == nullptr || src_slot == nullptr || w13 == nullptr || h == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w13)) return MOE_ERR_INVALID_ARG;
  if (static_cast<long long>(N) * H * 2 >= (1LL << 32)) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_grouped_gemm(1, false, 0, x, nullptr, w13, nullptr, h, false, offsets,
                                             E, rows, H, I, I, 2ll * I, ws, stream, src_slot, k, N));
}

moe_status moe_expert_gate_up_gathered_shared(const void* x, moe_dtype x_dt, int N, const int32_t* src_slot,
                                              int k, const int32_t* offsets, int E, int rows, int H, int I,
                                              const void* w13, const void* shared_w13, void* h, void* au,
                                              void* ws, size_t ws_bytes, hipStream_t stream) {
  if (x_dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (E < 1 || rows < 0 || N < 0 || H <= 0 || I <= 0 || offsets == nullptr) return MOE_ERR_INVALID_ARG;
  if (k < 1 || k > MOE_MAX_TOPK) return MOE_ERR_INVALID_ARG;
  if (E >= MOE_MAX_EXPERTS || H % 128 != 0 || I % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (static_cast<long long>(rows) + N >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if (rows + N == 0) return MOE_OK;
  if (ws == nullptr || ws_bytes < moe::gemm_schedule_bytes(rows + N, E + 1)) return MOE_ERR_WORKSPACE;
  if (x == nullptr || shared_w13 == nullptr || h == nullptr || (rows > 0 && (w13 == nullptr || src_slot == nullptr)))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(shared_w13) || (w13 != nullptr && !aligned16(w13))) return MOE_ERR_INVALID_ARG;
  if (au != nullptr && !aligned16(au)) return MOE_ERR_INVALID_ARG;
  if (static_cast<long long>(N) * H * 2 >= (1LL << 32)) return MOE_ERR_UNSUPPORTED;
  if (!moe::grouped_gemm_shared_supported(0, H, I, I, 2ll * I, N, true)) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_grouped_gemm(1, false, 0, x, nullptr, w13, nullptr, h, false, offsets,
                                             E, rows, H, I, I, 2ll * I, ws, stream, src_slot, k, N,
                                             shared_w13, N, nullptr, nullptr, au));
}

moe_status moe_expert_gate_up_gathered_shared_e4m3(const void* x, int N, const int32_t* src_slot, int k,
                                                   const int32_t* offsets, int E, int rows, int H, int I,
                                                   const uint8_t* w13, const float* w13_scale,
                                                   const uint8_t* shared_w13, const float* shared_w13_scale,
                                                   void* h, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (E < 1 || rows < 0 || N < 0 || H <= 0 || I <= 0 || offsets == nullptr) return MOE_ERR_INVALID_ARG;
  if (k < 1 || k > MOE_MAX_TOPK) return MOE_ERR_INVALID_ARG;
  if (E >= MOE_MAX_EXPERTS || H % 128 != 0 || I % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (static_cast<long long>(rows) + N >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if (rows + N == 0) return MOE_OK;
  if (ws == nullptr || ws_bytes < moe::gemm_schedule_bytes(rows + N, E + 1)) return MOE_ERR_WORKSPACE;
  if (x == nullptr || shared_w13 == nullptr || shared_w13_scale == nullptr || h == nullptr ||
      (rows > 0 && (w13 == nullptr || w13_scale == nullptr || src_slot == nullptr)))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(shared_w13) || (w13 != nullptr && !aligned16(w13))) return MOE_ERR_INVALID_ARG;
  if (static_cast<long long>(N) * H * 2 >= (1LL << 32)) return MOE_ERR_UNSUPPORTED;
  if (2LL * I * H >= (1LL << 32)) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_grouped_gemm(1, true, 0, x, nullptr, w13, w13_scale, h, false, offsets, E, rows, H,
                                             I, I, 2ll * I, ws, stream, src_slot, k, N, shared_w13, N, nullptr,
                                             nullptr, nullptr, shared_w13_scale));
}

moe_status moe_expert_down_shared_e4m3(const void* h, const int32_t* offsets, int E, int rows, int n_shared,
                                       int I, int H, const uint8_t* w2, const float* w2_scale,
                                       const uint8_t* shared_w2, const float* shared_w2_scale, void* out,
                                       void* ws, size_t ws_bytes, hipStream_t stream) {
  if (E < 1 || rows < 0 || n_shared < 0 || H <= 0 || I <= 0 || offsets == nullptr) return MOE_ERR_INVALID_ARG;
  if (E >= MOE_MAX_EXPERTS || H % 128 != 0 || I % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (static_cast<long long>(rows) + n_shared >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if (rows + n_shared == 0) return MOE_OK;
  if (ws == nullptr || ws_bytes < moe::gemm_schedule_bytes(rows + n_shared, E + 1)) return MOE_ERR_WORKSPACE;
  if (h == nullptr || out == nullptr || (n_shared > 0 && (shared_w2 == nullptr || shared_w2_scale == nullptr)) ||
      (rows > 0 && (w2 == nullptr || w2_scale == nullptr)))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(h) || (w2 != nullptr && !aligned16(w2)) || (shared_w2 != nullptr && !aligned16(shared_w2)))
    return MOE_ERR_INVALID_ARG;
  if (static_cast<long long>(H) * I >= (1LL << 32)) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_grouped_gemm(1, true, 1, h, nullptr, w2, w2_scale, out, false, offsets, E, rows, I,
                                             I, H, static_cast<long long>(H), ws, stream, nullptr, 1, 0, shared_w2,
                                             n_shared, nullptr, nullptr, nullptr, shared_w2_scale));
}

moe_status moe_dequantize_fp8(const uint8_t* q, const float* scale, int64_t rows, int cols, void* out,
                              hipStream_t stream) {
  if (rows < 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
  if (cols % 128 != 0 || rows * cols / 8 >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (q == nullptr || scale == nullptr || out == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_dequant_e4m3(q, scale, rows, cols, out, stream));
}

moe_status moe_expert_down_shared(const void* h, moe_dtype h_dt, const int32_t* offsets, int E, int rows,
                                  int n_shared, int I, int H, const void* w2, const void* shared_w2,
                                  const int32_t* src_slot, const float* topk_gate, void* out,
                                  moe_dtype out_dt, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (h_dt != MOE_BF16 || out_dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (E < 1 || rows < 0 || n_shared < 0 || H <= 0 || I <= 0 || offsets == nullptr) return MOE_ERR_INVALID_ARG;
  if (E >= MOE_MAX_EXPERTS || H % 128 != 0 || I % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (static_cast<long long>(rows) + n_shared >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if (rows + n_shared == 0) return MOE_OK;
  if (ws == nullptr || ws_bytes < moe::gemm_schedule_bytes(rows + n_shared, E + 1)) return MOE_ERR_WORKSPACE;
  if (h == nullptr || out == nullptr || (n_shared > 0 && shared_w2 == nullptr) || (rows > 0 && w2 == nullptr))
    return MOE_ERR_INVALID_ARG;
  if ((src_slot == nullptr) != (topk_gate == nullptr)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(h) || (w2 != nullptr && !aligned16(w2)) || (shared_w2 != nullptr && !aligned16(shared_w2)))
    return MOE_ERR_INVALID_ARG;
  if (!moe::grouped_gemm_shared_supported(1, I, I, H, static_cast<long long>(H), 0, false))
    return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_grouped_gemm(1, false, 1, h, nullptr, w2, nullptr, out, false, offsets, E,
                                             rows, I, I, H, static_cast<long long>(H), ws, stream, nullptr, 1,
                                             0, shared_w2, n_shared, src_slot, topk_gate));
}

moe_status moe_expert_down(const void* h, moe_dtype h_dt, const int32_t* offsets, int E, int rows,
                           int I, int H, const void* w2, moe_dtype w2_dt, const float* w2_scale,
                           void* out, moe_dtype out_dt, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  if (h_dt != MOE_F32 && h_dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (h_dt == MOE_F32 && (w2_dt != MOE_F32 || out_dt != MOE_F32)) return MOE_ERR_UNSUPPORTED;
  if (h_dt == MOE_BF16 && ((w2_dt != MOE_BF16 && w2_dt != MOE_FP8_E4M3) || out_dt != MOE_BF16))
    return MOE_ERR_UNSUPPORTED;
  const moe_status st = check_gemm(offsets, E, rows, H, I, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if (rows == 0) return MOE_OK;
  if (h == nullptr || w2 == nullptr || out == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(w2)) return MOE_ERR_INVALID_ARG;
  if (w2_dt == MOE_FP8_E4M3 && w2_scale == nullptr) return MOE_ERR_INVALID_ARG;
  const int ct = h_dt == MOE_F32 ? 0 : 1;
  return hip_status(moe::launch_grouped_gemm(ct, w2_dt == MOE_FP8_E4M3, 1, h, nullptr, w2, w2_scale,
                                             out, out_dt == MOE_F32, offsets, E, rows, I, I, H,
                                             static_cast<long long>(H), ws, stream));
}

moe_status moe_grouped_ffn(const void* a, const float* a_scale, moe_dtype a_dt,
                           const int32_t* offsets, int E, int rows, int H, int I, const void* w13,
                           const float* w13_scale, const void* w2, const float* w2_scale, void* out,
                           moe_dtype out_dt, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (a_dt != MOE_F32 && a_dt != MOE_BF16 && a_dt != MOE_FP8_E4M3) return MOE_ERR_UNSUPPORTED;
  if (out_dt != (a_dt == MOE_F32 ? MOE_F32 : MOE_BF16)) return MOE_ERR_UNSUPPORTED;
  const moe_status st = check_gemm(offsets, E, rows, H, I, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if (rows == 0) return MOE_OK;
  if (a == nullptr || w13 == nullptr || w2 == nullptr || out == nullptr) return MOE_ERR_INVALID_ARG;
  if (a_dt == MOE_FP8_E4M3 && (a_scale == nullptr || w13_scale == nullptr || w2_scale == nullptr))
    return MOE_ERR_INVALID_ARG;
  if (ws_bytes < moe_workspace_bytes(MOE_OP_GROUPED_FFN, rows, H, I, E, 1, a_dt)) return MOE_ERR_WORKSPACE;
  const size_t sched = moe::gemm_schedule_bytes(rows, E);
  const size_t gu = moe_workspace_bytes(MOE_OP_EXPERT_GEMM, rows, H, I, E, 1, a_dt);   // (fp8: + bf16 a)
  void* hbuf = static_cast<uint8_t*>(ws) + gu;
  const moe_dtype h_dt = a_dt == MOE_F32 ? MOE_F32 : MOE_BF16;
  moe_status s = moe_expert_gate_up(a, a_scale, a_dt, offsets, E, rows, H, I, w13, w13_scale, hbuf,
                                    ws, gu, stream);
  if (s != MOE_OK) return s;
  return moe_expert_down(hbuf, h_dt, offsets, E, rows, I, H, w2, a_dt, w2_scale, out, out_dt, ws,
                         sched, stream);
}

moe_status moe_combine(const void* expert_out, moe_dtype eo_dt, int N, int H, int k,
                       const int32_t* send_pos, const float* topk_gate, const void* shared_out,
                       void* y, moe_dtype y_dt, hipStream_t stream) {
  if (N < 0 || H <= 0 || k < 1) return MOE_ERR_INVALID_ARG;
  if ((eo_dt != MOE_F32 && eo_dt != MOE_BF16) || (y_dt != MOE_F32 && y_dt != MOE_BF16))
    return MOE_ERR_UNSUPPORTED;
  if (k > MOE_MAX_TOPK || N >= kMaxRowsPerLaunch || H % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (static_cast<long long>(N) * k >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  if (N == 0) return MOE_OK;
  if (expert_out == nullptr || send_pos == nullptr || y == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned16(expert_out) || !aligned16(y) || (shared_out != nullptr && !aligned16(shared_out)))
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_combine(expert_out, eo_dt == MOE_F32, N, H, k, send_pos, topk_gate,
                                        shared_out, y, y_dt == MOE_F32, stream));
}

moe_status moe_router_input_grad(const void* w_r, moe_dtype w_dt, int N, int E, int H, int k,
                                 const int32_t* topk_idx, const float* dz, const void* rest, void* dx,
                                 moe_dtype dx_dt, hipStream_t stream) {
  if (N < 0 || E < 1 || H <= 0 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if ((w_dt != MOE_F32 && w_dt != MOE_BF16) || (dx_dt != MOE_F32 && dx_dt != MOE_BF16)) return MOE_ERR_UNSUPPORTED;
  if (k > MOE_MAX_TOPK || E > MOE_MAX_EXPERTS || N >= kMaxRowsPerLaunch || H % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (static_cast<long long>(N) * k >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  if (N == 0) return MOE_OK;
  if (w_r == nullptr || topk_idx == nullptr || dz == nullptr || dx == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned16(w_r) || !aligned16(dx) || (rest != nullptr && !aligned16(rest))) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_combine(w_r, w_dt == MOE_F32, N, H, k, topk_idx, dz, rest, dx, dx_dt == MOE_F32,
                                        stream, /*rows_once=*/false));
}

moe_status moe_stream_probe(const void* src, size_t n16, int ratio, void* dst, hipStream_t stream) {
  if (ratio != 1 && ratio != 2 && ratio != 4 && ratio != 8 && ratio != 9 && ratio != 16) return MOE_ERR_UNSUPPORTED;
  if (n16 == 0) return MOE_OK;
  if (src == nullptr || dst == nullptr || !aligned16(src) || !aligned16(dst)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_stream_probe(src, n16, ratio, dst, stream));
}

// ---- backward pass

moe_status moe_combine_backward(const void* dy, moe_dtype dt, int N, int H, int k, const int32_t* send_pos,
                                const float* topk_gate, const void* expert_out, void* d_expert_out, float* d_gate,
                                hipStream_t stream) {
  if (N < 0 || H <= 0 || k < 1) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (k > MOE_MAX_TOPK || static_cast<long long>(N) * k >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  if ((static_cast<size_t>(H) * dtype_bytes(dt)) % 16 != 0) return MOE_ERR_UNSUPPORTED;
  if (N == 0) return MOE_OK;
  if (dy == nullptr || send_pos == nullptr || topk_gate == nullptr || expert_out == nullptr ||
      d_expert_out == nullptr || d_gate == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(dy) || !aligned16(expert_out) || !aligned16(d_expert_out)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_combine_backward(dy, dt == MOE_F32, N, H, k, send_pos, topk_gate, expert_out,
                                                 d_expert_out, d_gate, stream));
}

moe_status moe_expert_gate_up_preact(const void* x, moe_dtype x_dt, int N, const int32_t* src_slot, int k,
                                     const int32_t* offsets, int E, int rows, int H, int I, const void* w13, void* au,
                                     void* ws, size_t ws_bytes, hipStream_t stream) {
  if (x_dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  const moe_status st = check_gemm(offsets, E, rows, H, I, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if (src_slot != nullptr && (N < 1 || k < 1 || k > MOE_MAX_TOPK)) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (x == nullptr || w13 == nullptr || au == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w13) || !aligned16(au)) return MOE_ERR_INVALID_ARG;
  if (src_slot != nullptr && static_cast<long long>(N) * H * 2 >= (1LL << 32)) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_grouped_gemm(1, false, 1, x, nullptr, w13, nullptr, au, false, offsets, E, rows, H,
                                             I, 2 * I, 2ll * I, ws, stream, src_slot, src_slot ? k : 1,
                                             src_slot ? N : 0));
}

moe_status moe_swiglu_backward(const void* au, const void* dh, int rows, int I, void* d_au, void* h,
                               hipStream_t stream) {
  if (rows < 0 || I <= 0) return MOE_ERR_INVALID_ARG;
  if (I % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (au == nullptr || dh == nullptr || d_au == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned16(au) || !aligned16(dh) || !aligned16(d_au) || (h != nullptr && !aligned16(h)))
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_swiglu_backward(au, dh, rows, I, d_au, h, stream));
}

moe_status moe_expert_dgrad(const void* dC, const int32_t* offsets, int E, int rows, int K, int N, const void* w,
                            void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (E < 1 || rows < 0 || K <= 0 || N <= 0 || offsets == nullptr) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS || K % 32 != 0 || N % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (ws == nullptr || ws_bytes < moe::bwd_dgrad_ws_bytes(rows, E)) return MOE_ERR_WORKSPACE;
  if (dC == nullptr || w == nullptr || out == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned16(dC) || !aligned16(w) || !aligned16(out)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_expert_dgrad(dC, offsets, E, rows, K, N, w, out, ws, stream));
}

moe_status moe_expert_wgrad(const void* a, int M, const void* b, int N, const int32_t* b_rows, int b_div,
                            int b_nrows, const int32_t* offsets, int E, int rows, void* dw, moe_dtype dw_dt,
                            hipStream_t stream) {
  if (E < 1 || rows < 0 || M <= 0 || N <= 0 || offsets == nullptr) return MOE_ERR_INVALID_ARG;
  if (dw_dt != MOE_F32 && dw_dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (E > MOE_MAX_EXPERTS || M % 128 != 0 || N % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (b_rows != nullptr && (b_div < 1 || b_nrows < 1)) return MOE_ERR_INVALID_ARG;
  if (dw == nullptr || (rows > 0 && (a == nullptr || b == nullptr))) return MOE_ERR_INVALID_ARG;
  if (!aligned16(dw) || (rows > 0 && (!aligned16(a) || !aligned16(b)))) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_expert_wgrad(a, b, b_rows, b_div, b_nrows, offsets, E, rows, M, N, dw,
                                             dw_dt == MOE_F32, stream));
}

moe_status moe_router_backward(const float* topk_gate, const float* d_gate, int N, int k, const int32_t* offsets,
                               const int32_t* src_slot, int E, int rows, const void* x, moe_dtype x_dt, int H,
                               float* dz, void* dw_r, moe_dtype dw_dt, hipStream_t stream) {
  if (N < 0 || k < 1 || E < 1 || rows < 0 || H <= 0) return MOE_ERR_INVALID_ARG;
  if (x_dt != MOE_F32 && x_dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (dw_dt != MOE_F32 && dw_dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || static_cast<long long>(N) * k >= (1ll << 31))
    return MOE_ERR_UNSUPPORTED;
  if ((static_cast<size_t>(H) * dtype_bytes(x_dt)) % 16 != 0) return MOE_ERR_UNSUPPORTED;
  if (offsets == nullptr || dw_r == nullptr) return MOE_ERR_INVALID_ARG;
  if (N > 0 && (topk_gate == nullptr || d_gate == nullptr || dz == nullptr || x == nullptr)) return MOE_ERR_INVALID_ARG;
  if (rows > 0 && (src_slot == nullptr || N == 0)) return MOE_ERR_INVALID_ARG;
  if (x != nullptr && !aligned16(x)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_router_backward(topk_gate, d_gate, N, k, offsets, src_slot, E, rows, x,
                                                x_dt == MOE_F32, H, dz, dw_r, dw_dt == MOE_F32, stream));
}

}  // extern "C"
