// Internal launchers (one per kernel family); host code in moe_api.cpp validates the
// arguments before calling any of these.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

hipError_t launch_route(const float* z, int N, int E, int k, const float* bias, int n_group,
                        int topk_group, int32_t* topk_idx, float* topk_gate, hipStream_t s);

int layout_chunk_slots(long long nk);
int layout_num_chunks(long long nk);
hipError_t launch_dispatch_layout(const int32_t* topk_idx, int nk, int E, int32_t* n_e,
                                  int32_t* offsets, int32_t* send_pos, int32_t* src_slot,
                                  int32_t* counts, hipStream_t s);
// the device address of the current device's fixed layout scratch (MOE_LAYOUT_SCRATCH_BYTES)
hipError_t layout_scratch(int32_t** out);

hipError_t launch_permute_copy(const void* x, size_t row_bytes, int N, int k,
                               const int32_t* send_pos, void* out, hipStream_t s);
hipError_t launch_permute_fp8(const void* x, bool f32_in, long long rows, int H, int k,
                              const int32_t* send_pos, uint8_t* q, float* scale, hipStream_t s);

// router logits: parts of K the bf16 tile kernel uses (0: the plain fp32-FMA kernel),
// the workspace that many fp32 partial sums need, and the launch
int router_parts(int N, int H, int E, bool bf16);
size_t router_ws_bytes(int N, int H, int E, bool bf16);
hipError_t launch_router_logits(const void* x, bool bf16, int N, int H, const void* w_r, int E, float* z,
                                void* ws, hipStream_t s);

// rows_once: every row of eo is named by at most one slot (the layer's expert outputs), so
// its loads carry the non-temporal hint; false keeps them in the caches (rows re-read)
hipError_t launch_combine(const void* eo, bool eo_f32, int N, int H, int k, const int32_t* send_pos,
                          const float* gate, const void* shared, void* y, bool y_f32, hipStream_t s,
                          bool rows_once = true);
// read-mostly streaming probe: ratio in {1, 2, 4, 8, 9, 16}
hipError_t launch_stream_probe(const void* src, size_t n16, int ratio, void* dst, hipStream_t s);

// backward pass (backward.hip, grouped_gemm_bwd.hip)
hipError_t launch_combine_backward(const void* dy, bool f32, int N, int H, int k, const int32_t* send_pos,
                                   const float* gate, const void* eo, void* d_eo, float* d_gate, hipStream_t s);
hipError_t launch_swiglu_backward(const void* au, const void* dh, long long rows, int I, void* d_au, void* h,
                                  hipStream_t s);
hipError_t launch_router_backward(const float* gate, const float* d_gate, int N, int k, const int32_t* offsets,
                                  const int32_t* src_slot, int E, int rows, const void* x, bool x_f32, int H,
                                  float* dz, void* dw, bool dw_f32, hipStream_t s);
size_t bwd_dgrad_ws_bytes(int rows, int E);
hipError_t launch_expert_dgrad(const void* dC, const int32_t* offsets, int E, int rows, int K, int N, const void* w,
                               void* out, void* ws, hipStream_t s);
hipError_t launch_expert_wgrad(const void* a, const void* b, const int32_t* b_rows, int b_div, int b_nrows,
                               const int32_t* offsets, int E, int rows, int M, int N, void* dw, bool dw_f32,
                               hipStream_t s);
// the forward's tile schedule (prefix of m-tiles per segment, m-tile -> segment)
hipError_t launch_build_tiles(const int32_t* offsets, int E, int rows, int tile_rows, int cap, int32_t* prefix,
                              int32_t* tile_expert, int32_t* tile_counter, hipStream_t s);

size_t gemm_tile_cap(int rows, int E);
size_t gemm_schedule_bytes(int rows, int E);
// the fp8 gate/up's bf16 copy of its activations, kept after the schedule (rows x K)
size_t gemm_a8_bytes(int rows, int K);
hipError_t launch_grouped_gemm(int ct, bool b8, int mode, const void* a, const float* a_scale,
                               const void* b, const float* b_scale, void* out, bool out_f32,
                               const int32_t* offsets, int E, int rows, int K, int I, int n_out,
                               long long b_rows, void* sched, hipStream_t s,
                               const int32_t* a_rows = nullptr, int a_div = 1, int a_nrows = 0,
                               const void* shared_b = nullptr, int shared_rows = 0,
                               const int32_t* row_slot = nullptr, const float* row_gate = nullptr,
                               void* au = nullptr, const float* shared_b_scale = nullptr);
// bf16 values of e4m3 codes [rows, cols] with fp32 scales [rows, cols / 128] (code times the
// scale of its 128-column block, rounded to nearest even); rows * cols / 8 < 2^31
hipError_t launch_dequant_e4m3(const uint8_t* q, const float* scale, long long rows, int cols, void* out,
                               hipStream_t s);
// whether launch_grouped_gemm accepts a shared segment for these bf16 shapes
bool grouped_gemm_shared_supported(int mode, int K, int I, int n_out, long long b_rows, int a_nrows,
                                   bool gathered);

}  // namespace moe
