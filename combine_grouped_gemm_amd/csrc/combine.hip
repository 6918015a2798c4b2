// Combine (unpermute + gate-weighted sum back to token order):
//   y_t = sum_{j<k} g_{t,j} * expert_out[send_pos[t*k+j]]  (+ shared_out_t)
// ("EP / DeepEP explanation" page, sections 2 and 3; "DeepEP" page, section 7: the sum is
// kept in a wider type than the payload).
//
// Each workgroup takes one token and one span of its columns (the row is split into
// `spans` spans, so that small batches still fill the GPU); each lane owns 8 consecutive
// columns, gathers the k expert rows with 16-byte loads (up to 8 rows' loads issued before
// the sum), accumulates in fp32 in the order j = 0..k-1 then the shared row, rounds once
// and writes 16 bytes (bf16) or 32 bytes (fp32).  Gates and send positions are uniform
// across the workgroup, whose size (128 or 256 lanes) divides the row's 8-column groups
// when it can, so that no pass over the row leaves lanes idle.
#include <type_traits>

#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

constexpr int kCombMaxThreads = 256;

template <bool kEoF32>
__device__ __forceinline__ void load8(const void* base, size_t row, int H, int c, float (&v)[8]) {
  if (kEoF32) {
    const float4* p = reinterpret_cast<const float4*>(base) + (row * H) / 4 + 2 * c;
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 a = reinterpret_cast<const uint4*>(base)[(row * H) / 8 + c];
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(static_cast<uint16_t>(w[i] & 0xFFFFu));
      v[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(w[i] >> 16));
    }
  }
}

template <int U, bool kEoF32, bool kGated>
__device__ __forceinline__ void gather_sum(const void* eo, const int32_t* sp, const float* g, int H, int c,
                                           float (&acc)[8]) {
  float v[U][8];
  int r[U];
#pragma unroll
  for (int u = 0; u < U; ++u) r[u] = sp[u];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (r[u] >= 0) {
      load8<kEoF32>(eo, static_cast<size_t>(r[u]), H, c, v[u]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[u][i] = 0.0f;
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float gu = kGated ? g[u] : 1.0f;   // (fma with 1 is the plain sum)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(gu, v[u][i], acc[i]);
  }
}

template <bool kEoF32, bool kYF32, bool kGated>
__global__ __launch_bounds__(kCombMaxThreads) void combine_kernel(
    const void* __restrict__ eo, int H, int k, const int32_t* __restrict__ send_pos,
    const float* __restrict__ gate, const void* __restrict__ shared, void* __restrict__ y, int spans) {
  const int t = blockIdx.x / spans;
  const int span = blockIdx.x % spans;
  const int32_t* sp = send_pos + static_cast<size_t>(t) * k;
  const float* g = kGated ? gate + static_cast<size_t>(t) * k : nullptr;
  const int groups8 = H / 8;
  const int per_span = (groups8 + spans - 1) / spans;
  const int c_end = (span + 1) * per_span < groups8 ? (span + 1) * per_span : groups8;
  for (int c = span * per_span + threadIdx.x; c < c_end; c += blockDim.x) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int j = 0;
    for (; j + 8 <= k; j += 8) gather_sum<8, kEoF32, kGated>(eo, sp + j, g + j, H, c, acc);
    for (; j + 4 <= k; j += 4) gather_sum<4, kEoF32, kGated>(eo, sp + j, g + j, H, c, acc);
    for (; j < k; ++j) {
      const int r = sp[j];
      if (r < 0) continue;
      float v[8];
      load8<kEoF32>(eo, static_cast<size_t>(r), H, c, v);
      const float gj = kGated ? g[j] : 1.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(gj, v[i], acc[i]);
    }
    if (shared != nullptr) {
      float v[8];
      load8<kEoF32>(shared, static_cast<size_t>(t), H, c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    if (kYF32) {
      float4* p = reinterpret_cast<float4*>(y) + (static_cast<size_t>(t) * H) / 4 + 2 * c;
      p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
      uint4 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      o.z = pack_bf16x2(acc[4], acc[5]);
      o.w = pack_bf16x2(acc[6], acc[7]);
      reinterpret_cast<uint4*>(y)[(static_cast<size_t>(t) * H) / 8 + c] = o;
    }
  }
}

hipError_t launch_combine(const void* eo, bool eo_f32, int N, int H, int k, const int32_t* send_pos,
                          const float* gate, const void* shared, void* y, bool y_f32, hipStream_t s) {
  const int groups8 = H / 8;
  const int threads = groups8 % 256 == 0 || groups8 % 128 != 0 ? 256 : 128;
  // small batches: split each row into up to one span per workgroup pass, for ~8
  // workgroups per CU
  const int passes = (groups8 + threads - 1) / threads;
  int spans = 1;
  if (N < 2048) {
    const int want = (2048 + N - 1) / N;
    spans = want < passes ? want : passes;
  }
  const dim3 grid(static_cast<unsigned>(static_cast<long long>(N) * spans)), block(threads);
  // gate == null: the expert outputs already carry their gates (plain sum)
  auto go = [&](auto eo32, auto y32, auto gated) {
    hipLaunchKernelGGL((combine_kernel<decltype(eo32)::value, decltype(y32)::value, decltype(gated)::value>), grid,
                       block, 0, s, eo, H, k, send_pos, gate, shared, y, spans);
  };
  using T = std::true_type;
  using F = std::false_type;
  if (gate != nullptr) {
    if (eo_f32 && y_f32) go(T{}, T{}, T{});
    else if (eo_f32) go(T{}, F{}, T{});
    else if (y_f32) go(F{}, T{}, T{});
    else go(F{}, F{}, T{});
  } else {
    if (eo_f32 && y_f32) go(T{}, T{}, F{});
    else if (eo_f32) go(T{}, F{}, F{});
    else if (y_f32) go(F{}, T{}, F{});
    else go(F{}, F{}, F{});
  }
  return hipGetLastError();
}

}  // namespace moe
