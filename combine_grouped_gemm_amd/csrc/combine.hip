// Combine (unpermute + gate-weighted sum back to token order):
//   y_t = sum_{j<k} g_{t,j} * expert_out[send_pos[t*k+j]]  (+ shared_out_t)
// ("EP / DeepEP explanation" page, sections 2 and 3; "DeepEP" page, section 7: the sum is
// kept in a wider type than the payload).
//
// Each workgroup takes one token and one span of its columns (the row is split into
// `spans` spans, so that small batches still fill the GPU); each lane owns 8 consecutive
// columns per pass, accumulates in fp32 in the order j = 0..k-1 then the shared row, rounds
// once and writes 16 bytes (bf16) or 32 bytes (fp32).  Gates and send positions are uniform
// across the workgroup, whose size (128 or 256 lanes) divides the row's 8-column groups
// when it can, so that no pass over the row leaves lanes idle.
//
// k <= 8: a pass issues the k gathered 16-byte loads and the shared row's load together,
// and the next pass's loads before this pass's sum, so a lane keeps two passes' rows in
// flight and waits for memory once per pass.  Larger k: rows in batches of 8 and 4.
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

// 8 columns of one row as loaded: one 16-byte word (bf16) or two (fp32)
template <bool kEoF32>
struct Raw8 {
  uint4 w[kEoF32 ? 2 : 1];
};

// streaming 16-byte load: every expert row and shared row is read exactly once, so the
// loads carry the non-temporal hint (measured: a 9-rows-read-per-row-written stream moves
// ~10% more bytes per second with it)
typedef uint32_t stream_word_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const stream_word_t v = __builtin_nontemporal_load(reinterpret_cast<const stream_word_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// NT: the non-temporal hint (rows read once); otherwise plain loads (rows read by many
// tokens, such as the router weight's rows in the router's input gradient)
template <bool NT>
__device__ __forceinline__ uint4 load_row16(const uint4* p) {
  if (NT) return load_stream(p);
  return *p;
}

template <bool kEoF32, bool NT>
__device__ __forceinline__ void raw_load(const void* base, size_t row, int H, int c, Raw8<kEoF32>& r) {
  if (kEoF32) {
    const uint4* p = reinterpret_cast<const uint4*>(base) + (row * H) / 4 + 2 * c;
    r.w[0] = load_row16<NT>(p);
    r.w[kEoF32 ? 1 : 0] = load_row16<NT>(p + 1);
  } else {
    r.w[0] = load_row16<NT>(reinterpret_cast<const uint4*>(base) + (row * H) / 8 + c);
  }
}

template <bool kEoF32>
__device__ __forceinline__ void raw_values(const Raw8<kEoF32>& r, float (&v)[8]) {
  if (kEoF32) {
    const uint32_t w[8] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w,
                           r.w[kEoF32 ? 1 : 0].x, r.w[kEoF32 ? 1 : 0].y, r.w[kEoF32 ? 1 : 0].z, r.w[kEoF32 ? 1 : 0].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
  } else {
    const uint32_t w[4] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(static_cast<uint16_t>(w[i] & 0xFFFFu));
      v[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(w[i] >> 16));
    }
  }
}

// k <= KMAX <= 8: one pass = the k rows and the shared row of 8 columns, loaded together;
// the next pass is loaded before this one is summed
template <int KMAX, bool kEoF32, bool kYF32, bool kGated, bool kShared, bool NT>
__global__ __launch_bounds__(kCombMaxThreads) void combine_kernel_small_k(
    const void* __restrict__ eo, int H, int k, const int32_t* __restrict__ send_pos,
    const float* __restrict__ gate, const void* __restrict__ shared, void* __restrict__ y, int spans) {
  const int t = blockIdx.x / spans;
  const int span = blockIdx.x % spans;
  int r[KMAX];
  float g[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    r[j] = j < k ? send_pos[static_cast<size_t>(t) * k + j] : -1;
    g[j] = kGated && j < k ? gate[static_cast<size_t>(t) * k + j] : 1.0f;
  }
  const int groups8 = H / 8;
  const int per_span = (groups8 + spans - 1) / spans;
  const int c_end = (span + 1) * per_span < groups8 ? (span + 1) * per_span : groups8;
  constexpr int NB = KMAX + (kShared ? 1 : 0);
  auto issue = [&](int c, Raw8<kEoF32> (&b)[NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (r[j] >= 0) raw_load<kEoF32, NT>(eo, static_cast<size_t>(r[j]), H, c, b[j]);
    if (kShared) raw_load<kEoF32, true>(shared, static_cast<size_t>(t), H, c, b[NB - 1]);
  };
  auto finish = [&](int c, const Raw8<kEoF32> (&b)[NB]) __attribute__((always_inline)) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (r[j] < 0) continue;
      float v[8];
      raw_values<kEoF32>(b[j], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(g[j], v[i], acc[i]);   // (fma with 1 is the plain sum)
    }
    if (kShared) {
      float v[8];
      raw_values<kEoF32>(b[NB - 1], v);
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
  };
  Raw8<kEoF32> b0[NB], b1[NB];
  int c = span * per_span + threadIdx.x;
  if (c < c_end) issue(c, b0);
  // two passes per trip so that the buffers keep fixed registers
  for (;;) {
    if (c >= c_end) break;
    const int c1 = c + static_cast<int>(blockDim.x);
    if (c1 < c_end) issue(c1, b1);
    finish(c, b0);
    if (c1 >= c_end) break;
    const int c2 = c1 + static_cast<int>(blockDim.x);
    if (c2 < c_end) issue(c2, b0);
    finish(c1, b1);
    c = c2;
  }
}

hipError_t launch_combine(const void* eo, bool eo_f32, int N, int H, int k, const int32_t* send_pos,
                          const float* gate, const void* shared, void* y, bool y_f32, hipStream_t s,
                          bool rows_once) {
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
    constexpr bool A = decltype(eo32)::value, B = decltype(y32)::value, G = decltype(gated)::value;
    auto small = [&](auto kmax) {
      constexpr int KM = decltype(kmax)::value;
      if (shared != nullptr && rows_once)
        hipLaunchKernelGGL((combine_kernel_small_k<KM, A, B, G, true, true>), grid, block, 0, s, eo, H, k, send_pos,
                           gate, shared, y, spans);
      else if (shared != nullptr)
        hipLaunchKernelGGL((combine_kernel_small_k<KM, A, B, G, true, false>), grid, block, 0, s, eo, H, k, send_pos,
                           gate, shared, y, spans);
      else if (rows_once)
        hipLaunchKernelGGL((combine_kernel_small_k<KM, A, B, G, false, true>), grid, block, 0, s, eo, H, k, send_pos,
                           gate, shared, y, spans);
      else
        hipLaunchKernelGGL((combine_kernel_small_k<KM, A, B, G, false, false>), grid, block, 0, s, eo, H, k,
                           send_pos, gate, shared, y, spans);
    };
    if (k <= 2) small(std::integral_constant<int, 2>{});
    else if (k <= 4) small(std::integral_constant<int, 4>{});
    else if (k <= 8) small(std::integral_constant<int, 8>{});
    else hipLaunchKernelGGL((combine_kernel<A, B, G>), grid, block, 0, s, eo, H, k, send_pos, gate, shared, y, spans);
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

// ------------------------------------------------------------------------------------
// Read-mostly streaming probe (a measurement, not a step of the layer): dst[i] = the sum
// over j < R of src[j * n + i], as four 32-bit integer lanes per 16-byte word.  It reads
// R * n * 16 bytes (non-temporal, as combine reads) and writes n * 16 bytes, every access
// sequential: combine's access mix (R rows read per row written) without its gather.  Its
// rate is the ceiling against which combine's HBM rate is read.
// ------------------------------------------------------------------------------------

template <int R>
__global__ __launch_bounds__(256) void stream_probe_kernel(const uint4* __restrict__ src, size_t n,
                                                           uint4* __restrict__ dst) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    uint4 v[R];
#pragma unroll
    for (int j = 0; j < R; ++j) v[j] = load_stream(src + static_cast<size_t>(j) * n + i);
    uint4 a = v[0];
#pragma unroll
    for (int j = 1; j < R; ++j) {
      a.x += v[j].x;
      a.y += v[j].y;
      a.z += v[j].z;
      a.w += v[j].w;
    }
    dst[i] = a;
  }
}

hipError_t launch_stream_probe(const void* src, size_t n16, int ratio, void* dst, hipStream_t s) {
  // short-lived workgroups of about two words per lane (measured faster than a few long
  // grid-stride loops)
  const size_t want = (n16 + 511) / 512;
  const unsigned blocks = static_cast<unsigned>(want < 65535 ? (want > 0 ? want : 1) : 65535);
  const uint4* a = reinterpret_cast<const uint4*>(src);
  uint4* d = reinterpret_cast<uint4*>(dst);
  switch (ratio) {
    case 1: hipLaunchKernelGGL(stream_probe_kernel<1>, dim3(blocks), dim3(256), 0, s, a, n16, d); break;
    case 2: hipLaunchKernelGGL(stream_probe_kernel<2>, dim3(blocks), dim3(256), 0, s, a, n16, d); break;
    case 4: hipLaunchKernelGGL(stream_probe_kernel<4>, dim3(blocks), dim3(256), 0, s, a, n16, d); break;
    case 8: hipLaunchKernelGGL(stream_probe_kernel<8>, dim3(blocks), dim3(256), 0, s, a, n16, d); break;
    case 9: hipLaunchKernelGGL(stream_probe_kernel<9>, dim3(blocks), dim3(256), 0, s, a, n16, d); break;
    default: hipLaunchKernelGGL(stream_probe_kernel<16>, dim3(blocks), dim3(256), 0, s, a, n16, d); break;
  }
  return hipGetLastError();
}

}  // namespace moe
