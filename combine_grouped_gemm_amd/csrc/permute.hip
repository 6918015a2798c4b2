// Permute (the on-device stand-in of the dispatch exchange): each token row is read once
// and written to its k rows of the expert-ordered buffer ("EP / DeepEP explanation" page,
// section 3; "MoE part 4" page, section 4).  The fp8 variant quantizes each token once per
// 128-column block and writes the codes and the block scales with the same row index
// ("EP / DeepEP explanation" page, section 6; "DeepEP" page, section 7).
//
// One workgroup per token; 16-byte vector loads and stores, consecutive lanes on
// consecutive 16-byte chunks of a row, so every load and store is fully coalesced.  The
// send positions are uniform across the workgroup and live in scalar registers.
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

constexpr int kPermThreads = 256;

// a lane's (up to) four 16-byte chunks of the row are loaded together, then written to the
// token's k rows with non-temporal stores (the rows are written once, not read back here)
typedef uint32_t perm_word_t __attribute__((ext_vector_type(4)));
constexpr int kPermUnroll = 4;

__global__ __launch_bounds__(kPermThreads) void permute_copy_kernel(
    const uint4* __restrict__ x, int row_chunks, int k, const int32_t* __restrict__ send_pos,
    uint4* __restrict__ out) {
  const int t = blockIdx.x;
  const uint4* src = x + static_cast<size_t>(t) * row_chunks;
  const int32_t* sp = send_pos + static_cast<size_t>(t) * k;
  for (int c0 = threadIdx.x; c0 < row_chunks; c0 += kPermUnroll * kPermThreads) {
    perm_word_t v[kPermUnroll];
#pragma unroll
    for (int u = 0; u < kPermUnroll; ++u) {
      const int c = c0 + u * kPermThreads;
      if (c < row_chunks) {
        const uint4 a = src[c];
        v[u] = perm_word_t{a.x, a.y, a.z, a.w};
      }
    }
    for (int j = 0; j < k; ++j) {
      const int r = sp[j];
      if (r < 0) continue;
      perm_word_t* dst = reinterpret_cast<perm_word_t*>(out + static_cast<size_t>(r) * row_chunks);
#pragma unroll
      for (int u = 0; u < kPermUnroll; ++u) {
        const int c = c0 + u * kPermThreads;
        if (c < row_chunks) __builtin_nontemporal_store(v[u], dst + c);
      }
    }
  }
}

// 16 lanes cover one 128-column block (8 values each).  XT is the input element type.
template <bool kF32In>
__global__ __launch_bounds__(kPermThreads) void permute_fp8_kernel(
    const void* __restrict__ x, int H, int k, const int32_t* __restrict__ send_pos,
    uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int t = blockIdx.x;
  const int groups8 = H / 8;       // 8-value groups per row
  const int nblk = H / 128;        // scale blocks per row
  for (int c = threadIdx.x; c < groups8; c += kPermThreads) {
    float v[8];
    if (kF32In) {
      const float4* src = reinterpret_cast<const float4*>(x) + (static_cast<size_t>(t) * H) / 4 + 2 * c;
      const float4 a = src[0], b = src[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
      const uint4 a = reinterpret_cast<const uint4*>(x)[(static_cast<size_t>(t) * H) / 8 + c];
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_to_f32(static_cast<uint16_t>(w[i] & 0xFFFFu));
        v[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(w[i] >> 16));
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
    const float s = amax == 0.0f ? 1.0f : amax / 448.0f;  // IEEE division
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= f32_to_e4m3(v[i] / s) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= f32_to_e4m3(v[4 + i] / s) << (8 * i);
    const uint2 codes = make_uint2(lo, hi);
    const int blk = c / 16;
    for (int j = 0; j < k; ++j) {
      const int r = send_pos != nullptr ? send_pos[static_cast<size_t>(t) * k + j] : t;
      if (r < 0) continue;
      reinterpret_cast<uint2*>(q + static_cast<size_t>(r) * H)[c] = codes;
      if ((c & 15) == 0) scale[static_cast<size_t>(r) * nblk + blk] = s;
    }
  }
}

hipError_t launch_permute_copy(const void* x, size_t row_bytes, int N, int k,
                               const int32_t* send_pos, void* out, hipStream_t s) {
  const int row_chunks = static_cast<int>(row_bytes / 16);
  hipLaunchKernelGGL(permute_copy_kernel, dim3(N), dim3(kPermThreads), 0, s,
                     reinterpret_cast<const uint4*>(x), row_chunks, k, send_pos,
                     reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

hipError_t launch_permute_fp8(const void* x, bool f32_in, long long rows, int H, int k,
                              const int32_t* send_pos, uint8_t* q, float* scale, hipStream_t s) {
  // the grid's x dimension holds up to 2^31 - 1 workgroups, one per row
  if (f32_in)
    hipLaunchKernelGGL(permute_fp8_kernel<true>, dim3(static_cast<unsigned>(rows)), dim3(kPermThreads), 0, s,
                       x, H, k, send_pos, q, scale);
  else
    hipLaunchKernelGGL(permute_fp8_kernel<false>, dim3(static_cast<unsigned>(rows)), dim3(kPermThreads), 0, s,
                       x, H, k, send_pos, q, scale);
  return hipGetLastError();
}

}  // namespace moe
