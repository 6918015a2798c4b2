// Router logits z = x . W_r^T: the router's linear map from each token's hidden state to its
// E expert logits ("EP / DeepEP explanation" page, section 2; "MoE part 4" page, section 4.2
// has the top-k read them).  x [N, H], W_r [E, H] (one row per expert), z [N, E] fp32.
//
// bf16 operands run on the 256 x 256 MFMA tile kernel of the expert GEMMs (MODE_ROUTER).
// A DeepSeek-V3-shaped router (8192 tokens x 256 experts) is only 32 output tiles, an
// eighth of the CUs, so K is cut into S parts: 8 at that shape, one per XCD, and each XCD
// streams its H/8-column slice of x once while its slice of W_r stays in its L2.  The S
// fp32 partial sums go to the workspace and a second kernel adds them in part order, so z
// is the same on every run.  fp32 operands and shapes outside the tile kernel's limits take
// a plain LDS-tiled kernel with fp32 FMAs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "grouped_gemm.h"
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kMaxParts = 16;

// z[i] = part_0[i] + part_1[i] + ... + part_{S-1}[i], in that order (n4 float4s per part)
__global__ __launch_bounds__(256) void router_sum_kernel(const float4* __restrict__ part, int S, long long n4,
                                                         float4* __restrict__ z) {
  const long long step = static_cast<long long>(gridDim.x) * blockDim.x;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4; i += step) {
    float4 a = part[i];
    for (int s = 1; s < S; ++s) {
      const float4 b = part[s * n4 + i];
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
    }
    z[i] = a;
  }
}

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, size_t i) {
  if constexpr (BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  else return reinterpret_cast<const float*>(p)[i];
}

// 64 tokens x 64 experts per workgroup; thread (ty, tx) of 16 x 16 owns tokens ty + 16 i and
// experts tx + 16 j (i, j < 4); K in steps of 16 through LDS.  Out-of-range rows and
// columns load zeros and store nothing.
template <bool BF16>
__global__ __launch_bounds__(256) void router_simple_kernel(const void* __restrict__ x, const void* __restrict__ w,
                                                            int N, int H, int E, float* __restrict__ z) {
  __shared__ float xs[16][65];
  __shared__ float ws[16][65];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const long long t0 = static_cast<long long>(blockIdx.x) * 64;
  const int e0 = blockIdx.y * 64;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  for (int h0 = 0; h0 < H; h0 += 16) {
    for (int i = threadIdx.x; i < 64 * 16; i += 256) {
      const int r = i >> 4, kk = i & 15;
      const int h = h0 + kk;
      const long long t = t0 + r;
      const int e = e0 + r;
      xs[kk][r] = (t < N && h < H) ? load_elem<BF16>(x, static_cast<size_t>(t) * H + h) : 0.0f;
      ws[kk][r] = (e < E && h < H) ? load_elem<BF16>(w, static_cast<size_t>(e) * H + h) : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = ws[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const long long t = t0 + ty + 16 * i;
    if (t >= N) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx + 16 * j;
      if (e < E) z[static_cast<size_t>(t) * E + e] = acc[i][j];
    }
  }
}

}  // namespace

int router_parts(int N, int H, int E, bool bf16) {
  if (!bf16 || N <= 0 || H % 128 != 0 || E % 4 != 0) return 0;
  if (static_cast<long long>(E) * H * 2 >= (1LL << 32)) return 0;
  const long long tiles = static_cast<long long>((N + kWideTileRows - 1) / kWideTileRows) * ((E + 255) / 256);
  // the most parts (dividing the H / 128 column blocks, at most kMaxParts) that keep the
  // tiles within one per CU
  const int blocks = H / 128;
  int best = 1;
  for (int d = 2; d <= blocks && d <= kMaxParts; ++d)
    if (blocks % d == 0 && tiles * d <= 256) best = d;
  return best;
}

size_t router_ws_bytes(int N, int H, int E, bool bf16) {
  const int S = router_parts(N, H, E, bf16);
  if (S <= 1) return 0;
  return (static_cast<size_t>(S) * N * E * sizeof(float) + 255) & ~static_cast<size_t>(255);
}

hipError_t launch_router_logits(const void* x, bool bf16, int N, int H, const void* w_r, int E, float* z,
                                void* ws, hipStream_t s) {
  const int S = router_parts(N, H, E, bf16);
  if (S == 0) {
    const dim3 grid((N + 63) / 64, (E + 63) / 64), block(256);
    if (bf16) hipLaunchKernelGGL(router_simple_kernel<true>, grid, block, 0, s, x, w_r, N, H, E, z);
    else hipLaunchKernelGGL(router_simple_kernel<false>, grid, block, 0, s, x, w_r, N, H, E, z);
    return hipGetLastError();
  }
  GemmArgs p = {};
  p.a = reinterpret_cast<const uint8_t*>(x);
  p.b = reinterpret_cast<const uint8_t*>(w_r);
  p.out = S > 1 ? ws : static_cast<void*>(z);
  p.E = 1;
  p.K = H;
  p.rows = N;
  p.I = E;
  p.n_out = E;
  p.b_rows = E;
  p.out_f32 = 1;
  p.a_div = 1;
  p.k_split = S;
  hipError_t err = launch_grouped_gemm_wide(MODE_ROUTER, p, s);
  if (err != hipSuccess || S == 1) return err;
  const long long n4 = static_cast<long long>(N) * E / 4;
  const long long blocks = (n4 + 255) / 256;
  const dim3 grid(static_cast<unsigned>(blocks < 2048 ? blocks : 2048)), block(256);
  hipLaunchKernelGGL(router_sum_kernel, grid, block, 0, s, reinterpret_cast<const float4*>(ws), S, n4,
                     reinterpret_cast<float4*>(z));
  return hipGetLastError();
}

}  // namespace moe
