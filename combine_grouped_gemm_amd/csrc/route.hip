// Router top-k: one wavefront per token.
//
// Implements the router step of the layer ("EP / DeepEP explanation" page, section 2;
// "MoE part 4" page, section 4.2: correction bias, grouped top-k, renormalised gates;
// "Wide EP" page, "Group-limited routing").
//
// Each lane holds V consecutive experts of the token's logit row.  A logit becomes an
// order-preserving 32-bit key; key << 32 | (0xFFFF - expert) makes one unsigned 64-bit
// maximum pick the larger logit and, on equal logits, the lower expert index.  k rounds
// of a wave-wide maximum extract the top-k in descending order.  Removed experts (those
// already chosen, or outside the allowed groups) hold key 0, below every finite logit.
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {
namespace {

// Wave-wide maxima without LDS round trips: within each 16 lanes by DPP (lane ^ 1, lane ^ 2 by
// quad permutes, then the 8- and 16-lane mirrors), then across the 16-lane rows and the two
// wave halves by gfx950's permlane swaps.  Every lane ends with the maximum; every lane must
// take part.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int kRowHalfMirror = 0x141;   // lane i of 8 reads lane 7 - i
constexpr int kRowMirror = 0x140;       // lane i of 16 reads lane 15 - i

__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint32_t wave_max32(uint32_t v) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  v = umax32(v, dpp_mov<kQuadXor1>(v));
  v = umax32(v, dpp_mov<kQuadXor2>(v));
  v = umax32(v, dpp_mov<kRowHalfMirror>(v));
  v = umax32(v, dpp_mov<kRowMirror>(v));
  u32x2_t t = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = umax32(t[0], t[1]);
  t = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __builtin_amdgcn_readfirstlane(umax32(t[0], t[1]));
}

__device__ __forceinline__ uint64_t wave_max64(uint64_t v) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  uint32_t hi = static_cast<uint32_t>(v >> 32), lo = static_cast<uint32_t>(v);
  auto take = [&](uint32_t ohi, uint32_t olo) __attribute__((always_inline)) {
    const bool gt = ohi > hi || (ohi == hi && olo > lo);
    hi = gt ? ohi : hi;
    lo = gt ? olo : lo;
  };
  take(dpp_mov<kQuadXor1>(hi), dpp_mov<kQuadXor1>(lo));
  take(dpp_mov<kQuadXor2>(hi), dpp_mov<kQuadXor2>(lo));
  take(dpp_mov<kRowHalfMirror>(hi), dpp_mov<kRowHalfMirror>(lo));
  take(dpp_mov<kRowMirror>(hi), dpp_mov<kRowMirror>(lo));
  u32x2_t th = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  u32x2_t tl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  hi = th[0];
  lo = tl[0];
  take(th[1], tl[1]);
  th = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  tl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  hi = th[0];
  lo = tl[0];
  take(th[1], tl[1]);
  return (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(hi)) << 32) | __builtin_amdgcn_readfirstlane(lo);
}

}  // namespace

template <int V>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ z, int N, int E,
                                                    int k, const float* __restrict__ bias,
                                                    int n_group, int topk_group,
                                                    int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_gate) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (256 / kWave) + (threadIdx.x / kWave);
  if (t >= N) return;  // uniform per wave

  const float* zr = z + static_cast<size_t>(t) * E;
  uint32_t key[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int e = lane * V + v;
    if (e < E) {
      float f = zr[e];
      if (bias != nullptr) f = f + bias[e];
      key[v] = order_key(f);
    } else {
      key[v] = 0;
    }
  }

  if (n_group > 0) {
    // group score = largest key inside the group.  When a group is a run of seg = G / V
    // lanes (seg a power of two up to 16), every lane of the run gets its group's score by a
    // segmented maximum; otherwise one wave maximum per group, and lane g keeps group g's
    // score (seg = 1).  Lanes past the groups hold no candidate.
    const int G = E / n_group;
    const int lpg = G % V == 0 ? G / V : 0;
    const bool segmented = lpg > 0 && lpg <= 16 && (lpg & (lpg - 1)) == 0;
    const int seg = segmented ? lpg : 1;
    uint32_t gscore = 0;
    if (segmented) {   // (a lane's V experts all lie in one group)
#pragma unroll
      for (int v = 0; v < V; ++v) gscore = umax32(gscore, key[v]);
      if (seg >= 2) gscore = umax32(gscore, dpp_mov<kQuadXor1>(gscore));
      if (seg >= 4) gscore = umax32(gscore, dpp_mov<kQuadXor2>(gscore));
      if (seg >= 8) gscore = umax32(gscore, dpp_mov<kRowHalfMirror>(gscore));
      if (seg >= 16) gscore = umax32(gscore, dpp_mov<kRowMirror>(gscore));
    } else {
      for (int g = 0; g < n_group; ++g) {
        uint32_t m = 0;
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const int e = lane * V + v;
          if (e < E && e / G == g) m = key[v] > m ? key[v] : m;
        }
        m = wave_max32(m);
        if (lane == g) gscore = m;
      }
    }
    const int my_g = lane / seg;
    uint64_t cand = my_g < n_group
                        ? ((static_cast<uint64_t>(gscore) << 32) | (0xFFFFu - static_cast<uint32_t>(my_g)))
                        : 0;
    uint64_t allowed = 0;
    for (int r = 0; r < topk_group; ++r) {
      const uint64_t best = wave_max64(cand);
      const int g = static_cast<int>(0xFFFFu - static_cast<uint32_t>(best & 0xFFFFu));
      allowed |= 1ull << g;
      if (my_g == g) cand = 0;
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = lane * V + v;
      if (e < E && !((allowed >> (e / G)) & 1ull)) key[v] = 0;
    }
  }

  auto local_best = [&]() {
    uint64_t b = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const uint32_t e = static_cast<uint32_t>(lane * V + v);
      const uint64_t p = key[v] ? ((static_cast<uint64_t>(key[v]) << 32) | (0xFFFFu - e)) : 0;
      b = p > b ? p : b;
    }
    return b;
  };

  uint64_t lb = local_best();
  int my_e = 0;
  uint32_t my_key = 0;
  for (int j = 0; j < k; ++j) {
    const uint64_t best = wave_max64(lb);
    const int e = static_cast<int>(0xFFFFu - static_cast<uint32_t>(best & 0xFFFFu));
    if (lane == j) {
      my_e = e;
      my_key = static_cast<uint32_t>(best >> 32);
    }
    if (lane == e / V) {
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (lane * V + v == e) key[v] = 0;
      lb = local_best();
    }
  }

  // renormalised softmax over the k selected biased logits, fp32, summed j = 0..k-1
  const float val = key_to_float(my_key);
  const float m = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(uint32_t, val)));
  const float w = lane < k ? expf(val - m) : 0.0f;
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) sum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(uint32_t, w), j));
  if (lane < k) {
    topk_idx[static_cast<size_t>(t) * k + lane] = my_e;
    topk_gate[static_cast<size_t>(t) * k + lane] = w / sum;
  }
}

hipError_t launch_route(const float* z, int N, int E, int k, const float* bias, int n_group,
                        int topk_group, int32_t* topk_idx, float* topk_gate, hipStream_t s) {
  const dim3 grid((N + 3) / 4), block(256);
  if (E <= 64)
    hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, s, z, N, E, k, bias, n_group, topk_group, topk_idx, topk_gate);
  else if (E <= 128)
    hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, s, z, N, E, k, bias, n_group, topk_group, topk_idx, topk_gate);
  else if (E <= 256)
    hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, s, z, N, E, k, bias, n_group, topk_group, topk_idx, topk_gate);
  else if (E <= 512)
    hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, s, z, N, E, k, bias, n_group, topk_group, topk_idx, topk_gate);
  else
    hipLaunchKernelGGL(route_kernel<16>, grid, block, 0, s, z, N, E, k, bias, n_group, topk_group, topk_idx, topk_gate);
  return hipGetLastError();
}

}  // namespace moe
