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
    // group score = largest key inside the group; lane g keeps the score of group g
    const int G = E / n_group;
    uint32_t gscore = 0;
    for (int g = 0; g < n_group; ++g) {
      uint32_t m = 0;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int e = lane * V + v;
        if (e < E && e / G == g) m = key[v] > m ? key[v] : m;
      }
      m = wave_max_u32(m);
      if (lane == g) gscore = m;
    }
    uint64_t cand = lane < n_group
                        ? ((static_cast<uint64_t>(gscore) << 32) | (0xFFFFu - static_cast<uint32_t>(lane)))
                        : 0;
    uint64_t allowed = 0;
    for (int r = 0; r < topk_group; ++r) {
      const uint64_t best = wave_max_u64(cand);
      const int g = static_cast<int>(0xFFFFu - static_cast<uint32_t>(best & 0xFFFFu));
      allowed |= 1ull << g;
      if (lane == g) cand = 0;
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
    const uint64_t best = wave_max_u64(lb);
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
  const float m = __shfl(val, 0, kWave);
  const float w = lane < k ? expf(val - m) : 0.0f;
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) sum += __shfl(w, j, kWave);
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
