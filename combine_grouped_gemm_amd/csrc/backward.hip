// Elementwise and gather steps of the layer's backward pass ("DeepSeek MoE: EP and FSDP
// guide": the backward mirrors the forward, dispatch's backward being combine):
//
//   combine backward   d_expert_out[send_pos[s]] = g_s dy_t,  d_gate[s] = <dy_t, expert_out[send_pos[s]]>
//   SwiGLU backward    da = dh u s(a) (1 + a (1 - s(a))),  du = dh a s(a)   (s the logistic), h = a s(a) u
//   gates backward     dz_s = g_s (dg_s - sum_j g_j dg_j) over a token's k slots
//   router wgrad       dW_r[e] = sum over the slots s routed to e of dz_s x_{token(s)}
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_common.h"

namespace moe {
namespace {

template <bool F32>
struct Vec;
template <>
struct Vec<true> {   // 4 fp32 per 16 bytes
  static constexpr int kN = 4;
  __device__ static void load(const void* p, size_t i, float (&v)[4]) {
    const float4 q = reinterpret_cast<const float4*>(p)[i];
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
  __device__ static void store(void* p, size_t i, const float (&v)[4]) {
    reinterpret_cast<float4*>(p)[i] = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <>
struct Vec<false> {  // 8 bf16 per 16 bytes
  static constexpr int kN = 8;
  __device__ static void load(const void* p, size_t i, float (&v)[8]) {
    const uint4 q = reinterpret_cast<const uint4*>(p)[i];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_to_f32(static_cast<uint16_t>(w[j] & 0xFFFF));
      v[2 * j + 1] = bf16_to_f32(static_cast<uint16_t>(w[j] >> 16));
    }
  }
  __device__ static void store(void* p, size_t i, const float (&v)[8]) {
    reinterpret_cast<uint4*>(p)[i] = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
  }
};

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();   // red is free (its previous use has been read)
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float s = 0.0f;
  for (int w = 0; w < nw; ++w) s += red[w];
  return s;
}

// one workgroup per token
template <bool F32>
__global__ __launch_bounds__(256) void combine_backward_kernel(const void* __restrict__ dy, int H, int k,
                                                               const int32_t* __restrict__ send_pos,
                                                               const float* __restrict__ gate,
                                                               const void* __restrict__ eo, void* __restrict__ d_eo,
                                                               float* __restrict__ d_gate) {
  using V = Vec<F32>;
  constexpr int kV = V::kN;
  __shared__ float red[4];
  const long long t = blockIdx.x;
  const int chunks = H / kV;
  for (int j = 0; j < k; ++j) {
    const long long s = t * k + j;
    const int row = send_pos[s];
    if (row < 0) {   // (uniform over the workgroup)
      if (threadIdx.x == 0) d_gate[s] = 0.0f;
      continue;
    }
    const float g = gate[s];
    float dot = 0.0f;
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
      float a[kV], o[kV], d[kV];
      V::load(dy, static_cast<size_t>(t) * chunks + c, a);
      V::load(eo, static_cast<size_t>(row) * chunks + c, o);
#pragma unroll
      for (int q = 0; q < kV; ++q) {
        dot = fmaf(a[q], o[q], dot);
        d[q] = g * a[q];
      }
      V::store(d_eo, static_cast<size_t>(row) * chunks + c, d);
    }
    dot = block_sum(dot, red);
    if (threadIdx.x == 0) d_gate[s] = dot;
  }
}

// au [rows, 2I] (gate pre-activations in columns 0..I-1, up in I..2I-1), dh [rows, I];
// 8 columns per thread
__global__ __launch_bounds__(256) void swiglu_backward_kernel(const uint16_t* __restrict__ au,
                                                              const uint16_t* __restrict__ dh, long long rows, int I,
                                                              uint16_t* __restrict__ d_au, uint16_t* __restrict__ h) {
  const int cpr = I / 8;   // chunks per row
  const long long n = rows * cpr;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<long long>(gridDim.x) * blockDim.x) {
    const long long r = i / cpr;
    const int c = static_cast<int>(i - r * cpr);
    float a[8], u[8], d[8], da[8], du[8], hv[8];
    Vec<false>::load(au, static_cast<size_t>(r) * 2 * cpr + c, a);
    Vec<false>::load(au, static_cast<size_t>(r) * 2 * cpr + cpr + c, u);
    Vec<false>::load(dh, static_cast<size_t>(r) * cpr + c, d);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float sg = sigmoid_f32(a[q]);
      da[q] = d[q] * u[q] * sg * (1.0f + a[q] * (1.0f - sg));
      du[q] = d[q] * a[q] * sg;
      hv[q] = a[q] * sg * u[q];
    }
    Vec<false>::store(d_au, static_cast<size_t>(r) * 2 * cpr + c, da);
    Vec<false>::store(d_au, static_cast<size_t>(r) * 2 * cpr + cpr + c, du);
    if (h != nullptr) Vec<false>::store(h, static_cast<size_t>(r) * cpr + c, hv);
  }
}

// one thread per token
__global__ __launch_bounds__(256) void gates_backward_kernel(const float* __restrict__ gate,
                                                             const float* __restrict__ dg, int N, int k,
                                                             float* __restrict__ dz) {
  const long long t = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= N) return;
  const float* g = gate + t * k;
  const float* d = dg + t * k;
  float s = 0.0f;
  for (int j = 0; j < k; ++j) s = fmaf(g[j], d[j], s);
  for (int j = 0; j < k; ++j) dz[t * k + j] = g[j] * (d[j] - s);
}

// grid (E, column blocks): each thread sums 16-byte column chunks of x over the expert's
// layout rows (row r holds slot src_slot[r], token src_slot[r] / k), in row order
template <bool F32>
__global__ __launch_bounds__(256) void router_wgrad_kernel(const int32_t* __restrict__ offsets, int rows,
                                                           const int32_t* __restrict__ src_slot, int k,
                                                           const float* __restrict__ dz, const void* __restrict__ x,
                                                           int N, int H, void* __restrict__ dw, int dw_f32) {
  using V = Vec<F32>;
  constexpr int kV = V::kN;
  const int e = blockIdx.x;
  const int chunks = H / kV;
  const int c = blockIdx.y * blockDim.x + threadIdx.x;
  if (c >= chunks) return;
  int lo = offsets[e], hi = offsets[e + 1];
  lo = lo < 0 ? 0 : (lo > rows ? rows : lo);
  hi = hi < lo ? lo : (hi > rows ? rows : hi);
  const long long nk = static_cast<long long>(N) * k;
  float acc[kV];
#pragma unroll
  for (int q = 0; q < kV; ++q) acc[q] = 0.0f;
  for (int r = lo; r < hi; ++r) {
    long long s = src_slot[r];
    s = s < 0 ? 0 : (s < nk ? s : nk - 1);
    const float w = dz[s];
    float v[kV];
    V::load(x, static_cast<size_t>(s / k) * chunks + c, v);
#pragma unroll
    for (int q = 0; q < kV; ++q) acc[q] = fmaf(w, v[q], acc[q]);
  }
  if (dw_f32) {
    float* o = reinterpret_cast<float*>(dw) + static_cast<size_t>(e) * H + c * kV;
#pragma unroll
    for (int q = 0; q < kV; ++q) o[q] = acc[q];
  } else {
    uint16_t* o = reinterpret_cast<uint16_t*>(dw) + static_cast<size_t>(e) * H + c * kV;
#pragma unroll
    for (int q = 0; q < kV; ++q) o[q] = f32_to_bf16(acc[q]);
  }
}

}  // namespace

hipError_t launch_combine_backward(const void* dy, bool f32, int N, int H, int k, const int32_t* send_pos,
                                   const float* gate, const void* eo, void* d_eo, float* d_gate, hipStream_t s) {
  if (f32)
    hipLaunchKernelGGL(combine_backward_kernel<true>, dim3(N), dim3(256), 0, s, dy, H, k, send_pos, gate, eo, d_eo,
                       d_gate);
  else
    hipLaunchKernelGGL(combine_backward_kernel<false>, dim3(N), dim3(256), 0, s, dy, H, k, send_pos, gate, eo, d_eo,
                       d_gate);
  return hipGetLastError();
}

hipError_t launch_swiglu_backward(const void* au, const void* dh, long long rows, int I, void* d_au, void* h,
                                  hipStream_t s) {
  const long long n = rows * (I / 8);
  const long long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(swiglu_backward_kernel, dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)), dim3(256),
                     0, s, reinterpret_cast<const uint16_t*>(au), reinterpret_cast<const uint16_t*>(dh), rows, I,
                     reinterpret_cast<uint16_t*>(d_au), reinterpret_cast<uint16_t*>(h));
  return hipGetLastError();
}

hipError_t launch_router_backward(const float* gate, const float* d_gate, int N, int k, const int32_t* offsets,
                                  const int32_t* src_slot, int E, int rows, const void* x, bool x_f32, int H,
                                  float* dz, void* dw, bool dw_f32, hipStream_t s) {
  if (N > 0) {
    hipLaunchKernelGGL(gates_backward_kernel, dim3((N + 255) / 256), dim3(256), 0, s, gate, d_gate, N, k, dz);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int chunks = H / (x_f32 ? 4 : 8);
  const dim3 grid(E, (chunks + 255) / 256);
  if (x_f32)
    hipLaunchKernelGGL(router_wgrad_kernel<true>, grid, dim3(256), 0, s, offsets, rows, src_slot, k, dz, x, N, H, dw,
                       dw_f32 ? 1 : 0);
  else
    hipLaunchKernelGGL(router_wgrad_kernel<false>, grid, dim3(256), 0, s, offsets, rows, src_slot, k, dz, x, N, H, dw,
                       dw_f32 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace moe
