// Grouped GEMMs of the layer's backward pass ("DeepSeek MoE: EP and FSDP guide": the backward
// mirrors the forward and every expert keeps its own weight gradients; "MoE part 4" page,
// section 2: one launch over the experts' ragged row counts).
//
//   dgrad:  out[r, n] = sum_k dC[r, k] W_e[k, n]          r in segment e   (W_e [K, N], n contiguous)
//   wgrad:  dW_e[m, n] = sum_{r in segment e} A[r, m] B[r', n]              (r' = r, or gathered)
//
// The forward kernels read both operands with k contiguous.  Here one (dgrad: W_e) or both
// (wgrad: A and B, k being the row index) have k as the slow index, so those operands are
// transposed on their way into LDS: a lane loads 8 consecutive m (or n) at one k and stores
// them into 8 LDS rows.  In LDS every operand is 128 rows (the tile's m or n) of 32 k,
// rows padded from 64 to 80 bytes so that the MFMA fragment reads (32 rows x 16 bytes) hit
// distinct banks.
//
// Tiles are 128 x 128, 256 threads in 2 x 2 waves of 64 x 64 (2 x 2 blocks of
// v_mfma_f32_32x32x16_bf16), K in stages of 32 double-buffered through registers: stage
// ks+1 is loaded from memory while stage ks is multiplied.  Logical tiles are dealt to the
// XCDs in contiguous ranges (workgroup i runs on XCD i mod 8): dgrad orders them expert ->
// n-block -> m-tile, so the m-tiles sharing a weight slice run together; wgrad expert ->
// m-block -> n-block, so an expert's rows are read by one XCD.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_device.h"
#include "grouped_gemm.h"
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {
namespace {

constexpr int kBT = 128;          // tile rows and columns
constexpr int kBK = 32;           // k per stage
constexpr int kPitch = 80;        // LDS bytes per tile row (64 used)
constexpr int kOpBytes = kBT * kPitch;
constexpr int kBwdThreads = 256;

enum { BWD_DGRAD = 0, BWD_WGRAD = 1 };

struct BwdArgs {
  const uint16_t* a;           // dgrad: dC [rows, K]; wgrad: A [rows, M]
  const uint16_t* b;           // dgrad: W [E, K, N]; wgrad: B [b_nrows or rows, N]
  void* out;                   // dgrad: [rows, N] bf16; wgrad: [E, M, N] (bf16 or fp32)
  const int32_t* offsets;      // [E + 1]
  const int32_t* tile_prefix;  // dgrad: m-tiles before each expert (128-row tiles)
  const int32_t* tile_expert;  // dgrad: m-tile -> expert
  const int32_t* b_rows;       // wgrad: row r of B is row b_rows[r] / b_div of b, or null
  int b_div, b_nrows;
  int E, rows, M, N, K;        // dgrad: M unused (rows); wgrad: K unused (segments)
  int out_f32;
};

__device__ __forceinline__ void seg_of(const BwdArgs& p, int e, int& lo, int& hi) {
  lo = p.offsets[e];
  hi = p.offsets[e + 1];
  lo = lo < 0 ? 0 : (lo > p.rows ? p.rows : lo);
  hi = hi < lo ? lo : (hi > p.rows ? p.rows : hi);
}

template <int MODE>
__global__ __launch_bounds__(kBwdThreads, 2) void grouped_gemm_bwd_kernel(BwdArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kOpBytes];   // [buffer][operand]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- the tile
  const int nN = p.N / kBT;
  long long total;
  if (MODE == BWD_DGRAD) total = static_cast<long long>(p.tile_prefix[p.E]) * nN;
  else total = static_cast<long long>(p.E) * (p.M / kBT) * nN;
  const int xcd = blockIdx.x % kNumXcd;
  const long long slot = blockIdx.x / kNumXcd;
  const long long per_xcd = (total + kNumXcd - 1) / kNumXcd;
  const long long L = xcd * per_xcd + slot;
  if (slot >= per_xcd || L >= total) return;

  int e, m0, mcount, n0, klo, kcount;
  if (MODE == BWD_DGRAD) {
    // expert -> n-block -> m-tile: expert e owns logical tiles [prefix[e] nN, prefix[e+1] nN);
    // the last expert whose range starts at or before L (an empty expert's range is empty,
    // so the search passes over it)
    int lo_e = 0, hi_e = p.E - 1;
    while (lo_e < hi_e) {
      const int mid = (lo_e + hi_e + 1) >> 1;
      if (static_cast<long long>(p.tile_prefix[mid]) * nN <= L) lo_e = mid;
      else hi_e = mid - 1;
    }
    e = lo_e;
    const int mt_e = p.tile_prefix[e + 1] - p.tile_prefix[e];
    const long long local = L - static_cast<long long>(p.tile_prefix[e]) * nN;
    const int nblk = static_cast<int>(local / mt_e);
    const int mtile = static_cast<int>(local % mt_e);
    int lo, hi;
    seg_of(p, e, lo, hi);
    m0 = lo + mtile * kBT;
    mcount = hi - m0 < kBT ? hi - m0 : kBT;
    n0 = nblk * kBT;
    klo = 0;
    kcount = p.K;
  } else {
    const int mB = p.M / kBT;
    e = static_cast<int>(L / (static_cast<long long>(mB) * nN));
    const int local = static_cast<int>(L - static_cast<long long>(e) * mB * nN);
    m0 = (local / nN) * kBT;
    n0 = (local % nN) * kBT;
    mcount = kBT;
    int lo, hi;
    seg_of(p, e, lo, hi);
    klo = lo;
    kcount = hi - lo;
  }
  if (MODE == BWD_DGRAD && mcount <= 0) return;

  // ---- loads of one stage (2 chunks of 16 bytes per thread and operand)
  // k-contiguous operand (dgrad A): chunk c -> tile row c / 4, k chunk c % 4
  // m/n-contiguous operand: chunk c -> k row c / 16, 8 columns at 8 * (c % 16)
  uint4 ra[2], rb[2];
  auto load_stage = [&](int ks) __attribute__((always_inline)) {
    const int k0 = ks * kBK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + kBwdThreads * i;
      if (MODE == BWD_DGRAD) {
        int r = c >> 2;
        r = r < mcount ? r : mcount - 1;
        ra[i] = *reinterpret_cast<const uint4*>(p.a + static_cast<size_t>(m0 + r) * p.K + k0 + (c & 3) * 8);
        const int kr = c >> 4;
        rb[i] = *reinterpret_cast<const uint4*>(p.b + (static_cast<size_t>(e) * p.K + k0 + kr) * p.N + n0 +
                                                (c & 15) * 8);
      } else {
        const int kr = c >> 4;
        const bool in = k0 + kr < kcount;
        const int r = klo + (in ? k0 + kr : 0);
        ra[i] = in ? *reinterpret_cast<const uint4*>(p.a + static_cast<size_t>(r) * p.M + m0 + (c & 15) * 8)
                   : make_uint4(0, 0, 0, 0);
        int rbow = r;
        if (p.b_rows != nullptr) {
          rbow = p.b_rows[r] / p.b_div;
          rbow = rbow < 0 ? 0 : (rbow < p.b_nrows ? rbow : p.b_nrows - 1);
        }
        rb[i] = in ? *reinterpret_cast<const uint4*>(p.b + static_cast<size_t>(rbow) * p.N + n0 + (c & 15) * 8)
                   : make_uint4(0, 0, 0, 0);
      }
    }
  };
  // 8 values of one k at columns col .. col+7 into LDS rows col .. col+7
  auto put_transposed = [&](uint8_t* op, int kr, int col, uint4 v) __attribute__((always_inline)) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<uint16_t*>(op + (col + 2 * j) * kPitch + kr * 2) = static_cast<uint16_t>(w[j] & 0xFFFF);
      *reinterpret_cast<uint16_t*>(op + (col + 2 * j + 1) * kPitch + kr * 2) = static_cast<uint16_t>(w[j] >> 16);
    }
  };
  auto store_stage = [&](int buf) __attribute__((always_inline)) {
    uint8_t* la = lds[buf][0];
    uint8_t* lb = lds[buf][1];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + kBwdThreads * i;
      if (MODE == BWD_DGRAD) *reinterpret_cast<uint4*>(la + (c >> 2) * kPitch + (c & 3) * 16) = ra[i];
      else put_transposed(la, c >> 4, (c & 15) * 8, ra[i]);
      put_transposed(lb, c >> 4, (c & 15) * 8, rb[i]);
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  const int nk = (kcount + kBK - 1) / kBK;
  const int frow = lane & 31, fk = lane >> 5;
  if (nk > 0) {
    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
      const int buf = ks & 1;
      if (ks + 1 < nk) load_stage(ks + 1);
      const uint8_t* la = lds[buf][0];
      const uint8_t* lb = lds[buf][1];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        uint4 fa[2], fb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          fa[i] = *reinterpret_cast<const uint4*>(la + (wm * 64 + i * 32 + frow) * kPitch + (2 * s + fk) * 16);
          fb[i] = *reinterpret_cast<const uint4*>(lb + (wn * 64 + i * 32 + frow) * kPitch + (2 * s + fk) * 16);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mma_bf16(fa[i], fb[j], acc[i][j]);
      }
      if (ks + 1 < nk) store_stage(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: lane l holds column n0 + wn*64 + j*32 + l % 32 and, in register v, row
  // wm*64 + i*32 + 8 (v / 4) + 4 (l / 32) + v % 4 of the tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + frow;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * fk + (v & 3);
        if (MODE == BWD_DGRAD) {
          if (r < mcount)
            reinterpret_cast<uint16_t*>(p.out)[static_cast<size_t>(m0 + r) * p.N + col] = f32_to_bf16(acc[i][j][v]);
        } else {
          const size_t o = (static_cast<size_t>(e) * p.M + m0 + r) * p.N + col;
          if (p.out_f32) reinterpret_cast<float*>(p.out)[o] = acc[i][j][v];
          else reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_bf16(acc[i][j][v]);
        }
      }
    }
}

unsigned grid_for(long long tiles) {
  const long long per_xcd = (tiles + kNumXcd - 1) / kNumXcd;
  return static_cast<unsigned>(per_xcd * kNumXcd);
}

}  // namespace

size_t bwd_dgrad_ws_bytes(int rows, int E) {
  const size_t n = static_cast<size_t>(E) + 1 + (rows + kBT - 1) / kBT + E + kNumXcd;
  return (n * sizeof(int32_t) + 255) & ~static_cast<size_t>(255);
}

hipError_t launch_expert_dgrad(const void* dC, const int32_t* offsets, int E, int rows, int K, int N, const void* w,
                               void* out, void* ws, hipStream_t s) {
  const int cap = (rows + kBT - 1) / kBT + E;
  int32_t* prefix = reinterpret_cast<int32_t*>(ws);
  int32_t* tile_expert = prefix + E + 1;
  int32_t* counter = tile_expert + cap;
  hipError_t err = launch_build_tiles(offsets, E, rows, kBT, cap, prefix, tile_expert, counter, s);
  if (err != hipSuccess) return err;
  BwdArgs p = {};
  p.a = reinterpret_cast<const uint16_t*>(dC);
  p.b = reinterpret_cast<const uint16_t*>(w);
  p.out = out;
  p.offsets = offsets;
  p.tile_prefix = prefix;
  p.tile_expert = tile_expert;
  p.E = E;
  p.rows = rows;
  p.N = N;
  p.K = K;
  p.b_div = 1;
  hipLaunchKernelGGL(grouped_gemm_bwd_kernel<BWD_DGRAD>, dim3(grid_for(static_cast<long long>(cap) * (N / kBT))),
                     dim3(kBwdThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_expert_wgrad(const void* a, const void* b, const int32_t* b_rows, int b_div, int b_nrows,
                               const int32_t* offsets, int E, int rows, int M, int N, void* dw, bool dw_f32,
                               hipStream_t s) {
  BwdArgs p = {};
  p.a = reinterpret_cast<const uint16_t*>(a);
  p.b = reinterpret_cast<const uint16_t*>(b);
  p.out = dw;
  p.offsets = offsets;
  p.b_rows = b_rows;
  p.b_div = b_div > 0 ? b_div : 1;
  p.b_nrows = b_nrows;
  p.E = E;
  p.rows = rows;
  p.M = M;
  p.N = N;
  p.out_f32 = dw_f32 ? 1 : 0;
  const long long tiles = static_cast<long long>(E) * (M / kBT) * (N / kBT);
  hipLaunchKernelGGL(grouped_gemm_bwd_kernel<BWD_WGRAD>, dim3(grid_for(tiles)), dim3(kBwdThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
