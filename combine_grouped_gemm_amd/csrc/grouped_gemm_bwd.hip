// Grouped GEMMs of the layer's backward pass ("DeepSeek MoE: EP and FSDP guide": the backward
// mirrors the forward and every expert keeps its own weight gradients; "MoE part 4" page,
// section 2: one launch over the experts' ragged row counts).
//
//   dgrad:  out[r, n] = sum_k dC[r, k] W_e[k, n]          r in segment e   (W_e [K, N], n contiguous)
//   wgrad:  dW_e[m, n] = sum_{r in segment e} A[r, m] B[r', n]              (r' = r, or gathered)
//
// The forward kernels read both operands with k contiguous.  Here one (dgrad: W_e) or both
// (wgrad: A and B, k being the row index) have k as the slow index.  Two kernels:
//
//   - the main one (namespace `wide` below): 128 x 256 tiles, direct-to-LDS loads of the
//     operands as they lie in memory, and gfx950's transposing LDS read to form the MFMA
//     fragments of the k-strided operands.  Used for N % 256 == 0 (and K % 32 == 0 for
//     dgrad), with B not gathered for wgrad: every GEMM of the bf16 layer's backward.
//   - a general one for the other shapes (N % 128 == 0, gathered B): 128 x 128 tiles whose
//     k-strided operands are transposed on their way into LDS (a lane loads 8 consecutive m
//     or n at one k and stores them into 8 LDS rows; rows padded from 64 to 80 bytes so that
//     the fragment reads hit distinct banks), K in stages of 32 double-buffered through
//     registers.
//
// Both deal logical tiles to the XCDs in contiguous ranges (workgroup i runs on XCD i mod
// 8): dgrad orders them expert -> n-block -> m-tile, so the m-tiles sharing a weight slice run
// together; wgrad expert -> m-block -> n-block, dealt in chunks of 32 tiles round-robin over
// the XCDs when the launch is large (a wgrad tile's cost grows with its expert's rows).
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
  int deal;                    // wide wgrad: tiles dealt to the XCDs in chunks of `deal` (0: ranges)
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

// ------------------------------------------------------------------------------------
// The main kernel: 128 x 256 tiles, K in stages of 32 through a three-slot ring of
// direct-to-LDS loads, and the k-strided operands read out of LDS transposed.
//
// An operand whose k index is contiguous in memory (dgrad's dC) lies in LDS as 128 rows of
// 32 k (64 bytes; 16-byte chunk c of row r in slot c ^ ((r >> 2) & 3)) and is read with one
// 16-byte LDS read per MFMA fragment.  An operand whose m or n index is contiguous (dgrad's
// W_e, both wgrad operands) lies in LDS as it lies in memory: 32 rows of k, each holding the
// tile's 128 or 256 columns (chunk c of k-row r in slot
// c ^ 4 (r & 3)).  Its MFMA fragment (one column, 8 consecutive k per lane) takes two
// ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives the (i % 4)-th 16-bit
// element of the 8 bytes that lane 4j + i / 4 of the group addresses, for j = 0..3.  So
// when source lane s addresses k-row k0 + s / 4 at column c0 + 4 (s % 4), lane i holds
// column c0 + i at k-rows k0 .. k0 + 3.
//
// Each of the 4 waves computes 64 tile rows x 128 columns (2 x 4 blocks of
// v_mfma_f32_32x32x16_bf16, the n-operand first, so a lane's accumulators hold one tile row
// and runs of 4 adjacent columns).  While stage ks is multiplied, stage ks+2 is loaded into
// the slot stage ks-1 used; at the end of stage ks each wave waits for its loads of stage
// ks+1 and the workgroup synchronises.  Each stage of each operand is read through a buffer
// window ending after the stage's last valid row, so wgrad rows past an expert's segment
// (and dgrad tile rows past the segment) load zeros and add nothing.
// ------------------------------------------------------------------------------------
namespace wide {

constexpr int kTN = 256;     // tile columns
constexpr int kKS = 32;      // k per stage
constexpr int kSlots = 3;

// A tile of TM rows (128: 4 waves, dgrad and wgrad; 256: 8 waves, wgrad) x 256 columns; a
// wave computes 64 rows x 128 columns.  A stage of 32 k is (TM + 256) x 64 bytes: 24 KB (two
// workgroups per CU) or 32 KB (one workgroup of 8 waves per CU).
template <int TM>
struct Cfg {
  static constexpr int kWM = TM / 64;                  // waves along the rows
  static constexpr int kWaves = 2 * kWM;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kABytes = TM * kKS * 2;
  static constexpr int kBBytes = kTN * kKS * 2;
  static constexpr int kStage = kABytes + kBBytes;
  static constexpr int kAOps = kABytes / 1024 / kWaves;   // 1 KB loads per wave and stage
  static constexpr int kBOps = kBBytes / 1024 / kWaves;
  static constexpr int kOps = kAOps + kBOps;
  static constexpr int kOcc = TM == 128 ? 2 : 1;         // workgroups per CU
  static_assert(kABytes % (1024 * kWaves) == 0 && kBBytes % (1024 * kWaves) == 0, "loads spread evenly");
};

// k-contiguous rows of 64 bytes: chunk c of row r in slot c ^ ((r >> 2) & 3) (a fragment read
// of 32 rows and a 16-row load both spread over the 64 banks)
__device__ __forceinline__ int kc_key(int r) { return (r >> 2) & 3; }
// k-rows of the strided operands: chunk c of k-row r in slot c ^ 4 (r & 3)
__device__ __forceinline__ int mc_key(int k) { return 4 * (k & 3); }

// A buffer resource over `bytes` bytes from `base` (raw, stride 0): a load whose offset lies
// past the end returns zeros instead of touching memory.
__device__ __forceinline__ u32x4_t buffer_window(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4_t{static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}

// 16 bytes per lane from byte `voff` of a buffer window into LDS at lds_base + 16 * lane
// (zeros for offsets past the window).  Inline assembly, like dma16, so that the compiler
// adds no wait of its own before later LDS reads; M0 holds the LDS base, one wait state
// after its write.
__device__ __forceinline__ void dma16_window(u32x4_t rsrc, uint32_t voff, uint32_t lds_base) {
  __asm__ volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(lds_base)
      : "memory", "m0");
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;

// Byte offset, inside a slot whose k-rows are `pitch` bytes long, of lane `lane`'s first
// transposing read for the MFMA fragment of tile columns col0 .. col0 + 31 at k-rows 0 .. 15:
// in each 16-lane group lane i reads 8 bytes (4 columns) of k-row 8 (g / 2) + i / 4.  The
// swizzle key of a k-row depends on k mod 4 only, so k-rows 16 s + 4 r further are the same
// offset plus (16 s + 4 r) pitch.
__device__ __forceinline__ uint32_t tr_off(int pitch, int col0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int row = 8 * (g >> 1) + (i >> 2);
  const int byte = (col0 + 16 * (g & 1) + 4 * (i & 3)) * 2;
  return static_cast<uint32_t>(row * pitch + ((((byte >> 4) ^ mc_key(row)) << 4) | (byte & 15)));
}

// MFMA fragment of a k-strided operand: two transposing reads at the lane's tr_off address
// (absolute LDS byte address `addr`), k-rows 16 s + 0..3 and 16 s + 4..7 of each group;
// lane l ends up with column col0 + l % 32, k-rows 16 s + 8 (l / 32) + 0..7
template <int kPitchBytes>
__device__ __forceinline__ uint4 tr_frag_at(uint32_t addr, int s) {
  uint2 h[2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
    h[r] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_v4i16*>(
                                         static_cast<uintptr_t>(addr + (16 * s + 4 * r) * kPitchBytes))));
  return make_uint4(h[0].x, h[0].y, h[1].x, h[1].y);
}

template <int MODE, int TM>
__global__ __launch_bounds__(Cfg<TM>::kThreads, Cfg<TM>::kOcc) void grouped_gemm_bwd_wide_kernel(BwdArgs p) {
  using C = Cfg<TM>;
  constexpr int kWaves = C::kWaves, kABytes = C::kABytes, kStage = C::kStage, kAOps = C::kAOps;
  constexpr int kOps = C::kOps, kThreads = C::kThreads;
  static_assert(MODE == BWD_WGRAD || TM == 128, "dgrad tiles have 128 rows");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kSlots * kStage];
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_byte*)lds));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- the tile
  const int nN = p.N / kTN;
  long long total;
  if (MODE == BWD_DGRAD) total = static_cast<long long>(p.tile_prefix[p.E]) * nN;
  else total = static_cast<long long>(p.E) * (p.M / TM) * nN;
  const int xcd = blockIdx.x % kNumXcd;
  const long long slot = blockIdx.x / kNumXcd;
  long long L;
  if (MODE == BWD_WGRAD && p.deal > 0) {
    // chunk c of `deal` consecutive tiles goes to XCD c mod 8: a tile's cost is its expert's
    // row count, so under skew a contiguous range per XCD would leave one XCD with the hot
    // expert's tiles; a chunk keeps the tiles that share operand slices together
    const long long chunks = (total + p.deal - 1) / p.deal;
    const long long per_xcd = (chunks + kNumXcd - 1) / kNumXcd * p.deal;
    if (slot >= per_xcd) return;
    L = ((slot / p.deal) * kNumXcd + xcd) * p.deal + slot % p.deal;
    if (L >= total) return;
  } else {
    const long long per_xcd = (total + kNumXcd - 1) / kNumXcd;
    L = xcd * per_xcd + slot;
    if (slot >= per_xcd || L >= total) return;
  }
  int e, m0, mcount, n0, klo, kcount;
  if (MODE == BWD_DGRAD) {
    // expert -> n-block -> m-tile: expert e owns logical tiles [prefix[e] nN, prefix[e+1] nN);
    // the last expert whose range starts at or before L (an empty expert's range is empty)
    int lo_e = 0, hi_e = p.E - 1;
    while (lo_e < hi_e) {
      const int mid = (lo_e + hi_e + 1) >> 1;
      if (static_cast<long long>(p.tile_prefix[mid]) * nN <= L) lo_e = mid;
      else hi_e = mid - 1;
    }
    e = lo_e;
    const int mt_e = p.tile_prefix[e + 1] - p.tile_prefix[e];
    const long long local = L - static_cast<long long>(p.tile_prefix[e]) * nN;
    int lo, hi;
    seg_of(p, e, lo, hi);
    m0 = lo + static_cast<int>(local % mt_e) * TM;
    mcount = hi - m0 < TM ? hi - m0 : TM;
    n0 = static_cast<int>(local / mt_e) * kTN;
    klo = 0;
    kcount = p.K;
  } else {
    const int mB = p.M / TM;
    e = static_cast<int>(L / (static_cast<long long>(mB) * nN));
    const int local = static_cast<int>(L - static_cast<long long>(e) * mB * nN);
    m0 = (local / nN) * TM;
    n0 = (local % nN) * kTN;
    mcount = TM;
    int lo, hi;
    seg_of(p, e, lo, hi);
    klo = lo;
    kcount = hi - lo;
  }
  const int nk = (kcount + kKS - 1) / kKS;

  // ---- loads.  Stage ks covers k-rows k0 = ks kKS .. k0 + 31 of both operands, each read
  // through a buffer window that starts at the stage's first element and ends after the
  // last valid row, so rows past the data (wgrad: past the segment; dgrad: tile rows past
  // mcount) load zeros.  Op j of a wave fills its operand's 1 KB group wave + kWaves j; the
  // lane's byte offset inside the window is fixed for the tile.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  uint32_t voff_a[kAOps], voff_b[C::kBOps];
#pragma unroll
  for (int j = 0; j < kAOps; ++j) {
    const int g = wave + kWaves * j;
    if (MODE == BWD_DGRAD) {   // 16 rows of 64 bytes
      const int r = 16 * g + (lane >> 2);
      const int c = (lane & 3) ^ kc_key(r);
      voff_a[j] = static_cast<uint32_t>(r * p.K * 2 + c * 16);
    } else {                   // 1024 / (2 TM) k-rows of 2 TM bytes
      constexpr int kPer = 1024 / (2 * TM), kCh = 2 * TM / 16;
      const int kr = kPer * g + lane / kCh;
      const int c = (lane % kCh) ^ mc_key(kr);
      voff_a[j] = static_cast<uint32_t>(kr * p.M * 2 + c * 16);
    }
  }
#pragma unroll
  for (int j = 0; j < C::kBOps; ++j) {   // 2 k-rows of 512 bytes (256 n)
    const int kr = 2 * (wave + kWaves * j) + (lane >> 5);
    const int c = (lane & 31) ^ mc_key(kr);
    voff_b[j] = static_cast<uint32_t>(kr * p.N * 2 + c * 16);
  }
  auto windows = [&](int ks, u32x4_t& wa, u32x4_t& wb) __attribute__((always_inline)) {
    const int k0 = ks * kKS;
    if (MODE == BWD_DGRAD) {
      wa = buffer_window(p.a + (static_cast<size_t>(m0) * p.K + k0),
                         static_cast<uint32_t>(mcount - 1) * p.K * 2 + 2 * kKS);
      wb = buffer_window(p.b + ((static_cast<size_t>(e) * p.K + k0) * p.N + n0),
                         static_cast<uint32_t>(kKS - 1) * p.N * 2 + 2 * kTN);
    } else {
      const int left = kcount - k0 < kKS ? kcount - k0 : kKS;
      wa = buffer_window(p.a + (static_cast<size_t>(klo + k0) * p.M + m0),
                         static_cast<uint32_t>(left - 1) * p.M * 2 + 2 * TM);
      wb = buffer_window(p.b + (static_cast<size_t>(klo + k0) * p.N + n0),
                         static_cast<uint32_t>(left - 1) * p.N * 2 + 2 * kTN);
    }
  };
  auto issue = [&](const u32x4_t& wa, const u32x4_t& wb, int sl, int j) __attribute__((always_inline)) {
    const uint32_t base = lds0 + sl * kStage;
    if (j < kAOps) dma16_window(wa, voff_a[j], base + (wave_u + kWaves * j) * 1024);
    else dma16_window(wb, voff_b[j - kAOps], base + kABytes + (wave_u + kWaves * (j - kAOps)) * 1024);
  };

  // ---- fragment reads: per-lane byte offsets inside a slot, fixed for the tile
  uint32_t fo_a[2], fo_b[4];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    if (MODE == BWD_DGRAD) {   // x = s: row wm 64 + l % 32 (+ 32 i), 16-byte chunk 2 s + l / 32
      const int row = wm * 64 + (lane & 31);
      fo_a[x] = static_cast<uint32_t>(row * (2 * kKS) + (((2 * x + (lane >> 5)) ^ kc_key(row)) << 4));
    } else {                   // x = i: columns wm 64 + 32 i
      fo_a[x] = tr_off(TM * 2, wm * 64 + x * 32, lane);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) fo_b[j] = kABytes + tr_off(kTN * 2, wn * 128 + j * 32, lane);

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

  if (nk > 0) {
    u32x4_t wa, wb;
    windows(0, wa, wb);
#pragma unroll
    for (int j = 0; j < kOps; ++j) issue(wa, wb, 0, j);
    if (nk > 1) {
      windows(1, wa, wb);
#pragma unroll
      for (int j = 0; j < kOps; ++j) issue(wa, wb, 1, j);
      wait_vmcnt<kOps>();
    } else {
      wait_vmcnt<0>();
    }
    block_barrier();
    int sl = 0, sl2 = 2;   // ring slots of stages ks and ks + 2
    for (int ks = 0; ks < nk; ++ks) {
      if (ks + 2 < nk) {
        windows(ks + 2, wa, wb);
#pragma unroll
        for (int j = 0; j < kOps; ++j) issue(wa, wb, sl2, j);
      }
      const uint32_t sbase = lds0 + sl * kStage;
      uint32_t ra[2], rb[4];
#pragma unroll
      for (int x = 0; x < 2; ++x) ra[x] = sbase + fo_a[x];
#pragma unroll
      for (int j = 0; j < 4; ++j) rb[j] = sbase + fo_b[j];
#pragma unroll
      for (int s = 0; s < kKS / 16; ++s) {
        uint4 fa[2], fb[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (MODE == BWD_DGRAD)
            fa[i] = __builtin_bit_cast(
                uint4, *reinterpret_cast<lds_u32x4*>(static_cast<uintptr_t>(ra[s] + i * 32 * (2 * kKS))));
          else
            fa[i] = tr_frag_at<TM * 2>(ra[i], s);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[j] = tr_frag_at<kTN * 2>(rb[j], s);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mma_bf16(fb[j], fa[i], acc[i][j]);
      }
      if (ks + 1 < nk) {
        wait_lgkmcnt_all();
        if (ks + 2 < nk) wait_vmcnt<kOps>();
        else wait_vmcnt<0>();
        block_barrier();
      }
      sl = sl + 1 == kSlots ? 0 : sl + 1;
      sl2 = sl2 + 1 == kSlots ? 0 : sl2 + 1;
    }
  }

  // ---- epilogue: lane l holds tile row wm*64 + i*32 + l % 32 and, in registers 4q .. 4q+3
  // of block j, columns wn*128 + j*32 + 8q + 4 (l / 32) + 0..3.  bf16 tiles go through LDS
  // 128 rows at a time (16-byte chunk c of row r in slot c ^ (r % 32), its two 8-byte halves
  // swapped when r % 32 >= 16, so that the 32 rows one write instruction covers hit distinct
  // banks), and each store instruction writes whole 512-byte rows; fp32 tiles are stored
  // from the registers.
  const bool staged = MODE == BWD_DGRAD || !p.out_f32;
  if (staged) {
    static_assert(128 * kTN * 2 <= kSlots * kStage, "128 rows of a bf16 tile fit the ring");
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
    const size_t row0 = MODE == BWD_DGRAD ? static_cast<size_t>(m0) : static_cast<size_t>(e) * p.M + m0;
#pragma unroll
    for (int half = 0; half < TM / 128; ++half) {
      wait_lgkmcnt_all();
      block_barrier();   // every wave is past its last fragment reads (or the previous half's stores)
      if ((wm >> 1) == half) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = (wm & 1) * 64 + i * 32 + (lane & 31);   // row within the half
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int col = wn * 128 + j * 32 + 8 * q + 4 * (lane >> 5);
              const int chunk = (col >> 3) ^ (r & 31);
              const int half = ((col & 7) >> 2) ^ ((r >> 4) & 1);
              const f32x16_t& a = acc[i][j];
              *reinterpret_cast<uint2*>(lds + r * (kTN * 2) + chunk * 16 + half * 8) =
                  make_uint2(pack_bf16x2(a[4 * q], a[4 * q + 1]), pack_bf16x2(a[4 * q + 2], a[4 * q + 3]));
            }
        }
      }
      wait_lgkmcnt_all();
      block_barrier();
      // each thread takes 16-byte chunk tid % 32 of rows kRpt t + tid / 32: all its LDS reads
      // first (the chunk's slot is (tid % 32) ^ (row % 32), and row % 32 = (kRpt t) % 32 +
      // tid / 32, so a few per-lane bases serve every t), then the stores; weight gradients
      // are not read again by the step, so they bypass the caches (non-temporal stores)
      constexpr int kT = 128 * kTN * 2 / 16 / kThreads;
      constexpr int kRpt = kThreads / 32;
      const int w = tid >> 5, ch = tid & 31;
      uint32_t rbase[32 / kRpt];
#pragma unroll
      for (int q = 0; q < 32 / kRpt; ++q)
        rbase[q] = lds0 + static_cast<uint32_t>(w * (kTN * 2) + (((ch ^ w) ^ (q * kRpt)) << 4));
      uint4 v[kT];
#pragma unroll
      for (int t = 0; t < kT; ++t)
        v[t] = __builtin_bit_cast(uint4, *reinterpret_cast<lds_u32x4*>(static_cast<uintptr_t>(
                                             rbase[((t * kRpt) & 31) / kRpt] + t * kRpt * (kTN * 2))));
      uint16_t* o = out + (row0 + half * 128 + w) * p.N + n0 + ch * 8;
#pragma unroll
      for (int t = 0; t < kT; ++t) {
        if (MODE == BWD_DGRAD && half * 128 + kRpt * t + w >= mcount) continue;
        uint4 x = v[t];
        if (((t * kRpt) >> 4) & 1) x = make_uint4(x.z, x.w, x.x, x.y);   // the row's halves were swapped
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(o + static_cast<size_t>(t) * kRpt * p.N);
        if (MODE == BWD_WGRAD) __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, x), dst);
        else *dst = __builtin_bit_cast(u32x4_t, x);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wm * 64 + i * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + wn * 128 + j * 32 + 8 * q + 4 * (lane >> 5);
          const f32x16_t& a = acc[i][j];
          const size_t o = (static_cast<size_t>(e) * p.M + m0 + r) * p.N + col;
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + o) =
              make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
        }
    }
  }
}

}  // namespace wide


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
  const dim3 wgrid(grid_for(static_cast<long long>(cap) * (N / wide::kTN)));
  // (the tile kernel's per-lane window offsets are 32-bit: up to 128 rows of K and 32 k-rows
  // of N elements)
  if (N % wide::kTN == 0 && K % wide::kKS == 0 && K <= (1 << 22) && N <= (1 << 22))
    hipLaunchKernelGGL((wide::grouped_gemm_bwd_wide_kernel<BWD_DGRAD, 128>), wgrid, dim3(wide::Cfg<128>::kThreads), 0,
                       s, p);
  else
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
  // (256-row tiles of 8 waves, one workgroup per CU, measured 20-30% slower on the
  // DeepSeek-V3 weight gradients: with ~256 rows of K per expert a tile is 8 stages, and a
  // second workgroup on the CU hides one tile's first loads and last stores behind the
  // other's multiplies)
  if (b_rows == nullptr && N % wide::kTN == 0 && M <= (1 << 22) && N <= (1 << 22)) {
    const long long tiles = static_cast<long long>(E) * (M / 128) * (N / wide::kTN);
    // chunks of 32 tiles dealt round-robin to the XCDs once each XCD gets 8 or more chunks
    // (the DeepSeek-V3 weight gradients under a Zipf skew: dW13 11.3 -> 6.5 ms; uniform
    // routing within 3%); small launches (a shared expert's) keep contiguous ranges
    p.deal = tiles >= 32LL * 8 * kNumXcd ? 32 : 0;
    const unsigned grid =
        p.deal > 0 ? static_cast<unsigned>(((tiles + p.deal - 1) / p.deal + kNumXcd - 1) / kNumXcd * p.deal * kNumXcd)
                   : grid_for(tiles);
    hipLaunchKernelGGL((wide::grouped_gemm_bwd_wide_kernel<BWD_WGRAD, 128>), dim3(grid),
                       dim3(wide::Cfg<128>::kThreads), 0, s, p);
  } else {
    const long long tiles = static_cast<long long>(E) * (M / kBT) * (N / kBT);
    hipLaunchKernelGGL(grouped_gemm_bwd_kernel<BWD_WGRAD>, dim3(grid_for(tiles)), dim3(kBwdThreads), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace moe
