// Grouped expert GEMMs on CDNA4 matrix cores ("MoE part 4" page, section 2: one launch
// for many expert GEMMs with differing row counts n_e; section 4.1: FC1 -> activation ->
// FC2, here SwiGLU).
//
//   gate/up:  h[r, :]   = silu(a[r] . W_gate,e^T) * (a[r] . W_up,e^T)   for r in segment e
//   down:     out[r, :] = h[r] . W_down,e^T
//
// Operands are K-contiguous (a [rows, K], weights [n, K]), so both MFMA operands are
// 16-byte row fragments.  A workgroup (4 waves, 2 x 2) computes a 128-row x 256-column
// tile; each wave owns 64 x 128 (2 x 4 blocks of v_mfma_f32_32x32x16 for bf16 and fp8,
// v_mfma_f32_32x32x2 for fp32), so every 16-wide K step reads 6 fragments from LDS for 8
// MFMAs.  K advances in 128-byte stages: two stages of global loads are in flight in
// registers while the current stage, double-buffered in padded LDS, is multiplied.
//
// The gate/up tile takes 128 rows of W_gate and the same 128 rows of W_up, so each wave
// holds matching gate and up accumulators and applies SwiGLU in registers; h is written
// once.
//
// Tile schedule: a one-workgroup prologue turns offsets into a per-expert m-tile prefix.
// The GEMM is persistent (one workgroup per CU): the logical tiles are ordered expert ->
// n-block -> m-tile (the m-tiles sharing a weight block are adjacent) and split into 8
// contiguous ranges, one per XCD (workgroup i runs on XCD i mod 8), so tiles that share
// weights and activation rows run together under one L2.  Every tile costs the same
// whatever the skew of n_e, so ragged and hot experts spread evenly over the CUs.
//
// fp8 layers: the gate/up GEMM multiplies e4m3 codes on the fp8 MFMA, sums each 128-wide
// K block in a separate fp32 accumulator and adds it scaled by a_scale[row] *
// w_scale[col]; the down GEMM dequantizes e4m3 W_down on its way to LDS (code times its
// 128-column block's scale, rounded once to bf16, as a bf16 weight is stored) and multiplies
// it against bf16 h like a bf16 weight.
#include <type_traits>
#include <utility>

#include "gemm_device.h"
#include "grouped_gemm.h"
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {



constexpr int GBM = 128;          // rows of a tile
constexpr int GBN = 256;          // weight rows of a tile (gate/up: 128 gate + 128 up)
constexpr int GKB = 128;          // bytes of K per row and stage (compute type)
constexpr int GPITCH = GKB + 16;  // padded LDS row pitch: 8 consecutive rows hit 8 bank groups
constexpr int GTHREADS = 256;
constexpr int kAChunks = GBM * (GKB / 16) / GTHREADS;  // 16-byte A chunks per thread and stage (4)
constexpr int kBChunks = GBN * (GKB / 16) / GTHREADS;  // B chunks per thread and stage (8)

template <int CT> struct CTraits;
template <> struct CTraits<CT_F32> { static constexpr int esz = 4; };
template <> struct CTraits<CT_BF16> { static constexpr int esz = 2; };
template <> struct CTraits<CT_FP8> { static constexpr int esz = 1; };

// inclusive prefix sum over the 1024 threads of the block
__device__ int32_t block_scan_1024(int32_t x, int32_t* tot) {
  const int e = threadIdx.x;
  __syncthreads();
  tot[e] = x;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = e >= off ? tot[e - off] : 0;
    __syncthreads();
    tot[e] += v;
    __syncthreads();
  }
  return tot[e];
}

// Tile schedule prologue: m-tiles (of tile_rows rows) of each expert, their prefix and the
// m-tile -> expert table.  Offsets are clamped into [0, rows] so malformed input cannot
// index out of range.  With shared_rows > 0 a last segment E of shared_rows rows (the
// shared expert) follows, and prefix has E + 2 entries.  With tall_list, the routed experts
// of tile_rows < n_e <= tall_rows get no m-tiles and are listed instead (tall_list[0] = their
// count, then the experts in order), and tall_list[E + 1 ..] holds kNumXcd zeroed counters.
// tile_counter: n_counters zeroed counters (one per XCD, and the wide kernel's shared tail).
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets, int E,
                                                           int rows, int tile_rows, int tile_cap,
                                                           int32_t* __restrict__ prefix,
                                                           int32_t* __restrict__ tile_expert,
                                                           int32_t* __restrict__ tile_counter,
                                                           int shared_rows, int tall_rows,
                                                           int32_t* __restrict__ tall_list, int n_counters) {
  __shared__ int32_t tot[1024];
  const int e = threadIdx.x;
  const int n_seg = E + (shared_rows > 0 ? 1 : 0);
  int mt = 0, tall = 0;
  if (e < E) {
    int lo = offsets[e], hi = offsets[e + 1];
    lo = lo < 0 ? 0 : (lo > rows ? rows : lo);
    hi = hi < lo ? lo : (hi > rows ? rows : hi);
    tall = tall_list != nullptr && hi - lo > tile_rows && hi - lo <= tall_rows ? 1 : 0;
    mt = tall ? 0 : (hi - lo + tile_rows - 1) / tile_rows;
  } else if (e < n_seg) {
    mt = (shared_rows + tile_rows - 1) / tile_rows;
  }
  const int32_t end = block_scan_1024(mt, tot);
  const int start = end - mt;
  if (e < n_seg) {
    prefix[e] = start < tile_cap ? start : tile_cap;
    for (int i = 0; i < mt && start + i < tile_cap; ++i) tile_expert[start + i] = e;
  }
  if (e == n_seg - 1) prefix[n_seg] = end < tile_cap ? end : tile_cap;
  if (e < n_counters) tile_counter[e] = 0;
  if (tall_list != nullptr) {
    const int32_t tend = block_scan_1024(tall, tot);
    if (tall) tall_list[tend] = e;
    if (e == 1023) tall_list[0] = tend;
    if (e < kNumXcd) tall_list[E + 1 + e] = 0;
  }
}

template <int CT>
struct Frag;
template <>
struct Frag<CT_BF16> {
  uint4 v;
  __device__ __forceinline__ void load(const uint8_t* p) { v = *reinterpret_cast<const uint4*>(p); }
};
template <>
struct Frag<CT_FP8> {
  uint2 v;
  __device__ __forceinline__ void load(const uint8_t* p) { v = *reinterpret_cast<const uint2*>(p); }
};
template <>
struct Frag<CT_F32> {
  uint4 v0, v1;
  __device__ __forceinline__ void load(const uint8_t* p) {
    v0 = reinterpret_cast<const uint4*>(p)[0];
    v1 = reinterpret_cast<const uint4*>(p)[1];
  }
};

__device__ __forceinline__ f32x16_t mma(const Frag<CT_BF16>& a, const Frag<CT_BF16>& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a.v),
                                                 __builtin_bit_cast(bf16x8_t, b.v), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mma(const Frag<CT_FP8>& a, const Frag<CT_FP8>& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(__builtin_bit_cast(long, a.v),
                                                    __builtin_bit_cast(long, b.v), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mma(const Frag<CT_F32>& a, const Frag<CT_F32>& b, f32x16_t c) {
  // lanes 0-31 supply k = s and lanes 32-63 k = 8 + s of the 16-wide step; the same
  // assignment on both operands makes the 8 products sum over all 16 k.
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.v0.x), __uint_as_float(b.v0.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.v0.y), __uint_as_float(b.v0.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.v0.z), __uint_as_float(b.v0.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.v0.w), __uint_as_float(b.v0.w), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.v1.x), __uint_as_float(b.v1.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.v1.y), __uint_as_float(b.v1.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.v1.z), __uint_as_float(b.v1.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.v1.w), __uint_as_float(b.v1.w), c, 0, 0, 0);
  return c;
}

// Weight row of tile row `row` (0..GBN-1).
template <int MODE>
__device__ __forceinline__ long long weight_row(int row, int nblk, int I, int n_out) {
  if (MODE == MODE_GATE_UP)
    return row < GBN / 2 ? static_cast<long long>(nblk) * (GBN / 2) + row
                         : I + static_cast<long long>(nblk) * (GBN / 2) + (row - GBN / 2);
  long long r = static_cast<long long>(nblk) * GBN + row;
  return r < n_out ? r : n_out - 1;
}

template <int CT, bool B8, int MODE>
__global__ __launch_bounds__(GTHREADS, 1) void grouped_gemm_kernel(GemmArgs p) {
  constexpr int esz = CTraits<CT>::esz;
  constexpr int BK = GKB / esz;                 // K elements per stage
  constexpr int KSTEPS = BK / 16;               // 16-wide MFMA steps per stage
  constexpr bool kScaled = CT == CT_FP8;   // per-block scales on both operands: a second accumulator
  constexpr int kStagesPerBlock = 128 / BK;     // stages per 128-wide scale block
  constexpr int kAStage = GBM * GPITCH;
  constexpr int kBStage = GBN * GPITCH;
  constexpr int kBGlobal = B8 ? 8 : 16;         // global bytes per B chunk

  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][kAStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][kBStage];
  __shared__ float lds_sa[2][GBM];
  __shared__ float lds_sb[2][GBN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int t_row = tid >> 3;        // tile row of chunk 0 (chunk i: + 32 i)
  const int t_c = tid & 7;           // 16-byte column chunk

  const int nN = MODE == MODE_GATE_UP ? p.I / (GBN / 2) : (p.n_out + GBN - 1) / GBN;
  const long long total = static_cast<long long>(p.tile_prefix[p.E]) * nN;
  const int xcd = blockIdx.x % kNumXcd;
  const int slot = blockIdx.x / kNumXcd;
  const int per_xcd = gridDim.x / kNumXcd;
  const long long t_beg = total * xcd / kNumXcd;
  const long long t_end = total * (xcd + 1) / kNumXcd;

  const int nk = p.K / BK;
  const uint32_t a_rb = static_cast<uint32_t>(p.K) * esz;            // A row bytes
  const uint32_t b_rb = static_cast<uint32_t>(p.K) * (B8 ? 1 : esz);  // B row bytes
  const int kblocks = p.K / 128;

  // LDS offsets (bytes within a stage buffer)
  const int frag_k = (lane >> 5) * 8 * esz;
  const int a_frag = (wm * 64 + (lane & 31)) * GPITCH + frag_k;            // + mb * 32 rows
  const int b_frag = MODE == MODE_GATE_UP ? (wn * 64 + (lane & 31)) * GPITCH + frag_k   // + (nb>>1)*128 + (nb&1)*32 rows
                                          : (wn * 128 + (lane & 31)) * GPITCH + frag_k; // + nb * 32 rows
  const int st_off = t_row * GPITCH + t_c * 16;                            // + i * 32 rows

  for (long long L = t_beg + slot; L < t_end; L += per_xcd) {
    // ---- decode the logical tile: expert -> n-block -> m-tile
    const int e = p.tile_expert[L / nN];
    const int pe = p.tile_prefix[e];
    const int mt_e = p.tile_prefix[e + 1] - pe;
    const long long local = L - static_cast<long long>(pe) * nN;
    const int nblk = static_cast<int>(local / mt_e);
    const int mtile = static_cast<int>(local % mt_e);
    int seg_lo = p.offsets[e], seg_hi = p.offsets[e + 1];
    seg_lo = seg_lo < 0 ? 0 : (seg_lo > p.rows ? p.rows : seg_lo);
    seg_hi = seg_hi < seg_lo ? seg_lo : (seg_hi > p.rows ? p.rows : seg_hi);
    const int m0 = seg_lo + mtile * GBM;
    const int mlast = seg_hi - 1 - m0;   // last valid tile row (rows past it re-read it)

    // uniform tile bases; per-chunk offsets are 32-bit
    const uint8_t* a_tile = p.a + static_cast<size_t>(m0) * a_rb;
    const long long b_row0 = MODE == MODE_GATE_UP ? static_cast<long long>(nblk) * (GBN / 2)
                                                  : static_cast<long long>(nblk) * GBN;
    const uint8_t* b_tile = p.b + (static_cast<size_t>(e) * p.b_rows + b_row0) * b_rb;
    const int b_rows_left = MODE == MODE_GATE_UP ? GBN : static_cast<int>(p.n_out - b_row0);  // valid B tile rows
    const float* sa_tile = CT == CT_FP8 ? p.a_scale + static_cast<size_t>(m0) * kblocks : nullptr;
    const float* sb_tile =
        kScaled || B8 ? p.b_scale + (static_cast<size_t>(e) * p.b_rows + b_row0) * kblocks : nullptr;

    struct Regs {
      uint4 a[kAChunks];
      uint4 b[kBChunks];
      uint2 b8[kBChunks];
      float s8[kBChunks];   // (B8) the scale of each e4m3 chunk's row and K block
      float sa, sb;
    };

    auto b_tile_row = [&](int r) __attribute__((always_inline)) -> uint32_t {
      // weight row (relative to b_row0) of tile row r
      if (MODE == MODE_GATE_UP) return r < GBN / 2 ? r : static_cast<uint32_t>(p.I) + (r - GBN / 2);
      return r < b_rows_left ? r : b_rows_left - 1;
    };

    auto issue = [&](Regs& r, int ks) __attribute__((always_inline)) {
      const uint8_t* ab = a_tile + static_cast<size_t>(ks) * GKB;
#pragma unroll
      for (int i = 0; i < kAChunks; ++i) {
        int row = t_row + 32 * i;
        row = row < mlast ? row : mlast;
        r.a[i] = *reinterpret_cast<const uint4*>(ab + (static_cast<uint32_t>(row) * a_rb + t_c * 16));
      }
      const uint8_t* bb = b_tile + static_cast<size_t>(ks) * (B8 ? BK : GKB);
#pragma unroll
      for (int i = 0; i < kBChunks; ++i) {
        const uint32_t off = b_tile_row(t_row + 32 * i) * b_rb + t_c * kBGlobal;
        if (B8) r.b8[i] = *reinterpret_cast<const uint2*>(bb + off);
        else r.b[i] = *reinterpret_cast<const uint4*>(bb + off);
      }
      if (B8) {
        const int kb = (ks * BK) / 128;
#pragma unroll
        for (int i = 0; i < kBChunks; ++i) r.s8[i] = sb_tile[static_cast<size_t>(b_tile_row(t_row + 32 * i)) * kblocks + kb];
      }
      if (kScaled) {
        const int kb = (ks * BK) / 128;
        r.sa = 1.0f;
        if (CT == CT_FP8 && tid < GBM) r.sa = sa_tile[static_cast<size_t>(tid < mlast ? tid : mlast) * kblocks + kb];
        r.sb = sb_tile[static_cast<size_t>(b_tile_row(tid)) * kblocks + kb];
      }
    };
    auto commit = [&](Regs& r, int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < kAChunks; ++i) *reinterpret_cast<uint4*>(&lds_a[buf][st_off + i * 32 * GPITCH]) = r.a[i];
#pragma unroll
      for (int i = 0; i < kBChunks; ++i) {
        uint4 v;
        if (B8) {
          const uint2 lo = e4m3x4_scaled_to_bf16x4(r.b8[i].x, r.s8[i]), hi = e4m3x4_scaled_to_bf16x4(r.b8[i].y, r.s8[i]);
          v = make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else {
          v = r.b[i];
        }
        *reinterpret_cast<uint4*>(&lds_b[buf][st_off + i * 32 * GPITCH]) = v;
      }
      if (kScaled) {
        if (tid < GBM) lds_sa[buf][tid] = r.sa;
        lds_sb[buf][tid] = r.sb;
      }
    };

    f32x16_t acc[2][4];
    f32x16_t part[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = f32x16_t{};
        if (kScaled) part[i][j] = f32x16_t{};
      }

    auto b_frag_row = [](int nb) constexpr -> int {
      return MODE == MODE_GATE_UP ? (nb >> 1) * (GBN / 2) + (nb & 1) * 32 : nb * 32;
    };
    auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        Frag<CT> fa[2], fb[4];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) fa[mb].load(&lds_a[buf][a_frag + mb * 32 * GPITCH + s * 16 * esz]);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) fb[nb].load(&lds_b[buf][b_frag + b_frag_row(nb) * GPITCH + s * 16 * esz]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            if (kScaled)
              part[mb][nb] = mma(fa[mb], fb[nb], part[mb][nb]);
            else
              acc[mb][nb] = mma(fa[mb], fb[nb], acc[mb][nb]);
          }
      }
    };
    auto apply_scales = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int brow = (MODE == MODE_GATE_UP ? wn * 64 : wn * 128) + b_frag_row(nb);
        const float sb = lds_sb[buf][brow + (lane & 31)];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            float sc = sb;
            if (CT == CT_FP8) sc = lds_sa[buf][wm * 64 + mb * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)] * sb;
            acc[mb][nb][v] += part[mb][nb][v] * sc;
            part[mb][nb][v] = 0.0f;
          }
        }
      }
    };

    __syncthreads();  // the previous tile's last reads of both LDS buffers are done
    if (!kScaled) {
      // two stages of global loads in flight: stage ks in LDS buffer ks & 1, stages ks+1
      // and ks+2 in registers
      Regs r0, r1;
      issue(r0, 0);
      if (nk > 1) issue(r1, 1);
      commit(r0, 0);
      __syncthreads();
      for (int ks = 0; ks < nk; ks += 2) {
        if (ks + 2 < nk) issue(r0, ks + 2);
        compute(0);
        if (ks + 1 < nk) commit(r1, 1);
        __syncthreads();
        if (ks + 1 >= nk) break;
        if (ks + 3 < nk) issue(r1, ks + 3);
        compute(1);
        if (ks + 2 < nk) commit(r0, 0);
        __syncthreads();
      }
    } else {
      // one stage in flight (the scaled variants hold a second set of accumulators)
      Regs r0;
      issue(r0, 0);
      commit(r0, 0);
      __syncthreads();
      for (int ks = 0; ks < nk; ++ks) {
        const int cur = ks & 1;
        if (ks + 1 < nk) issue(r0, ks + 1);
        compute(cur);
        if ((ks + 1) % kStagesPerBlock == 0) apply_scales(cur);
        if (ks + 1 < nk) commit(r0, cur ^ 1);
        __syncthreads();
      }
    }

    // ---- epilogue
    const int mend = seg_hi;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = m0 + wm * 64 + mb * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (r >= mend) continue;
        if (MODE == MODE_GATE_UP) {
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const float g = acc[mb][nb][v];
            const float u = acc[mb][nb + 2][v];
            const float hv = silu_f32(g) * u;
            const size_t o = static_cast<size_t>(r) * p.I + static_cast<size_t>(nblk) * (GBN / 2) + wn * 64 +
                             nb * 32 + (lane & 31);
            if (p.out_f32) reinterpret_cast<float*>(p.out)[o] = hv;
            else reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_bf16(hv);
          }
        } else {
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const int col = nblk * GBN + wn * 128 + nb * 32 + (lane & 31);
            if (col >= p.n_out) continue;
            const size_t o = static_cast<size_t>(r) * p.n_out + col;
            if (p.out_f32) reinterpret_cast<float*>(p.out)[o] = acc[mb][nb][v];
            else reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_bf16(acc[mb][nb][v]);
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// Unscaled bf16 variant with direct-to-LDS loads.
//
// A workgroup of WM x 4 waves computes a 128-row x BN-column tile (gate/up: BN/2 W_gate
// rows + the same BN/2 W_up rows -> BN/2 h columns); each wave owns 128/WM x BN/4 on
// v_mfma_f32_32x32x16_bf16.  K advances in stages of ROWB bytes per row;
// global_load_lds_dwordx4 writes each lane's 16 bytes straight into LDS at
// base + 16 * lane, so a stage needs no staging registers.  One wave instruction fills a
// 1 KiB group of 1024/ROWB tile rows.  Inside a row the 16-byte chunk c sits in slot
// c ^ key(r): the LDS serves a 16-byte-per-lane read 16 lanes at a time from 64 four-byte
// banks, and the key makes any 16 consecutive rows of one chunk land in 16 distinct
// 16-byte bank slots.  Stage waits are explicit (s_waitcnt vmcnt) followed by a plain
// s_barrier, which keeps the later stages in flight across the barrier.
// ------------------------------------------------------------------------------------

constexpr int kDmaOcc = 1;   // workgroups per CU


constexpr int kDM = 128;    // rows of a tile
constexpr int kDGroup = 1024;                           // bytes of one DMA wave instruction
template <int BN, int ROWB, int STAGES, int WM, int WN>
struct DmaCfg {
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kRowsPerGroup = kDGroup / ROWB;
  static constexpr int kChunks = ROWB / 16;             // 16-byte chunks per row and stage
  static constexpr int kAGroups = kDM / kRowsPerGroup;
  static constexpr int kBGroups = BN / kRowsPerGroup;
  static constexpr int kStageBytes = (kAGroups + kBGroups) * kDGroup;
  static constexpr int kPerWave = (kAGroups + kBGroups) / kWaves;   // DMA instructions per wave and stage
  static constexpr int kAPerWave = kAGroups / kWaves;
  static constexpr int kKSteps = ROWB / 32;             // 16-wide bf16 k-steps per stage
  static constexpr int kNB = BN / WN / 32;              // 32-column blocks per wave
  static constexpr int kMB = kDM / WM / 32;             // 32-row blocks per wave
  static_assert(kAGroups % kWaves == 0 && kBGroups % kWaves == 0, "groups spread evenly");
  static_assert(ROWB != 128 || kWaves % 2 == 0, "the 128-byte swizzle needs the group parity of the wave");
  static_assert(STAGES * kStageBytes <= 160 * 1024, "LDS");
  // swizzle key of tile row r (rows of a fragment start at multiples of 32)
  __device__ static __forceinline__ int key(int r) {
    return ROWB == 128 ? ((r & 7) ^ ((r >> 3) & 1)) : ((r >> 2) & 3);
  }
};

template <int MODE, int BN, int ROWB, int STAGES, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64, kDmaOcc) void grouped_gemm_dma_kernel(GemmArgs p) {
  using C = DmaCfg<BN, ROWB, STAGES, WM, WN>;
  constexpr int KSTEPS = C::kKSteps;
  constexpr int NB = C::kNB;
  constexpr int MB = C::kMB;
  constexpr int kDmaWaves = C::kWaves;
  constexpr int PER = C::kPerWave;
  static_assert(KSTEPS % 2 == 0, "a stage must end in fragment set 1 so the next starts in set 0");
  static_assert(MODE != MODE_GATE_UP || NB % 2 == 0, "gate/up pairs");

  static_assert(STAGES * C::kStageBytes * kDmaOcc <= 160 * 1024, "LDS of the resident workgroups");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[STAGES * C::kStageBytes];
  const uint32_t lds_addr0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_byte*)lds));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // each wave owns MB 32-row blocks x BN/WN columns of the tile.  Row blocks are dealt to
  // the WM row waves in turn (wave wm takes blocks wm, wm + WM, ...), so a ragged tile
  // still spreads its rows evenly over the SIMDs.
  const int wm = wave / WN, wn = wave % WN;
  const int lrow = lane / C::kChunks;           // row inside a DMA group
  // global chunk this lane loads: the slot it fills is lane % kChunks, XOR the row's key.
  // Every group this wave fills has the parity of the wave (groups w, w + waves, ...; 16 A
  // groups of 8 rows precede the B groups), which the 128-byte key needs for bit 3 of the row.
  const int lchunk = (lane % C::kChunks) ^ C::key(lrow + (ROWB == 128 ? (wave & 1) * 8 : 0));

  const int n_cols = MODE == MODE_GATE_UP ? p.I : p.n_out;
  const int tile_cols = MODE == MODE_GATE_UP ? BN / 2 : BN;
  const int nN = (n_cols + tile_cols - 1) / tile_cols;
  const long long total = static_cast<long long>(p.tile_prefix[p.E]) * nN;
  const int xcd = blockIdx.x % kNumXcd;
  const int slot = blockIdx.x / kNumXcd;
  const int per_xcd = gridDim.x / kNumXcd;
  const long long t_beg = total * xcd / kNumXcd;
  const long long t_end = total * (xcd + 1) / kNumXcd;

  const int nk = p.K / (ROWB / 2);
  const uint32_t rb = static_cast<uint32_t>(p.K) * 2;   // row bytes of both operands

  const int key = C::key(lane & 31);
  const int h = lane >> 5;
  int koff[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) koff[s] = ((2 * s + h) ^ key) * 16;
  int a_frag[MB], b_frag[NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) a_frag[mb] = ((mb * WM + wm) * 32 + (lane & 31)) * ROWB;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    // gate/up: the first NB/2 blocks are W_gate rows, the last NB/2 the same W_up rows
    const int r = MODE == MODE_GATE_UP
                      ? (nb / (NB / 2)) * (BN / 2) + wn * (BN / (2 * WN)) + (nb % (NB / 2)) * 32 + (lane & 31)
                      : wn * (BN / WN) + nb * 32 + (lane & 31);
    b_frag[nb] = C::kAGroups * kDGroup + r * ROWB;
  }

  for (long long L = t_beg + slot; L < t_end; L += per_xcd) {
    const int e = p.tile_expert[L / nN];
    const int pe = p.tile_prefix[e];
    const int mt_e = p.tile_prefix[e + 1] - pe;
    const long long local = L - static_cast<long long>(pe) * nN;
    const int nblk = static_cast<int>(local / mt_e);
    const int mtile = static_cast<int>(local % mt_e);
    int seg_lo = p.offsets[e], seg_hi = p.offsets[e + 1];
    seg_lo = seg_lo < 0 ? 0 : (seg_lo > p.rows ? p.rows : seg_lo);
    seg_hi = seg_hi < seg_lo ? seg_lo : (seg_hi > p.rows ? p.rows : seg_hi);
    // the expert's rows are split into mt_e tiles of equal size (a multiple of 32 rows):
    // the tiles that share a weight panel do equal work and stream it together, which
    // keeps more of the panel's second and third reads in L2
    const int rpt = ((seg_hi - seg_lo + mt_e - 1) / mt_e + 31) / 32 * 32;
    const int m0 = seg_lo + mtile * rpt;
    const int mend = m0 + rpt < seg_hi ? m0 + rpt : seg_hi;
    const int mlast = mend - 1 - m0;
    const int c0 = nblk * tile_cols;
    const int clast = n_cols - 1 - c0;

    // gathered operand: tile row r is row a_rows[m0 + r] / a_div of a (the launcher checks
    // that a_nrows * rb fits in 32 bits)
    const uint8_t* a_tile = p.a_rows ? p.a : p.a + static_cast<size_t>(m0) * rb;
    const uint8_t* b_tile = p.b + static_cast<size_t>(e) * p.b_rows * rb;

    // this lane's source offsets; wave w fills groups w, w + waves, ... (A groups first).
    // Rows past the segment (A) or past the matrix (B) re-read the last valid one.
    uint32_t src[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int g = wave + kDmaWaves * j;
      if (j < C::kAPerWave) {
        int r = g * C::kRowsPerGroup + lrow;
        r = r < mlast ? r : mlast;
        if (p.a_rows) {
          int t = p.a_rows[m0 + r] / p.a_div;
          t = t < 0 ? 0 : (t < p.a_nrows ? t : p.a_nrows - 1);
          r = t;
        }
        src[j] = static_cast<uint32_t>(r) * rb + lchunk * 16;
      } else {
        const int r = (g - C::kAGroups) * C::kRowsPerGroup + lrow;   // tile weight row
        uint32_t wr;
        if (MODE == MODE_GATE_UP) {
          const int c = r % (BN / 2);
          const int cc = c < clast ? c : clast;
          wr = (r < BN / 2 ? 0u : static_cast<uint32_t>(p.I)) + static_cast<uint32_t>(c0 + cc);
        } else {
          wr = static_cast<uint32_t>(c0 + (r < clast ? r : clast));
        }
        src[j] = wr * rb + lchunk * 16;
      }
    }

    auto dma_slice = [&](int ks, int buf, int j) __attribute__((always_inline)) {
      const uint32_t base = __builtin_amdgcn_readfirstlane(
          lds_addr0 + static_cast<uint32_t>(buf * C::kStageBytes + (wave + kDmaWaves * j) * kDGroup));
      const size_t k_off = static_cast<size_t>(ks) * ROWB;
      dma16((j < C::kAPerWave ? a_tile : b_tile) + k_off + src[j], base);
    };

    f32x16_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = f32x16_t{};

    auto load_frags = [&]<int ACT>(int buf, int s, Frag<CT_BF16> (&fa)[MB], Frag<CT_BF16> (&fb)[NB])
        __attribute__((always_inline)) {
      const uint8_t* base = lds + buf * C::kStageBytes;
#pragma unroll
      for (int mb = 0; mb < ACT; ++mb) fa[mb].load(base + a_frag[mb] + koff[s]);
      if (ACT > 0) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) fb[nb].load(base + b_frag[nb] + koff[s]);
      }
    };
    // the MB*NB MFMAs of one k-step; after MFMA i, run `between(i)` (kept in place by
    // scheduling fences so that it issues while the MFMA pipe is busy)
    auto mfma_step = [&]<int ACT>(Frag<CT_BF16> (&fa)[MB], Frag<CT_BF16> (&fb)[NB], auto&& between)
        __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < MB * NB; ++i) {
        if (i / NB < ACT) acc[i / NB][i % NB] = mma(fa[i / NB], fb[i % NB], acc[i / NB][i % NB]);
        __builtin_amdgcn_sched_barrier(0);
        between(i);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto nothing = [](int) __attribute__((always_inline)) {};

    // ---- pipeline (STAGES LDS buffers).  Stage ks lives in buffer ks % STAGES.  While
    // stage ks is multiplied, stage ks+STAGES-1 is loaded into the buffer stage ks-1 used:
    // its loads are spread over the MFMAs of every k-step but the last (a burst of them
    // would overflow the address unit's queue and stall the issuing waves).  At the start
    // of the last k-step each wave waits for stage ks+1, the barrier makes that hold for all
    // waves and frees buffer ks % STAGES, and the first fragments of stage ks+1 are read
    // while the last k-step's MFMAs run.
    static_assert(STAGES >= 2 && (STAGES - 2) * PER < 64, "buffers, and the loads a wait may leave in flight");
    constexpr int kAhead = STAGES - 1;                     // stages loading while one is used
    // wait until at most n stages of loads remain in flight (n < kAhead)
    auto wait_stages = [](int n) __attribute__((always_inline)) {
      [&]<int... I>(std::integer_sequence<int, I...>) {
        ((n == I ? wait_vmcnt<I * PER>() : void()), ...);
      }(std::make_integer_sequence<int, kAhead>{});
    };
    constexpr int kSlots = (KSTEPS - 1) * MB * NB;         // MFMA slots that may carry a load
    static_assert(PER <= kSlots, "not enough MFMA slots to spread a stage's loads");
    wait_vmcnt<0>();   // the previous tile's epilogue stores have drained
    block_barrier();   // and every wave is past its last LDS reads
    for (int st = 0; st < kAhead && st < nk; ++st)
#pragma unroll
      for (int j = 0; j < PER; ++j) dma_slice(st, st, j);
    wait_stages((kAhead < nk ? kAhead : nk) - 1);   // stage 0 landed
    block_barrier();

    // 32-row blocks of this wave that hold rows of the segment: MFMAs and fragment reads of
    // the others are skipped (the loads and barriers are the same on every path)
    int act = ((mlast + 32) / 32 - wm + WM - 1) / WM;
    act = act < 0 ? 0 : (act > MB ? MB : act);

    auto k_loop = [&](auto act_c) __attribute__((always_inline)) {
      constexpr int ACT = decltype(act_c)::value;
      Frag<CT_BF16> f0a[MB], f0b[NB], f1a[MB], f1b[NB];
      load_frags.template operator()<ACT>(0, 0, f0a, f0b);
      int buf = 0;
      // one stage; LOAD: stage ks + kAhead exists and is loaded now, NEXT: stage ks + 1
      // exists.  The three kinds of stage run in separate loops, so that no branch on these
      // conditions sits between the MFMAs (at such a join the compiler's LDS wait before
      // the first MFMA of the last k-step would also cover the next stage's fresh reads).
      auto stage = [&]<bool LOAD, bool NEXT>(int ks) __attribute__((always_inline)) {
        const int nbuf = buf == STAGES - 1 ? 0 : buf + 1;
        const int lbuf = buf == 0 ? STAGES - 1 : buf - 1;    // (ks + STAGES - 1) % STAGES
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          Frag<CT_BF16>(&ca)[MB] = (s & 1) ? f1a : f0a;
          Frag<CT_BF16>(&cb)[NB] = (s & 1) ? f1b : f0b;
          Frag<CT_BF16>(&na)[MB] = (s & 1) ? f0a : f1a;
          Frag<CT_BF16>(&nb)[NB] = (s & 1) ? f0b : f1b;
          if (s + 1 < KSTEPS) {
            load_frags.template operator()<ACT>(buf, s + 1, na, nb);
            __builtin_amdgcn_sched_barrier(0);
            // load j of stage ks+kAhead goes after MFMA slot (j * kSlots) / PER
            mfma_step.template operator()<ACT>(ca, cb, [&](int i) __attribute__((always_inline)) {
              const int slot_i = s * MB * NB + i;
#pragma unroll
              for (int j = 0; j < PER; ++j)
                if (LOAD && (j * kSlots) / PER == slot_i) dma_slice(ks + kAhead, lbuf, j);
            });
          } else {
            // last k-step of stage ks
            if constexpr (NEXT) {
              wait_lgkmcnt_all();                       // this wave's reads of buffer `buf` are done
              // stage ks+1 landed; the stages issued after it may stay in flight
              if constexpr (LOAD) wait_stages(kAhead - 1);
              else wait_stages(nk - 2 - ks);
              block_barrier();
              load_frags.template operator()<ACT>(nbuf, 0, na, nb);
            }
            __builtin_amdgcn_sched_barrier(0);
            mfma_step.template operator()<ACT>(ca, cb, nothing);
          }
        }
        buf = nbuf;
      };
      int ks = 0;
      for (; ks < nk - kAhead; ++ks) stage.template operator()<true, true>(ks);
      for (; ks < nk - 1; ++ks) stage.template operator()<false, true>(ks);
      stage.template operator()<false, false>(ks);
    };
    // one instantiation of the k-loop per number of active 32-row blocks (0..MB)
    [&]<int... A>(std::integer_sequence<int, A...>) {
      ((act == A ? k_loop(std::integral_constant<int, A>{}) : void()), ...);
    }(std::make_integer_sequence<int, MB + 1>{});

    // ---- epilogue
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = m0 + (mb * WM + wm) * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (r >= mend) continue;
        if (MODE == MODE_GATE_UP) {
#pragma unroll
          for (int nb = 0; nb < NB / 2; ++nb) {
            const int col = c0 + wn * (BN / (2 * WN)) + nb * 32 + (lane & 31);
            if (col >= n_cols) continue;
            const float g = acc[mb][nb][v];
            const float u = acc[mb][nb + NB / 2][v];
            const float hv = silu_f32(g) * u;
            reinterpret_cast<uint16_t*>(p.out)[static_cast<size_t>(r) * p.I + col] = f32_to_bf16(hv);
          }
        } else {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int col = c0 + wn * (BN / WN) + nb * 32 + (lane & 31);
            if (col >= n_cols) continue;
            reinterpret_cast<uint16_t*>(p.out)[static_cast<size_t>(r) * p.n_out + col] = f32_to_bf16(acc[mb][nb][v]);
          }
        }
      }
    }
  }
}

// the 128-row direct-to-LDS kernel's shape: 256 weight rows, stages of 128 bytes per row,
// three stages in LDS, 2 x 4 waves
constexpr int kDmaBN = 256, kDmaRowB = 128, kDmaStages = 3, kDmaWM = 2, kDmaWN = 4;

// m-tiles at the finest granularity any kernel uses (16 rows)
size_t gemm_tile_cap(int rows, int E) {
  return static_cast<size_t>((rows + kStreamTileRows - 1) / kStreamTileRows) + E;
}

// the 256 x 256 kernel numbers its tiles in 32 bits and splits them over the 8 XCDs by
// multiplying the count by the XCD index: 8 x an upper bound of the tile count stays below 2^31
// (the 320 x 128 tiles: at most one per expert, with twice the n-blocks)
static bool wide_tiles_fit(int mode, int rows, int n_seg, int I, int n_out) {
  const long long n_blocks = mode == MODE_GATE_UP ? (I + 63) / 64 : (n_out + 127) / 128;
  return static_cast<long long>(gemm_tile_cap(rows, n_seg)) * n_blocks * kNumXcd < (1LL << 31);
}

// the wide kernel stores a tile's outputs through a buffer window over its rows (at most 320):
// the window and every offset in it stay below 2^31 bytes (gate/up: the pre-activation rows
// of 4 I bytes too)
static bool wide_out_fits(int mode, int I, int n_out) {
  return static_cast<long long>(kWideTallRows) * 4 * (mode == MODE_GATE_UP ? I : n_out) < (1LL << 31);
}

bool grouped_gemm_shared_supported(int mode, int K, int I, int n_out, long long b_rows, int a_nrows,
                                   bool gathered) {
  const long long rbytes = 2LL * K;
  return K % 128 == 0 && (mode == MODE_GATE_UP ? I : n_out) % 8 == 0 && wide_out_fits(mode, I, n_out) &&
         b_rows * rbytes < (1LL << 32) &&
         (gathered ? static_cast<long long>(a_nrows) : kWideTileRows) * rbytes < (1LL << 32);
}

hipError_t launch_build_tiles(const int32_t* offsets, int E, int rows, int tile_rows, int cap, int32_t* prefix,
                              int32_t* tile_expert, int32_t* tile_counter, hipStream_t s) {
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, s, offsets, E, rows, tile_rows, cap, prefix,
                     tile_expert, tile_counter, 0, 0, nullptr, kNumXcd);
  return hipGetLastError();
}

// prefix [E + 1], tile_expert [cap], counters [8 + 1: one per XCD and the shared tail], list
// of 320-row experts [E + 1] and its counters [8]
size_t gemm_schedule_bytes(int rows, int E) {
  const size_t n = 2 * (static_cast<size_t>(E) + 1 + kNumXcd) + 1 + gemm_tile_cap(rows, E);
  return (n * sizeof(int32_t) + 255) & ~static_cast<size_t>(255);
}

// bf16 GEMMs on 256 x 256 tiles: every gate/up and every routed down (E > 1).  A single
// dense down GEMM (the shared expert on its own: 8192 x 7168 outputs) makes 3.5 wide tiles
// per CU but exactly 7 of 128 x 256, so it keeps the smaller tiles.  The wide kernel takes
// its tiles from a counter per XCD.

static int persistent_grid() {
  // one workgroup per CU (256 CUs); a multiple of the 8 XCDs
  return 256;
}

// bf16 copy of e4m3 rows [rows, K] with fp32 scales [rows, K / 128]: each value is its code times
// the scale of its 128-column block, rounded to the nearest bf16 (even on ties).  One 16-byte
// store per 8 codes; n8 = rows * K / 8 < 2^31.
__global__ __launch_bounds__(256) void dequant_e4m3_kernel(const uint2* __restrict__ q,
                                                           const float* __restrict__ scale, int n8, int K,
                                                           uint4* __restrict__ out) {
  const int g8 = K / 8, nblk = K / 128;
  for (int i = blockIdx.x * 256 + static_cast<int>(threadIdx.x); i < n8; i += gridDim.x * 256) {
    const int r = i / g8, c = i - r * g8;
    out[i] = e4m3x8_scaled_to_bf16x8(q[i], scale[static_cast<size_t>(r) * nblk + c / 16]);
  }
}

hipError_t launch_dequant_e4m3(const uint8_t* q, const float* scale, long long rows, int cols, void* out,
                               hipStream_t s) {
  const int n8 = static_cast<int>(rows * cols / 8);
  if (n8 == 0) return hipSuccess;
  const int blocks = (n8 + 255) / 256 < 16384 ? (n8 + 255) / 256 : 16384;
  hipLaunchKernelGGL(dequant_e4m3_kernel, dim3(blocks), dim3(256), 0, s, reinterpret_cast<const uint2*>(q), scale,
                     n8, cols, reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

// bytes of the dequantized activations the fp8 gate/up keeps after its tile schedule
size_t gemm_a8_bytes(int rows, int K) {
  return (static_cast<size_t>(rows) * K * 2 + 255) & ~static_cast<size_t>(255);
}

hipError_t launch_grouped_gemm(int ct, bool b8, int mode, const void* a, const float* a_scale,
                               const void* b, const float* b_scale, void* out, bool out_f32,
                               const int32_t* offsets, int E, int rows, int K, int I, int n_out,
                               long long b_rows, void* sched, hipStream_t s, const int32_t* a_rows,
                               int a_div, int a_nrows, const void* shared_b, int shared_rows,
                               const int32_t* row_slot, const float* row_gate, void* au,
                               const float* shared_b_scale) {
  // with a shared segment the schedule covers E + 1 segments and rows + shared_rows rows
  const int n_seg = E + (shared_rows > 0 ? 1 : 0);
  int32_t* prefix = reinterpret_cast<int32_t*>(sched);
  int32_t* tile_expert = prefix + n_seg + 1;
  const int cap = static_cast<int>(gemm_tile_cap(rows + shared_rows, n_seg));
  int32_t* tile_counter = tile_expert + cap;
  int32_t* tall_list = tile_counter + kNumXcd + 1;   // [E + 1] + [kNumXcd] counters
  // few rows per expert and e4m3 weights: the weight-streaming kernel (16-row m-tiles)
  const bool stream = (mode == MODE_GATE_UP ? ct == CT_FP8 : b8) && shared_rows == 0 && a_rows == nullptr &&
                      static_cast<long long>(rows) <= static_cast<long long>(kStreamTileRows) * E &&
                      (mode == MODE_GATE_UP ? I % 64 == 0 : n_out % 128 == 0) &&
                      static_cast<long long>(gemm_tile_cap(rows, E)) * (mode == MODE_GATE_UP ? I / 64 : n_out / 128) <
                          (1LL << 31);
  const bool dma = ct == CT_BF16 && !b8;   // bf16 operands: the direct-to-LDS kernels
  // fp8 gate/up above decode sizes: the activations are dequantized to bf16 (into the workspace,
  // after the schedule) and multiplied against the e4m3 weights on the 256 x 256 kernel, which
  // loads the weights' codes and block scales straight to LDS and converts each fragment as it
  // reads it
  if (mode == MODE_GATE_UP && ct == CT_FP8 && !b8 && !stream && a_rows == nullptr && shared_rows == 0 &&
      au == nullptr && K % 128 == 0 && I % 8 == 0 && wide_out_fits(mode, I, n_out) && b_rows * K < (1LL << 32) &&
      static_cast<long long>(kWideTileRows) * 2 * K < (1LL << 32) &&
      static_cast<long long>(rows) * K / 8 < (1LL << 31) && wide_tiles_fit(mode, rows, E, I, n_out)) {
    void* deq = static_cast<uint8_t*>(sched) + gemm_schedule_bytes(rows, E);
    const hipError_t e = launch_dequant_e4m3(static_cast<const uint8_t*>(a), a_scale, rows, K, deq, s);
    if (e != hipSuccess) return e;
    return launch_grouped_gemm(CT_BF16, true, mode, deq, nullptr, b, b_scale, out, out_f32, offsets, E, rows, K,
                               I, n_out, b_rows, sched, s);
  }
  // 256 x 256 tiles while every operand offset fits the kernel's 32-bit arithmetic
  const long long rbytes = 2LL * K;
  const bool wide_ok = dma && K % 128 == 0 && (mode == MODE_GATE_UP ? I : n_out) % 8 == 0 &&
                       wide_out_fits(mode, I, n_out) &&
                       b_rows * rbytes < (1LL << 32) &&
                       (a_rows ? static_cast<long long>(a_nrows) : kWideTileRows) * rbytes < (1LL << 32) &&
                       wide_tiles_fit(mode, rows + shared_rows, n_seg, I, n_out);
  // e4m3 weights (down; gate/up with dequantized activations, gathered or not, and the shared
  // expert's rows as one more segment) at more than 16 rows per expert: the 256 x 256 kernel,
  // which converts each weight fragment (code times its block's scale) as it reads it from LDS
  const bool wide8 = (mode == MODE_DOWN || mode == MODE_GATE_UP) && ct == CT_BF16 && b8 && !stream && K % 128 == 0 &&
                     n_out % 8 == 0 && wide_out_fits(mode, I, n_out) &&
                     b_rows * K < (1LL << 32) && b_rows * (K / 128) * 4 < (1LL << 32) &&
                     (a_rows ? static_cast<long long>(a_nrows) : kWideTileRows) * rbytes < (1LL << 32) &&
                     (shared_rows == 0 || shared_b_scale != nullptr) && row_gate == nullptr && au == nullptr &&
                     (a_rows == nullptr || mode == MODE_GATE_UP) &&
                     wide_tiles_fit(mode, rows + shared_rows, n_seg, I, n_out);
  if ((shared_rows > 0 || row_gate != nullptr || au != nullptr) && (!(wide_ok || wide8) || stream))
    return hipErrorNotSupported;   // (callers check first)
  const bool wide = wide_ok && (shared_rows > 0 || row_gate != nullptr || au != nullptr ||
                                mode == MODE_GATE_UP || E > 1);
  const int tile_rows = stream ? kStreamTileRows : (wide || wide8 ? kWideTileRows : (dma ? kDM : GBM));
  // bf16 GEMMs on the 256 x 256 kernel: experts of 257..320 rows as one tile (down: 320 x 128,
  // gate/up: 320 x 256); the down GEMM on e4m3 weights as well (320 x 128)
  const bool tall = wide || (wide8 && mode == MODE_DOWN);
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, s, offsets, E, rows, tile_rows, cap,
                     prefix, tile_expert, tile_counter, shared_rows, kWideTallRows,
                     tall ? tall_list : nullptr, kNumXcd + 1);
  GemmArgs p;
  p.a = reinterpret_cast<const uint8_t*>(a);
  p.a_scale = a_scale;
  p.b = reinterpret_cast<const uint8_t*>(b);
  p.b_scale = b_scale;
  p.out = out;
  p.offsets = offsets;
  p.tile_prefix = prefix;
  p.tile_expert = tile_expert;
  p.a_rows = a_rows;
  p.a_div = a_div > 0 ? a_div : 1;
  p.a_nrows = a_nrows;
  p.E = E;
  p.K = K;
  p.rows = rows;
  p.I = I;
  p.n_out = n_out;
  p.tile_cap = cap;
  p.b_rows = b_rows;
  p.out_f32 = out_f32 ? 1 : 0;
  p.tile_counter = nullptr;
  p.shared_b = reinterpret_cast<const uint8_t*>(shared_b);
  p.shared_rows = shared_rows;
  p.row_slot = row_gate != nullptr ? row_slot : nullptr;
  p.row_gate = row_slot != nullptr ? row_gate : nullptr;
  p.k_split = 1;
  p.au = au;
  p.shared_b_scale = shared_b_scale;
  if (stream) return launch_grouped_gemm_stream(mode, p, s);
  if (wide || wide8) {
    p.tile_counter = tile_counter;
    if (tall) {
      p.tall_list = tall_list;
      p.tall_counter = tall_list + E + 1;
    }
    return launch_grouped_gemm_wide(mode, p, s, wide8);
  }
  const dim3 grid(persistent_grid()), block(GTHREADS);
#define MOE_LAUNCH(CT_, B8_, MODE_) \
  hipLaunchKernelGGL((grouped_gemm_kernel<CT_, B8_, MODE_>), grid, block, 0, s, p)
#define MOE_LAUNCH_DMA(MODE_) \
  hipLaunchKernelGGL((grouped_gemm_dma_kernel<MODE_, kDmaBN, kDmaRowB, kDmaStages, kDmaWM, \
                                              kDmaWN>), \
                     dim3(persistent_grid() * kDmaOcc), \
                     dim3(DmaCfg<kDmaBN, kDmaRowB, kDmaStages, kDmaWM, kDmaWN>::kThreads), 0, s, p)
  if (mode == MODE_GATE_UP) {
    if (ct == CT_F32) MOE_LAUNCH(CT_F32, false, MODE_GATE_UP);
    else if (ct == CT_BF16) MOE_LAUNCH_DMA(MODE_GATE_UP);
    else MOE_LAUNCH(CT_FP8, false, MODE_GATE_UP);
  } else {
    if (ct == CT_F32) MOE_LAUNCH(CT_F32, false, MODE_DOWN);
    else if (b8) MOE_LAUNCH(CT_BF16, true, MODE_DOWN);
    else MOE_LAUNCH_DMA(MODE_DOWN);
  }
#undef MOE_LAUNCH_DMA
#undef MOE_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
