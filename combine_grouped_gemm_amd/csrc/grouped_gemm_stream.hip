// Weight-streaming grouped expert GEMMs for layers with few rows per expert ("MoE part 4"
// page, section 2: one launch for many expert GEMMs with differing row counts n_e; section
// 4.1: FC1 -> activation -> FC2, here SwiGLU), for e4m3 expert weights with one fp32 scale
// per 128-wide K block ("DeepEP" page, low-latency decode kernels, FP8 dispatch).
//
//   gate/up:  h[r, :]   = silu(a[r] . W_gate,e^T) * (a[r] . W_up,e^T)     a: e4m3 codes + scales
//   down:     out[r, :] = h[r] . W_down,e^T                               h: bf16
//
// At decode sizes (a few rows per expert) the work is bound by reading every routed
// expert's weights once from HBM; the matrix-core work is an order of magnitude below
// that.  So nothing is shared through LDS: every wave is an independent worker that
// streams a 128-row weight panel of one expert against a 16-row m-tile of that expert's
// rows, loading straight into the registers that feed v_mfma_f32_16x16x32 (fp8 for
// gate/up, bf16 for down, the e4m3 weights converted to bf16 exactly in registers).
//
// K is taken in 128-wide blocks (one scale block).  Inside a block, lane l covers
// row/column l % 16 and the 32 K elements [32 q, 32 q + 32) with q = l / 16, as two (e4m3)
// or four (bf16) 16-byte loads; MFMA step j uses elements 32 q + 8 j .. + 8.  A and B use
// the same assignment, so each step sums 32 distinct K elements and the four steps cover
// the block.  Each block's product is summed in its own fp32 accumulator and added to the
// total scaled by a_scale[row] * w_scale[col] (gate/up) or w_scale[col] (down).
//
// A wave keeps STAGES K blocks of loads in flight in registers, across tile boundaries:
// its tiles form one stream of (tile, K block) steps.  Tiles are ordered expert -> n-block
// -> m-tile, split into 8 contiguous ranges (one per XCD, workgroup i runs on XCD i mod
// 8), and dealt round-robin to the waves of that XCD, so neighbouring panels of one
// expert stream at the same time under one L2 and share its activation rows.
#include <type_traits>

#include "grouped_gemm.h"
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kSCB = 8;      // 16-row weight blocks of a panel (128 weight rows)
constexpr int kSWaves = 4;   // waves per workgroup

constexpr int kStreamStages = 3;     // K blocks each wave keeps in flight
constexpr int kStreamWgPerCu = 1;    // workgroups per CU

template <int MODE>
struct StreamStage {
  static constexpr int kA = MODE == MODE_GATE_UP ? 2 : 4;  // 16-byte A loads per lane and K block
  uint4 b[kSCB][2];
  uint4 a[kA];
  float sa;      // gate/up: a_scale of row l % 16
  float sb[2];   // w_scale of weight row l % 16 of blocks l / 16 and l / 16 + 4
};

// Panel weight-row offset of block cb: gate/up takes 64 gate rows and the matching 64 up
// rows (block cb >= 4 is up block cb - 4), down takes 128 consecutive rows.
template <int MODE>
__device__ __forceinline__ int panel_row(int cb, int I) {
  if (MODE == MODE_GATE_UP) return cb < 4 ? 16 * cb : I + 16 * (cb - 4);
  return 16 * cb;
}

// VEC: the K blocks per row are a multiple of 4, and the scales are loaded as float4 groups
// of 4 consecutive K blocks, one load per row every 4 steps.
template <int MODE, int STAGES, int WG_PER_CU, bool VEC>
__global__ __launch_bounds__(kSWaves * 64, WG_PER_CU) void grouped_gemm_stream_kernel(GemmArgs p) {
  static_assert(!VEC || STAGES <= 4, "a scale group is reloaded 4 steps after it is taken");
  constexpr bool kGU = MODE == MODE_GATE_UP;
  constexpr int kPanelCols = kGU ? 64 : 128;        // output columns of a panel
  constexpr int kAEsz = kGU ? 1 : 2;                // bytes per A element
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int q = lane >> 4;

  const int K = p.K;
  const int nk = K / 128;
  const int kblocks = nk;
  const uint32_t arb = static_cast<uint32_t>(K) * kAEsz;   // A row bytes
  const int nN = kGU ? p.I / kPanelCols : p.n_out / kPanelCols;

  // this wave's tiles: t_beg + w, t_beg + w + W, ... below t_end (the launcher checks
  // that tile_cap * nN fits in 31 bits)
  const uint32_t total_tiles = static_cast<uint32_t>(p.tile_prefix[p.E]) * nN;
  const int xcd = blockIdx.x % kNumXcd;
  const int W = (gridDim.x / kNumXcd) * kSWaves;
  const int w = (blockIdx.x / kNumXcd) * kSWaves + (threadIdx.x >> 6);
  const uint32_t t_beg = static_cast<uint32_t>(static_cast<uint64_t>(total_tiles) * xcd / kNumXcd);
  const uint32_t t_end = static_cast<uint32_t>(static_cast<uint64_t>(total_tiles) * (xcd + 1) / kNumXcd);
  const uint32_t span = t_end - t_beg;
  const int n_my = span > static_cast<uint32_t>(w) ? static_cast<int>((span - w + W - 1) / W) : 0;
  if (n_my == 0) return;
  const int total = n_my * nk;   // steps

  // lane offsets that hold for every tile: weight row c of each block, K quarter q; the
  // weight scales of row c of blocks q and q + 4 (one load each per K block, handed to the
  // lanes that need them by ds_bpermute)
  const uint32_t voff_b = static_cast<uint32_t>(c) * K + 32 * q;
  const uint32_t voff_sb0 = static_cast<uint32_t>(panel_row<MODE>(q, p.I) + c) * kblocks;
  const uint32_t voff_sb1 = static_cast<uint32_t>(panel_row<MODE>(q + 4, p.I) + c) * kblocks;

  struct Tile {
    int e, m0, seg_hi, row0;
  };
  auto tile_at = [&](int j) __attribute__((always_inline)) -> Tile {
    const uint32_t L = t_beg + w + static_cast<uint32_t>(j) * W;
    Tile t;
    t.e = p.tile_expert[L / static_cast<uint32_t>(nN)];
    const int pe = p.tile_prefix[t.e];
    const uint32_t mt_e = static_cast<uint32_t>(p.tile_prefix[t.e + 1] - pe);
    const uint32_t local = L - static_cast<uint32_t>(pe) * nN;
    const int nblk = static_cast<int>(local / mt_e);
    const int mtile = static_cast<int>(local % mt_e);
    int lo, hi;
    expert_segment(p, t.e, lo, hi);
    t.m0 = lo + mtile * kStreamTileRows;
    t.seg_hi = hi;
    t.row0 = nblk * kPanelCols;  // gate/up: first gate row (= h column); down: first W_down row
    return t;
  };

  // ---- load cursor (runs STAGES steps ahead of the compute cursor)
  int ld_j = 0, ld_kb = 0;
  const uint8_t* ld_a = nullptr;   // A rows of the tile (uniform base)
  const uint8_t* ld_b = nullptr;   // weight panel base
  const float* ld_sa = nullptr;
  const float* ld_sb = nullptr;
  uint32_t voff_a = 0, voff_sa = 0;
  auto set_load_tile = [&](int j) __attribute__((always_inline)) {
    const Tile t = tile_at(j);
    int r = t.m0 + c;
    r = r < t.seg_hi ? r : t.seg_hi - 1;   // rows past the segment re-read its last row
    const int rl = r - t.m0;
    ld_a = p.a + static_cast<size_t>(t.m0) * arb;
    voff_a = static_cast<uint32_t>(rl) * arb + q * 32 * kAEsz;
    const size_t wrow = static_cast<size_t>(t.e) * p.b_rows + t.row0;
    ld_b = p.b + wrow * K;
    ld_sb = p.b_scale + wrow * kblocks;
    if (kGU) {
      ld_sa = p.a_scale + static_cast<size_t>(t.m0) * kblocks;
      voff_sa = static_cast<uint32_t>(rl) * kblocks;
    }
  };
  auto advance_load = [&]() __attribute__((always_inline)) {
    // past the last step the cursor stays put: the spare loads re-read the last K block
    if (ld_kb + 1 < nk) {
      ++ld_kb;
    } else if (ld_j + 1 < n_my) {
      ++ld_j;
      ld_kb = 0;
      set_load_tile(ld_j);
    }
  };
  // scale groups (VEC): taken into g_cur by the compute cursor at K blocks 0 mod 4, loaded
  // into g_next by the load cursor at the same K blocks, at most 4 steps earlier
  struct ScaleGroup {
    float4 sb[2];
    float4 sa;
  };
  ScaleGroup g_cur, g_next;
  auto issue = [&](StreamStage<MODE>& st) __attribute__((always_inline)) {
    const uint8_t* bk = ld_b + static_cast<size_t>(ld_kb) * 128;
#pragma unroll
    for (int cb = 0; cb < kSCB; ++cb) {
      const uint8_t* bp = bk + static_cast<size_t>(panel_row<MODE>(cb, p.I)) * K + voff_b;
      st.b[cb][0] = *reinterpret_cast<const uint4*>(bp);
      st.b[cb][1] = *reinterpret_cast<const uint4*>(bp + 16);
    }
    const uint8_t* ak = ld_a + static_cast<size_t>(ld_kb) * 128 * kAEsz + voff_a;
#pragma unroll
    for (int i = 0; i < StreamStage<MODE>::kA; ++i) st.a[i] = *reinterpret_cast<const uint4*>(ak + 16 * i);
    if constexpr (VEC) {
      if ((ld_kb & 3) == 0) {
        if (kGU) g_next.sa = *reinterpret_cast<const float4*>(ld_sa + voff_sa + ld_kb);
        g_next.sb[0] = *reinterpret_cast<const float4*>(ld_sb + voff_sb0 + ld_kb);
        g_next.sb[1] = *reinterpret_cast<const float4*>(ld_sb + voff_sb1 + ld_kb);
      }
    } else {
      if (kGU) st.sa = ld_sa[voff_sa + ld_kb];
      st.sb[0] = ld_sb[voff_sb0 + ld_kb];
      st.sb[1] = ld_sb[voff_sb1 + ld_kb];
    }
  };

  // ---- compute cursor
  int c_j = 0, c_kb = 0;
  f32x4_t acc[kSCB];
#pragma unroll
  for (int cb = 0; cb < kSCB; ++cb) acc[cb] = f32x4_t{};

  auto compute = [&](const StreamStage<MODE>& st) __attribute__((always_inline)) {
    f32x4_t part[kSCB];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 av = st.a[kGU ? (j >> 1) : j];
#pragma unroll
      for (int cb = 0; cb < kSCB; ++cb) {
        const uint4 bv = st.b[cb][j >> 1];
        const uint32_t b0 = (j & 1) ? bv.z : bv.x;
        const uint32_t b1 = (j & 1) ? bv.w : bv.y;
        const f32x4_t cin = j == 0 ? f32x4_t{} : part[cb];
        if constexpr (kGU) {
          const uint32_t a0 = (j & 1) ? av.z : av.x;
          const uint32_t a1 = (j & 1) ? av.w : av.y;
          const long aop = static_cast<long>((static_cast<uint64_t>(a1) << 32) | a0);
          const long bop = static_cast<long>((static_cast<uint64_t>(b1) << 32) | b0);
          part[cb] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(aop, bop, cin, 0, 0, 0);
        } else {
          // 8 e4m3 codes -> 8 bf16 (exact; unit scale)
          uint4 wb;
          wb.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b0, 1.0f, false));
          wb.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b0, 1.0f, true));
          wb.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b1, 1.0f, false));
          wb.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b1, 1.0f, true));
          part[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                             __builtin_bit_cast(bf16x8_t, wb), cin, 0, 0, 0);
        }
      }
    }
    // scale this K block's products into the totals; D row 4 q + v, column c
    float sb_own[2], sa_own = 0.0f;
    if constexpr (VEC) {
      if ((c_kb & 3) == 0) g_cur = g_next;
      sb_own[0] = g_cur.sb[0].x;
      sb_own[1] = g_cur.sb[1].x;
      sa_own = g_cur.sa.x;
      // shift the next K block's scales into .x
#pragma unroll
      for (int h = 0; h < 2; ++h) g_cur.sb[h] = make_float4(g_cur.sb[h].y, g_cur.sb[h].z, g_cur.sb[h].w, 0.0f);
      if (kGU) g_cur.sa = make_float4(g_cur.sa.y, g_cur.sa.z, g_cur.sa.w, 0.0f);
    } else {
      sb_own[0] = st.sb[0];
      sb_own[1] = st.sb[1];
      if (kGU) sa_own = st.sa;
    }
    float sb[kSCB];
#pragma unroll
    for (int cb = 0; cb < kSCB; ++cb) sb[cb] = __shfl(sb_own[cb >> 2], c + 16 * (cb & 3), 64);
    if constexpr (kGU) {
      float sav[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) sav[v] = __shfl(sa_own, 4 * q + v, 64);
#pragma unroll
      for (int cb = 0; cb < kSCB; ++cb)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[cb][v] += part[cb][v] * (sav[v] * sb[cb]);
    } else {
#pragma unroll
      for (int cb = 0; cb < kSCB; ++cb)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[cb][v] += part[cb][v] * sb[cb];
    }
  };

  auto epilogue = [&]() __attribute__((always_inline)) {
    const Tile t = tile_at(c_j);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = t.m0 + 4 * q + v;
      if (r < t.seg_hi) {
        if constexpr (kGU) {
          uint16_t* hrow = reinterpret_cast<uint16_t*>(p.out) + static_cast<size_t>(r) * p.I + t.row0 + c;
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const float g = acc[cb][v];
            const float u = acc[cb + 4][v];
            hrow[16 * cb] = f32_to_bf16(silu_f32(g) * u);
          }
        } else if (p.out_f32) {
          float* orow = reinterpret_cast<float*>(p.out) + static_cast<size_t>(r) * p.n_out + t.row0 + c;
#pragma unroll
          for (int cb = 0; cb < kSCB; ++cb) orow[16 * cb] = acc[cb][v];
        } else {
          uint16_t* orow = reinterpret_cast<uint16_t*>(p.out) + static_cast<size_t>(r) * p.n_out + t.row0 + c;
#pragma unroll
          for (int cb = 0; cb < kSCB; ++cb) orow[16 * cb] = f32_to_bf16(acc[cb][v]);
        }
      }
    }
#pragma unroll
    for (int cb = 0; cb < kSCB; ++cb) acc[cb] = f32x4_t{};
  };

  auto step = [&](const StreamStage<MODE>& st) __attribute__((always_inline)) {
    compute(st);
    if (c_kb + 1 < nk) {
      ++c_kb;
    } else {
      epilogue();
      ++c_j;
      c_kb = 0;
    }
  };

  StreamStage<MODE> st[STAGES];
  set_load_tile(0);
#pragma unroll
  for (int s = 0; s < STAGES; ++s) {
    issue(st[s]);
    advance_load();
  }
  int i = 0;
  for (; i + STAGES <= total; i += STAGES) {
#pragma unroll
    for (int s = 0; s < STAGES; ++s) {
      step(st[s]);
      issue(st[s]);
      advance_load();
    }
  }
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (i + s < total) step(st[s]);
}

hipError_t launch_grouped_gemm_stream(int mode, const GemmArgs& p, hipStream_t s) {
  const dim3 grid(256 * kStreamWgPerCu), block(kSWaves * 64);
  const bool vec = (p.K / 128) % 4 == 0;
#define MOE_LAUNCH_STREAM(MODE_, VEC_)                                                                      \
  hipLaunchKernelGGL((grouped_gemm_stream_kernel<MODE_, kStreamStages, kStreamWgPerCu, VEC_>), grid, \
                     block, 0, s, p)
  if (mode == MODE_GATE_UP) {
    if (vec) MOE_LAUNCH_STREAM(MODE_GATE_UP, true);
    else MOE_LAUNCH_STREAM(MODE_GATE_UP, false);
  } else {
    if (vec) MOE_LAUNCH_STREAM(MODE_DOWN, true);
    else MOE_LAUNCH_STREAM(MODE_DOWN, false);
  }
#undef MOE_LAUNCH_STREAM
  return hipGetLastError();
}

}  // namespace moe
