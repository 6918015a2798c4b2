// Grouped expert GEMMs on CDNA4 matrix cores ("MoE part 4" page, section 2: one launch
// for many expert GEMMs with differing row counts n_e; section 4.1: FC1 -> activation ->
// FC2, here SwiGLU).
//
//   gate/up:  h[r, :]   = silu(a[r] . W_gate,e^T) * (a[r] . W_up,e^T)   for r in segment e
//   down:     out[r, :] = h[r] . W_down,e^T
//
// Operands are K-contiguous (a [rows, K], weights [n, K]), so both MFMA operands are
// 16-byte row fragments.  A workgroup (4 waves, 2 x 2) computes a 128-row x 128-column
// tile with v_mfma_f32_32x32x16 (bf16 and fp8) or v_mfma_f32_32x32x2 (fp32); K advances
// in 128-byte stages through double-buffered, padded LDS, the next stage's global loads
// in flight while the current one is multiplied.
//
// The gate/up tile takes 64 rows of W_gate and the same 64 rows of W_up, so each wave
// holds matching gate and up accumulators and applies SwiGLU in registers; h is written
// once.
//
// Tile schedule: a one-workgroup prologue turns offsets into a per-expert m-tile prefix.
// The GEMM is persistent: the logical tiles are ordered expert -> n-block -> m-tile (the
// m-tiles sharing a weight block are adjacent) and split into 8 contiguous ranges, one
// per XCD (workgroup i runs on XCD i mod 8), so tiles that share weights and activation
// rows share an L2.  Every tile has the same cost whatever the skew of n_e, so ragged and
// hot experts spread evenly over the CUs.
//
// fp8 layers: the gate/up GEMM multiplies e4m3 codes on the fp8 MFMA, sums each 128-wide
// K block in a separate fp32 accumulator and adds it scaled by a_scale[row] *
// w_scale[col]; the down GEMM converts e4m3 W_down to bf16 (exactly) on its way to LDS,
// multiplies against bf16 h, and scales each 128-wide K block by w_scale[col].
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

enum { CT_F32 = 0, CT_BF16 = 1, CT_FP8 = 2 };
enum { MODE_GATE_UP = 0, MODE_DOWN = 1 };

constexpr int GBM = 128;          // rows of a tile
constexpr int GBN = 128;          // weight rows of a tile
constexpr int GKB = 128;          // bytes of K per row and stage (compute type)
constexpr int GPITCH = GKB + 16;  // padded LDS row pitch: 8 consecutive rows hit 8 bank groups
constexpr int GTHREADS = 256;
constexpr int kNumXcd = 8;

template <int CT> struct CTraits;
template <> struct CTraits<CT_F32> { static constexpr int esz = 4; };
template <> struct CTraits<CT_BF16> { static constexpr int esz = 2; };
template <> struct CTraits<CT_FP8> { static constexpr int esz = 1; };

struct GemmArgs {
  const uint8_t* a;            // [rows, K] compute-type elements (e4m3 codes for CT_FP8)
  const float* a_scale;        // [rows, K / 128]            (CT_FP8)
  const uint8_t* b;            // [E, b_rows, K]: compute type, or e4m3 codes when B8
  const float* b_scale;        // [E, b_rows, K / 128]       (CT_FP8, B8)
  void* out;                   // gate/up: h [rows, I]; down: out [rows, H]
  const int32_t* offsets;      // [E + 1]
  const int32_t* tile_prefix;  // [E + 1]
  const int32_t* tile_expert;  // [tile_cap]
  int E, K, rows, I, n_out, tile_cap;
  long long b_rows;
  int out_f32;
};

// Tile schedule prologue: m-tiles of each expert, their prefix and the m-tile -> expert
// table.  Offsets are clamped into [0, rows] so malformed input cannot index out of range.
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets, int E,
                                                           int rows, int tile_cap,
                                                           int32_t* __restrict__ prefix,
                                                           int32_t* __restrict__ tile_expert) {
  __shared__ int32_t tot[1024];
  const int e = threadIdx.x;
  int mt = 0;
  if (e < E) {
    int lo = offsets[e], hi = offsets[e + 1];
    lo = lo < 0 ? 0 : (lo > rows ? rows : lo);
    hi = hi < lo ? lo : (hi > rows ? rows : hi);
    mt = (hi - lo + GBM - 1) / GBM;
  }
  tot[e] = mt;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = e >= off ? tot[e - off] : 0;
    __syncthreads();
    tot[e] += v;
    __syncthreads();
  }
  const int start = tot[e] - mt;
  if (e < E) {
    prefix[e] = start < tile_cap ? start : tile_cap;
    for (int i = 0; i < mt && start + i < tile_cap; ++i) tile_expert[start + i] = e;
  }
  if (e == E - 1) prefix[E] = tot[e] < tile_cap ? tot[e] : tile_cap;
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
  const float av[8] = {__uint_as_float(a.v0.x), __uint_as_float(a.v0.y), __uint_as_float(a.v0.z),
                       __uint_as_float(a.v0.w), __uint_as_float(a.v1.x), __uint_as_float(a.v1.y),
                       __uint_as_float(a.v1.z), __uint_as_float(a.v1.w)};
  const float bv[8] = {__uint_as_float(b.v0.x), __uint_as_float(b.v0.y), __uint_as_float(b.v0.z),
                       __uint_as_float(b.v0.w), __uint_as_float(b.v1.x), __uint_as_float(b.v1.y),
                       __uint_as_float(b.v1.z), __uint_as_float(b.v1.w)};
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s], bv[s], c, 0, 0, 0);
  return c;
}

// CT: compute type held in LDS.  B8: B is stored as e4m3 and converted to bf16 (CT_BF16)
// on its way to LDS.  Scaled: per-128-K block scales (CT_FP8: A and B; B8: B only).
template <int CT, bool B8, int MODE>
__global__ __launch_bounds__(GTHREADS) void grouped_gemm_kernel(GemmArgs p) {
  constexpr int esz = CTraits<CT>::esz;
  constexpr int BK = GKB / esz;                 // K elements per stage
  constexpr int KSTEPS = BK / 16;               // 16-wide MFMA steps per stage
  constexpr bool kScaled = (CT == CT_FP8) || B8;
  constexpr int kStagesPerBlock = 128 / BK;     // stages per 128-wide scale block
  constexpr int kStageBytes = GBM * GPITCH;

  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][kStageBytes];
  __shared__ float lds_sa[2][GBM];
  __shared__ float lds_sb[2][GBN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  const int nN = MODE == MODE_GATE_UP ? p.I / 64 : p.n_out / GBN;
  const long long total = static_cast<long long>(p.tile_prefix[p.E]) * nN;
  const int xcd = blockIdx.x % kNumXcd;
  const int slot = blockIdx.x / kNumXcd;
  const int per_xcd = gridDim.x / kNumXcd;
  const long long t_beg = total * xcd / kNumXcd;
  const long long t_end = total * (xcd + 1) / kNumXcd;

  const int nk = p.K / BK;
  const size_t a_row_bytes = static_cast<size_t>(p.K) * esz;
  const size_t b_row_bytes = static_cast<size_t>(p.K) * (B8 ? 1 : esz);
  const int kblocks = p.K / 128;

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
    const int mend = seg_hi;

    // ---- per-thread global sources: 4 A chunks and 4 B chunks per stage
    const uint8_t* a_src[4];
    const uint8_t* b_src[4];
    int lds_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + GTHREADS * i;
      const int row = q >> 3, c = q & 7;
      int ar = m0 + row;
      ar = ar < mend ? ar : mend - 1;
      a_src[i] = p.a + static_cast<size_t>(ar) * a_row_bytes + c * 16;
      long long br;
      if (MODE == MODE_GATE_UP)
        br = row < 64 ? static_cast<long long>(nblk) * 64 + row : p.I + static_cast<long long>(nblk) * 64 + (row - 64);
      else
        br = static_cast<long long>(nblk) * GBN + row;
      b_src[i] = p.b + (static_cast<size_t>(e) * p.b_rows + br) * b_row_bytes + c * (B8 ? 8 : 16);
      lds_off[i] = row * GPITCH + c * 16;
    }
    // scale sources: threads 0..127 -> A row scales, 128..255 -> B row scales
    const float* s_src = nullptr;
    if (kScaled) {
      if (tid < GBM) {
        if (CT == CT_FP8) {
          int ar = m0 + tid;
          ar = ar < mend ? ar : mend - 1;
          s_src = p.a_scale + static_cast<size_t>(ar) * kblocks;
        }
      } else {
        const int row = tid - GBM;
        long long br;
        if (MODE == MODE_GATE_UP)
          br = row < 64 ? static_cast<long long>(nblk) * 64 + row : p.I + static_cast<long long>(nblk) * 64 + (row - 64);
        else
          br = static_cast<long long>(nblk) * GBN + row;
        s_src = p.b_scale + (static_cast<size_t>(e) * p.b_rows + br) * kblocks;
      }
    }

    uint4 ra[4], rb[4];
    float rs = 1.0f;
    auto load_stage = [&](int ks) {
#pragma unroll
      for (int i = 0; i < 4; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + static_cast<size_t>(ks) * GKB);
      if (B8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint2 w = *reinterpret_cast<const uint2*>(b_src[i] + static_cast<size_t>(ks) * BK);
          const uint2 lo = e4m3x4_to_bf16x4(w.x), hi = e4m3x4_to_bf16x4(w.y);
          rb[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + static_cast<size_t>(ks) * GKB);
      }
      if (kScaled && s_src != nullptr) rs = s_src[(ks * BK) / 128];
    };
    auto store_stage = [&](int buf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<uint4*>(&lds_a[buf][lds_off[i]]) = ra[i];
        *reinterpret_cast<uint4*>(&lds_b[buf][lds_off[i]]) = rb[i];
      }
      if (kScaled) {
        if (tid < GBM) lds_sa[buf][tid] = rs;
        else lds_sb[buf][tid - GBM] = rs;
      }
    };

    f32x16_t acc[2][2];
    f32x16_t part[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[i][j] = f32x16_t{};
        part[i][j] = f32x16_t{};
      }

    // fragment addresses inside a stage buffer
    const int frag_k = (lane >> 5) * 8 * esz;
    int a_frag[2], b_frag[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) a_frag[mb] = (wm * 64 + mb * 32 + (lane & 31)) * GPITCH + frag_k;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int brow = MODE == MODE_GATE_UP ? nb * 64 + wn * 32 : wn * 64 + nb * 32;
      b_frag[nb] = (brow + (lane & 31)) * GPITCH + frag_k;
    }

    __syncthreads();  // the previous tile's last reads of both buffers are done
    load_stage(0);
    store_stage(0);
    __syncthreads();

    for (int ks = 0; ks < nk; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < nk) load_stage(ks + 1);
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        Frag<CT> fa[2], fb[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) fa[mb].load(&lds_a[cur][a_frag[mb] + s * 16 * esz]);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) fb[nb].load(&lds_b[cur][b_frag[nb] + s * 16 * esz]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            if (kScaled)
              part[mb][nb] = mma(fa[mb], fb[nb], part[mb][nb]);
            else
              acc[mb][nb] = mma(fa[mb], fb[nb], acc[mb][nb]);
          }
      }
      if (kScaled && ((ks + 1) % kStagesPerBlock == 0)) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int brow = MODE == MODE_GATE_UP ? nb * 64 + wn * 32 : wn * 64 + nb * 32;
          const float sb = lds_sb[cur][brow + (lane & 31)];
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              float sc = sb;
              if (CT == CT_FP8) {
                const int r = wm * 64 + mb * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                sc = lds_sa[cur][r] * sb;
              }
              acc[mb][nb][v] += part[mb][nb][v] * sc;
              part[mb][nb][v] = 0.0f;
            }
          }
        }
      }
      if (ks + 1 < nk) store_stage(cur ^ 1);
      __syncthreads();
    }

    // ---- epilogue
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = m0 + wm * 64 + mb * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (r >= mend) continue;
        if (MODE == MODE_GATE_UP) {
          const float g = acc[mb][0][v];
          const float u = acc[mb][1][v];
          const float hv = g / (1.0f + expf(-g)) * u;
          const size_t o = static_cast<size_t>(r) * p.I + static_cast<size_t>(nblk) * 64 + wn * 32 + (lane & 31);
          if (p.out_f32) reinterpret_cast<float*>(p.out)[o] = hv;
          else reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_bf16(hv);
        } else {
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const size_t o = static_cast<size_t>(r) * p.n_out + static_cast<size_t>(nblk) * GBN + wn * 64 + nb * 32 + (lane & 31);
            if (p.out_f32) reinterpret_cast<float*>(p.out)[o] = acc[mb][nb][v];
            else reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_bf16(acc[mb][nb][v]);
          }
        }
      }
    }
  }
}

size_t gemm_tile_cap(int rows, int E) { return static_cast<size_t>((rows + GBM - 1) / GBM) + E; }

size_t gemm_schedule_bytes(int rows, int E) {
  const size_t n = static_cast<size_t>(E) + 1 + gemm_tile_cap(rows, E);
  return (n * sizeof(int32_t) + 255) & ~static_cast<size_t>(255);
}

static int persistent_grid() {
  // 256 CUs x 2 resident workgroups; a multiple of the 8 XCDs
  return 512;
}

hipError_t launch_grouped_gemm(int ct, bool b8, int mode, const void* a, const float* a_scale,
                               const void* b, const float* b_scale, void* out, bool out_f32,
                               const int32_t* offsets, int E, int rows, int K, int I, int n_out,
                               long long b_rows, void* sched, hipStream_t s) {
  int32_t* prefix = reinterpret_cast<int32_t*>(sched);
  int32_t* tile_expert = prefix + E + 1;
  const int cap = static_cast<int>(gemm_tile_cap(rows, E));
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, s, offsets, E, rows, cap, prefix,
                     tile_expert);
  GemmArgs p;
  p.a = reinterpret_cast<const uint8_t*>(a);
  p.a_scale = a_scale;
  p.b = reinterpret_cast<const uint8_t*>(b);
  p.b_scale = b_scale;
  p.out = out;
  p.offsets = offsets;
  p.tile_prefix = prefix;
  p.tile_expert = tile_expert;
  p.E = E;
  p.K = K;
  p.rows = rows;
  p.I = I;
  p.n_out = n_out;
  p.tile_cap = cap;
  p.b_rows = b_rows;
  p.out_f32 = out_f32 ? 1 : 0;
  const dim3 grid(persistent_grid()), block(GTHREADS);
#define MOE_LAUNCH(CT_, B8_, MODE_) \
  hipLaunchKernelGGL((grouped_gemm_kernel<CT_, B8_, MODE_>), grid, block, 0, s, p)
  if (mode == MODE_GATE_UP) {
    if (ct == CT_F32) MOE_LAUNCH(CT_F32, false, MODE_GATE_UP);
    else if (ct == CT_BF16) MOE_LAUNCH(CT_BF16, false, MODE_GATE_UP);
    else MOE_LAUNCH(CT_FP8, false, MODE_GATE_UP);
  } else {
    if (ct == CT_F32) MOE_LAUNCH(CT_F32, false, MODE_DOWN);
    else if (b8) MOE_LAUNCH(CT_BF16, true, MODE_DOWN);
    else MOE_LAUNCH(CT_BF16, false, MODE_DOWN);
  }
#undef MOE_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
