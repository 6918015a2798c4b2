// bf16 grouped expert GEMM on 256 x 256 tiles ("MoE part 4" page, section 2: one launch for
// many expert GEMMs with differing row counts n_e; section 4.1: FC1 -> activation -> FC2).
//
//   gate/up:  h[r, :]   = silu(a[r] . W_gate,e^T) * (a[r] . W_up,e^T)   for r in segment e
//   down:     out[r, :] = h[r] . W_down,e^T
//   router:   part_s[t, :] = x[t, K_s] . W_r[:, K_s]^T over the s-th of k_split column ranges
//             ("EP / DeepEP explanation" page, section 2: logits z = sum_s part_s)
//
// A persistent workgroup of 4 waves (2 x 2) per CU computes 256 rows x 256 weight rows;
// each wave owns 128 x 128 as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16 (accumulators in
// the 256 AGPRs), so a 16-wide k-step reads 8 fragments from LDS for 16 MFMAs.  At 256 x
// 256 a CU loads 1 KB per 256 k-products: half the vector-memory instructions per flop of
// a 128 x 256 tile, whose loads keep the CU's address unit (one 16-byte-per-lane load per
// 16 clocks at best) busy most of the time.
//
// K advances in stages of 64 (128 bytes per row), all loads direct to LDS (16 bytes per
// lane).  LDS (160 KB) holds two buffers of activation rows (32 KB each) and a ring of
// three buffers of weight rows.  While stage ks is multiplied:
//   - k-steps 0-1 load the weight rows of stage ks+2 into the ring slot stage ks-1 used;
//   - after k-step 2 each wave waits for its loads of stage ks+1 (everything but the
//     weight rows just issued) and the workgroup synchronises;
//   - k-step 3 loads the activation rows of stage ks+2 into the buffer stage ks used, and
//     reads the first fragments of stage ks+1 while its MFMAs run.
// Weight rows are read once per m-tile and come from HBM, so they get the longer lead
// (1.25-1.75 stages); activation rows (a, or x through the layout's src_slot map) are
// re-read by the 8-28 n-blocks of an expert and mostly hit L2 (0.75-1 stage).  Load
// counters complete in order, so loads are issued in the order they are waited for.
//
// Every 16-byte chunk c of a row r sits in LDS slot c ^ key(r), key(r) = (r & 7) ^ ((r >> 3) & 1):
// a fragment read (32 rows, two chunks) and an 8-row load both touch all 64 banks once.
//
// The weight fragment is the MFMA's first operand, so a lane's accumulator holds one token
// row and runs of 4 adjacent output columns: the epilogue stores 8 bytes per lane.
//
// Ragged tiles: an expert's n_e rows are split into ceil(n_e / 256) tiles of equal size
// (a multiple of 32 rows).  32-row blocks are dealt to the two row waves in turn, and a
// wave skips the MFMAs and fragment reads of blocks without rows.
#include <utility>

#include "gemm_device.h"
#include "grouped_gemm.h"
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kTM = kWideTileRows;     // rows of a tile (256)
constexpr int kTN = 256;               // weight rows of a tile (gate/up: 128 W_gate + the same 128 W_up)
constexpr int kRowB = 128;             // bytes of K per row and stage
constexpr int kPart = kTM * kRowB;     // one stage of activation or weight rows (32 KB)
constexpr int kWBase = 2 * kPart;      // weight ring after the two activation buffers
constexpr int kLdsBytes = 5 * kPart;   // 160 KB
constexpr int kThreads = 256;
constexpr int kMB = 4, kNB = 4;        // 32 x 32 blocks per wave
constexpr int kLd = kPart / 1024 / 4;  // 1 KB loads per wave and part (8)
static_assert(kTM == kTN, "activation and weight parts have the same shape");

__device__ __forceinline__ int slot_key(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_wide_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_byte*)lds));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // loads: wave w moves the 8-row groups w, w + 4, ... of a part; lane l fills LDS slot l % 8
  // of row l / 8 of the group, so it loads chunk (l % 8) ^ key(row).  Bit 3 of every row of
  // such a group is the wave's parity.
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ slot_key(lrow + (wave & 1) * 8);

  const int n_cols = MODE == MODE_GATE_UP ? p.I : p.n_out;
  const int tile_cols = MODE == MODE_GATE_UP ? kTN / 2 : kTN;
  const int nN = (n_cols + tile_cols - 1) / tile_cols;
  // router: m-tiles of the single segment [0, rows); tiles ordered part -> n-block -> m-tile,
  // so with k_split = 8 each XCD's range is one column part (its slice of W_r stays in L2)
  const int mt_r = MODE == MODE_ROUTER ? (p.rows + kTM - 1) / kTM : 0;
  // routed tiles (expert -> n-block -> m-tile), then the shared segment's (m-tile -> n-block)
  const long long n_r = MODE == MODE_ROUTER ? static_cast<long long>(p.k_split) * mt_r * nN
                                            : static_cast<long long>(p.tile_prefix[p.E]) * nN;
  const long long n_s = MODE != MODE_ROUTER && p.shared_rows > 0
                            ? static_cast<long long>(p.tile_prefix[p.E + 1] - p.tile_prefix[p.E]) * nN
                            : 0;
  const int xcd = blockIdx.x % kNumXcd;
  const int slot = blockIdx.x / kNumXcd;
  const int per_xcd = gridDim.x / kNumXcd;
  // each XCD takes a contiguous range of the routed tiles and one of the shared segment's
  // (4 m-tiles x all n-blocks for an 8192-row shared expert: its rows are read once per XCD)
  const long long r_beg = n_r * xcd / kNumXcd, r_cnt = n_r * (xcd + 1) / kNumXcd - r_beg;
  const long long s_beg = n_s * xcd / kNumXcd, s_cnt = n_s * (xcd + 1) / kNumXcd - s_beg;
  const long long v_end = r_cnt + s_cnt;   // this XCD's tiles, numbered 0 .. v_end - 1
  auto tile_of = [&](long long v) __attribute__((always_inline)) {
    return v < r_cnt ? r_beg + v : n_r + s_beg + (v - r_cnt);
  };
  const int kspan = MODE == MODE_ROUTER ? p.K / p.k_split : p.K;   // K of one tile
  const int nk = kspan / 64;                                // even: kspan % 128 == 0
  const uint32_t rb = static_cast<uint32_t>(p.K) * 2;       // row bytes of both operands

  const int hk = lane >> 5;
  const int fkey = slot_key(lane & 31);
  int koff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) koff[s] = ((2 * s + hk) ^ fkey) * 16;
  int a_frag[kMB], b_frag[kNB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) a_frag[mb] = ((mb * 2 + wm) * 32 + (lane & 31)) * kRowB;
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    // gate/up: blocks 0-1 are W_gate rows, blocks 2-3 the same W_up rows
    const int r = MODE == MODE_GATE_UP ? (nb >> 1) * (kTN / 2) + wn * 64 + (nb & 1) * 32 + (lane & 31)
                                       : wn * 128 + nb * 32 + (lane & 31);
    b_frag[nb] = r * kRowB;
  }

  // Tiles: from the XCD's counter (dynamic), or every per_xcd-th of the XCD's range.  With
  // the counter, tiles adjacent in the order (the m-tiles sharing a weight panel, the
  // n-blocks sharing activation rows) start close together in time whatever the earlier
  // tiles cost.  Wave 0 takes the next index during the tile's second-to-last stage (late
  // enough that the take is still close to the start, early enough to hide its latency) and
  // hands it to the other waves at the tile boundary through the last word of ring slot 2
  // (no load writes that slot between a boundary and the first stage).
  int32_t* const tile_word = reinterpret_cast<int32_t*>(lds + kLdsBytes - 4);
  const bool dynamic = p.tile_counter != nullptr;
  int32_t grabbed = 0;   // (lane 0 of wave 0) the counter value taken for the next tile
  long long v = slot;
  if (dynamic) {
    if (tid == 0) *tile_word = atomicAdd(p.tile_counter + xcd, 1);
    __syncthreads();
    v = *tile_word;
  }
  if (v >= v_end) return;

  struct Tile {
    int m0, mend, mlast, c0, kp;   // (kp: the router's column part)
    const uint8_t* a;
    const uint8_t* b;
    uint32_t a_src[kLd], b_src[kLd];
  };
  auto setup = [&](long long L, Tile& t) __attribute__((always_inline)) {
    int e, mt_e, nblk, mtile, seg_lo, seg_hi, kp = 0;
    if (MODE == MODE_ROUTER) {
      e = 0;
      mt_e = mt_r;
      const long long per = static_cast<long long>(mt_r) * nN;
      kp = static_cast<int>(L / per);
      const int local = static_cast<int>(L - kp * per);
      nblk = local / mt_r;
      mtile = local % mt_r;
      seg_lo = 0;
      seg_hi = p.rows;
    } else if (L < n_r) {
      e = p.tile_expert[L / nN];
      const int pe = p.tile_prefix[e];
      mt_e = p.tile_prefix[e + 1] - pe;
      const long long local = L - static_cast<long long>(pe) * nN;
      nblk = static_cast<int>(local / mt_e);
      mtile = static_cast<int>(local % mt_e);
      expert_segment(p, e, seg_lo, seg_hi);
    } else {   // the shared segment [rows, rows + shared_rows), weights shared_b
      e = p.E;
      mt_e = p.tile_prefix[p.E + 1] - p.tile_prefix[p.E];
      const long long local = L - n_r;
      mtile = static_cast<int>(local / nN);
      nblk = static_cast<int>(local % nN);
      seg_lo = p.rows;
      seg_hi = p.rows + p.shared_rows;
    }
    const int rpt = ((seg_hi - seg_lo + mt_e - 1) / mt_e + 31) / 32 * 32;
    t.m0 = seg_lo + mtile * rpt;
    t.mend = t.m0 + rpt < seg_hi ? t.m0 + rpt : seg_hi;
    t.mlast = t.mend - 1 - t.m0;
    t.c0 = nblk * tile_cols;
    t.kp = kp;
    const int clast = n_cols - 1 - t.c0;
    // gathered operand: tile row r is row a_rows[m0 + r] / a_div of a (the launcher checks
    // that a_nrows * rb fits in 32 bits); rows past the segment or the matrix re-read the
    // last valid one
    t.a = p.a_rows ? p.a : p.a + static_cast<size_t>(t.m0) * rb;
    t.b = e < p.E ? p.b + static_cast<size_t>(e) * p.b_rows * rb : p.shared_b;
    if (MODE == MODE_ROUTER) {
      t.a += static_cast<size_t>(kp) * kspan * 2;
      t.b += static_cast<size_t>(kp) * kspan * 2;
    }
#pragma unroll
    for (int j = 0; j < kLd; ++j) {
      const int r = (wave + 4 * j) * 8 + lrow;   // tile row of this lane's loads
      int ra = r < t.mlast ? r : t.mlast;
      if (p.a_rows) {   // (the shared segment's row r is token r - rows)
        int tok = e < p.E ? p.a_rows[t.m0 + ra] / p.a_div : t.m0 + ra - p.rows;
        ra = tok < 0 ? 0 : (tok < p.a_nrows ? tok : p.a_nrows - 1);
      }
      t.a_src[j] = static_cast<uint32_t>(ra) * rb + lchunk * 16;
      uint32_t wr;
      if (MODE == MODE_GATE_UP) {
        const int c = r % (kTN / 2);
        const int cc = c < clast ? c : clast;
        wr = (r < kTN / 2 ? 0u : static_cast<uint32_t>(p.I)) + static_cast<uint32_t>(t.c0 + cc);
      } else {
        wr = static_cast<uint32_t>(t.c0 + (r < clast ? r : clast));
      }
      t.b_src[j] = wr * rb + lchunk * 16;
    }
  };
  // activation rows of stage ks into buffer buf; weight rows of stage ks into ring slot ws
  auto load_a = [&](const Tile& t, int ks, int buf, int j) __attribute__((always_inline)) {
    const uint32_t base =
        __builtin_amdgcn_readfirstlane(lds0 + static_cast<uint32_t>(buf * kPart + (wave + 4 * j) * 1024));
    dma16(t.a + static_cast<size_t>(ks) * kRowB + t.a_src[j], base);
  };
  auto load_w = [&](const Tile& t, int ks, int ws, int j) __attribute__((always_inline)) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(
        lds0 + static_cast<uint32_t>(kWBase + ws * kPart + (wave + 4 * j) * 1024));
    dma16(t.b + static_cast<size_t>(ks) * kRowB + t.b_src[j], base);
  };
  // prologue loads of a tile (stage 0 and 1); the caller waits for stage 0 and synchronises
  auto prologue = [&](const Tile& t) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kLd; ++j) load_a(t, 0, 0, j);
#pragma unroll
    for (int j = 0; j < kLd; ++j) load_w(t, 0, 0, j);
#pragma unroll
    for (int j = 0; j < kLd; ++j) load_w(t, 1, 1, j);
#pragma unroll
    for (int j = 0; j < kLd; ++j) load_a(t, 1, 1, j);
  };

  Tile cur;
  long long L = tile_of(v);
  setup(L, cur);
  prologue(cur);
  wait_vmcnt<2 * kLd>();   // stage 0 landed; stage 1 may be in flight
  block_barrier();

  for (;;) {
    const Tile& t = cur;   // (rewritten at the boundary, after the epilogue's last use)
    f32x16_t acc[kMB][kNB];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
      for (int j = 0; j < kNB; ++j) acc[i][j] = f32x16_t{};

    int act = ((t.mlast + 32) / 32 - wm + 1) / 2;   // 32-row blocks of this wave that hold rows
    act = act < 0 ? 0 : (act > kMB ? kMB : act);

    auto k_loop = [&](auto act_c) __attribute__((always_inline)) {
      constexpr int ACT = decltype(act_c)::value;
      constexpr int kReads = ACT > 0 ? ACT + kNB : 0;   // fragment reads per k-step
      uint4 f0a[kMB], f0b[kNB], f1a[kMB], f1b[kNB];
      // fragment read r of a k-step, in the order the MFMAs use them: a0, b0..b3, a1, a2, a3
      auto read_frag = [&](int r, int aoff, int boff, int s, uint4(&fa)[kMB], uint4(&fb)[kNB])
          __attribute__((always_inline)) {
        if (r == 0) fa[0] = *reinterpret_cast<const uint4*>(lds + aoff + a_frag[0] + koff[s]);
        else if (r <= kNB) fb[r - 1] = *reinterpret_cast<const uint4*>(lds + boff + b_frag[r - 1] + koff[s]);
        else fa[r - kNB] = *reinterpret_cast<const uint4*>(lds + aoff + a_frag[r - kNB] + koff[s]);
      };
      // the 16 MFMAs of a k-step on (ca, cb).  After MFMA i come fragment read i / 2 of the
      // next k-step (into na, nb, when READ) and then between(i), all held in place by
      // scheduling fences: the wave never stalls on a burst of LDS or memory instructions
      // while the matrix pipe has nothing queued.
      auto mfma_step = [&]<bool READ>(uint4(&ca)[kMB], uint4(&cb)[kNB], uint4(&na)[kMB], uint4(&nb)[kNB],
                                      int aoff, int boff, int s, auto&& between) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kMB * kNB; ++i) {
          if (i / kNB < ACT) acc[i / kNB][i % kNB] = mma_bf16(cb[i % kNB], ca[i / kNB], acc[i / kNB][i % kNB]);
          __builtin_amdgcn_sched_barrier(0);
          if (READ && (i & 1) == 0 && i / 2 < kReads) read_frag(i / 2, aoff, boff, s, na, nb);
          between(i);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      auto nothing = [](int) __attribute__((always_inline)) {};

#pragma unroll
      for (int r = 0; r < kReads; ++r) read_frag(r, 0, kWBase, 0, f0a, f0b);
      // stage ks: activation rows in buffer PAR = ks & 1, weight rows in ring slot ws = ks % 3.
      // FULL: stage ks+2 exists; NEXT: stage ks+1 exists
      auto stage = [&]<bool FULL, bool NEXT, int PAR>(int ks, int ws) __attribute__((always_inline)) {
        constexpr int buf = PAR, nbuf = PAR ^ 1;
        const int ws1 = ws == 2 ? 0 : ws + 1, ws2 = ws1 == 2 ? 0 : ws1 + 1;
        const int aoff = buf * kPart, boff = kWBase + ws * kPart;
        mfma_step.template operator()<true>(f0a, f0b, f1a, f1b, aoff, boff, 1, [&](int i) __attribute__((always_inline)) {
          if (FULL && (i & 3) == 1) load_w(t, ks + 2, ws2, i >> 2);
        });
        mfma_step.template operator()<true>(f1a, f1b, f0a, f0b, aoff, boff, 2, [&](int i) __attribute__((always_inline)) {
          if (FULL && (i & 3) == 1) load_w(t, ks + 2, ws2, 4 + (i >> 2));
        });
        mfma_step.template operator()<true>(f0a, f0b, f1a, f1b, aoff, boff, 3, nothing);
        if constexpr (NEXT) {
          // stage ks+1 (activation rows from k-step 3 of stage ks-1, weight rows from k-steps
          // 0-1 of stage ks-1) has landed once at most this stage's weight loads remain
          wait_lgkmcnt_all();
          if constexpr (FULL) wait_vmcnt<kLd>();
          else wait_vmcnt<0>();
          block_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_step.template operator()<NEXT>(f1a, f1b, f0a, f0b, nbuf * kPart, kWBase + ws1 * kPart, 0,
                                            [&](int i) __attribute__((always_inline)) {
          if (FULL && (i & 1) == 1) load_a(t, ks + 2, buf, i >> 1);
          // second-to-last stage (its wait for loads is behind it): take the next tile
          if (!FULL && NEXT && i == 0 && dynamic && tid == 0) grabbed = atomicAdd(p.tile_counter + xcd, 1);
        });
      };
      int ks = 0, ws = 0;
      for (; ks < nk - 2; ks += 2) {
        stage.template operator()<true, true, 0>(ks, ws);
        ws = ws == 2 ? 0 : ws + 1;
        stage.template operator()<true, true, 1>(ks + 1, ws);
        ws = ws == 2 ? 0 : ws + 1;
      }
      stage.template operator()<false, true, 0>(nk - 2, ws);
      ws = ws == 2 ? 0 : ws + 1;
      stage.template operator()<false, false, 1>(nk - 1, ws);
    };
    [&]<int... A>(std::integer_sequence<int, A...>) {
      ((act == A ? k_loop(std::integral_constant<int, A>{}) : void()), ...);
    }(std::make_integer_sequence<int, kMB + 1>{});

    // ---- tile boundary: every wave is past its last LDS reads; the next tile is known
    block_barrier();
    long long vn = v + per_xcd;
    if (dynamic) {
      if (tid == 0) *tile_word = grabbed;
      wait_lgkmcnt_all();
      block_barrier();
      vn = *tile_word;
    }
    const bool more = vn < v_end;
    const long long Ln = more ? tile_of(vn) : 0;

    // ---- epilogue: lane l holds token row (2 mb + wm) * 32 + l % 32 of the tile and, in
    // registers 4q .. 4q+3 of block nb, output columns nb * 32 + 8q + 4 (l / 32) + 0..3:
    // one 8-byte store per run (16 bytes for fp32 router sums; n_cols % 4 == 0, so a run is
    // all in or all out)
    // down with gates: a routed row carries the gate of its slot (the shared rows gate 1).
    // The gates are loaded first and waited for once: a load pending across the stores'
    // row and column branches would make the compiler wait for every store before the next.
    float gsv[kMB];
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      const int r = t.m0 + (mb * 2 + wm) * 32 + (lane & 31);
      gsv[mb] = 1.0f;
      if (MODE == MODE_DOWN && p.row_gate != nullptr && r < p.rows && r < t.mend) {
        int sl = p.row_slot[r];
        sl = sl < 0 ? 0 : (sl < p.rows ? sl : p.rows - 1);
        gsv[mb] = p.row_gate[sl];
      }
    }
    if (MODE == MODE_DOWN) wait_vmcnt<0>();
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      const int r = t.m0 + (mb * 2 + wm) * 32 + (lane & 31);
      if (r >= t.mend) continue;
      const float gs = gsv[mb];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (MODE == MODE_GATE_UP) {
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const int col = t.c0 + wn * 64 + nb * 32 + 8 * q + 4 * hk;
            if (col >= n_cols) continue;
            float hv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float g = acc[mb][nb][4 * q + u];
              const float up = acc[mb][nb + 2][4 * q + u];
              hv[u] = silu_f32(g) * up;
            }
            if (p.au != nullptr) {   // the pre-activations, for the backward pass
              const f32x16_t& ga = acc[mb][nb];
              const f32x16_t& ua = acc[mb][nb + 2];
              uint16_t* arow = reinterpret_cast<uint16_t*>(p.au) + static_cast<size_t>(r) * 2 * p.I;
              *reinterpret_cast<uint2*>(arow + col) =
                  make_uint2(pack_bf16x2(ga[4 * q], ga[4 * q + 1]), pack_bf16x2(ga[4 * q + 2], ga[4 * q + 3]));
              *reinterpret_cast<uint2*>(arow + p.I + col) =
                  make_uint2(pack_bf16x2(ua[4 * q], ua[4 * q + 1]), pack_bf16x2(ua[4 * q + 2], ua[4 * q + 3]));
            }
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + static_cast<size_t>(r) * p.I + col) =
                make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
          }
        } else if (MODE == MODE_ROUTER) {
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) {
            const int col = t.c0 + wn * 128 + nb * 32 + 8 * q + 4 * hk;
            if (col >= n_cols) continue;
            const f32x16_t& a = acc[mb][nb];
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) +
                                       (static_cast<size_t>(t.kp) * p.rows + r) * p.n_out + col) =
                make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
          }
        } else {
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) {
            const int col = t.c0 + wn * 128 + nb * 32 + 8 * q + 4 * hk;
            if (col >= n_cols) continue;
            const f32x16_t& a = acc[mb][nb];
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + static_cast<size_t>(r) * p.n_out + col) =
                make_uint2(pack_bf16x2(a[4 * q] * gs, a[4 * q + 1] * gs),
                           pack_bf16x2(a[4 * q + 2] * gs, a[4 * q + 3] * gs));
          }
        }
      }
    }
    if (!more) break;
    // the next tile's first stages load while these stores drain: the wait below covers the
    // stores (older) and stage 0, and leaves stage 1 in flight
    setup(Ln, cur);
    prologue(cur);
    wait_vmcnt<2 * kLd>();
    block_barrier();
    v = vn;
    L = Ln;
  }
}

}  // namespace

hipError_t launch_grouped_gemm_wide(int mode, const GemmArgs& p, hipStream_t s) {
  const dim3 grid(256), block(kThreads);   // persistent: one workgroup per CU, a multiple of the 8 XCDs
  if (mode == MODE_GATE_UP)
    hipLaunchKernelGGL(grouped_gemm_wide_kernel<MODE_GATE_UP>, grid, block, 0, s, p);
  else if (mode == MODE_DOWN)
    hipLaunchKernelGGL(grouped_gemm_wide_kernel<MODE_DOWN>, grid, block, 0, s, p);
  else
    hipLaunchKernelGGL(grouped_gemm_wide_kernel<MODE_ROUTER>, grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
