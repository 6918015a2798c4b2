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
// row and runs of 4 adjacent output columns; pairing the runs of lanes l and l + 32 (one
// cross-lane exchange), the epilogue stores 16 bytes per lane.
//
// Ragged tiles: an expert's n_e rows are split into ceil(n_e / 256) tiles of equal size
// (a multiple of 32 rows).  A tile with an even number R of 32-row blocks deals them to the
// two row waves in turn, and a wave skips the MFMAs and fragment reads of blocks without
// rows: R / 2 row blocks x 4 column blocks per wave.  With R odd that layout leaves one row
// wave a block short, so a tile with R = 1, 3 or 5 runs 1 x 4 instead: each wave takes all
// R row blocks and 64 of the 256 weight rows (gate/up: 32 W_gate rows and the same 32 W_up
// rows), 2 R MFMAs per k-step against (R + 1) / 2 x 4.  The accumulators are the same 16
// blocks in both layouts; only the epilogue's row and column of each block differ.
//
// Down GEMM, experts of 257..320 rows: split in two, each half would stream the expert's whole
// weight panel; instead the expert runs as one tile of 320 rows x 128 weight rows (5 x 2 blocks
// per wave, 160 accumulators), whose LDS holds two 40 KB activation buffers and a five-slot
// ring of 16 KB weight stages, so the weight rows load 3.25-3.75 stages ahead.  These tiles
// come first, from counters of their own.
#include <utility>

#include "gemm_device.h"
#include "grouped_gemm.h"
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kRowB = 128;      // bytes of K per activation row and stage
constexpr int kThreads = 256;
constexpr int kMB1 = 5, kNB1 = 2;   // at most 5 row blocks x 2 column blocks (1 x 4 layout)

// Shape of a tile and of its LDS.  G = 0: 256 rows x 256 weight rows, two activation
// buffers and a three-slot weight ring (5 x 32 KB).  G = 1 (down GEMM, an expert of 257-320
// rows in one tile): 320 rows x 128 weight rows, two activation buffers of 40 KB and a
// five-slot weight ring of 16 KB slots, so the weight rows load 3.25-3.75 stages ahead.
// G = 2 (gate/up, an expert of 257-320 rows in one tile): 320 rows x 256 weight rows, two
// activation buffers of 40 KB and a five-slot ring of 16 KB half-stages of weights (K = 32:
// 64 bytes per row, chunks swizzled like the e4m3 rows), so the weight rows load 1-2 stages
// ahead; its fifth row block's accumulators live in VGPRs (the first 256 in the AGPRs).  W8:
// e4m3 weight rows of 64 bytes per stage (G = 0 only).
template <int G, bool W8>
struct Geo {
  static constexpr int TM = G ? kWideTallRows : kWideTileRows;
  static constexpr int TN = G == 1 ? 128 : 256;
  static constexpr int MB = TM / 64, NB = TN / 64;   // 32 x 32 blocks per wave (2 x 2 layout)
  static constexpr int WRowB = W8 || G == 2 ? 64 : kRowB;   // bytes of a weight row per stage (G = 2: half)
  static constexpr int PartA = TM * kRowB;           // one stage of activation rows
  static constexpr int WPart = TN * WRowB;           // one stage of weight rows
  static constexpr int WS = G != 0 ? 5 : 3;          // weight ring slots
  static constexpr int LdA = PartA / 4096;           // 1 KB loads per wave and stage (8; 10)
  static constexpr int LdW = WPart / 4096;           // (8, W8 4; 4)
  static constexpr int StageLd = LdW + (W8 ? 1 : 0); // + the scale gather (W8)
  static constexpr int WBase = 2 * PartA;            // weight ring after the activation buffers
  static constexpr int SBase = WBase + WS * WPart;   // (W8) scale ring: a slot of 1 KB per weight slot
  static constexpr int LdsTot = SBase + (W8 ? WS * 1024 : 0);
  static_assert(!W8 || G != 2, "e4m3 weights: 256 x 256 and 320 x 128 tiles");
  static_assert(TM % 64 == 0 && TN % 64 == 0 && (TN / 2) % 32 == 0, "2 x 2 waves of 32-row blocks");
};
static_assert(Geo<1, false>::LdsTot <= Geo<0, false>::LdsTot && Geo<2, false>::LdsTot <= Geo<0, false>::LdsTot,
              "every shape fits the kernel's LDS");
// the kernel's LDS array (W8: the 320 x 128 tiles' five slots of activation, weight and scale
// stages take the most)
template <bool W8>
constexpr int kLdsBytes = W8 ? (Geo<1, true>::LdsTot > Geo<0, true>::LdsTot ? Geo<1, true>::LdsTot : Geo<0, true>::LdsTot)
                             : Geo<0, false>::LdsTot;
static_assert(kLdsBytes<true> <= Geo<0, false>::LdsTot, "the e4m3 shapes fit the LDS");

__device__ __forceinline__ int slot_key(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// r * b + c for a row r and a row size b below 2^24 whose product fits 32 bits, as one 24-bit
// multiply-add with a 32-bit result: a plain 32-bit multiply-add is formed as a 64-bit
// v_mad_u64_u32 whose register pair stays live (and is spilled) when the value is kept
// through the K loop.
__device__ __forceinline__ uint32_t row_off(uint32_t r, uint32_t b, uint32_t c) { return __umul24(r, b) + c; }

// A raw buffer resource over `bytes` bytes from `base`: a store whose 16 bytes do not all lie
// inside writes nothing.
typedef __amdgpu_buffer_rsrc_t buf_rsrc_t;
__device__ __forceinline__ buf_rsrc_t make_window(void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ void store16(buf_rsrc_t w, uint32_t off, uint4 v) {
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(u32x4v{v.x, v.y, v.z, v.w}, w, static_cast<int>(off), 0, 0);
}

// Lanes l and l + 32 hold the same output row: lane l < 32 columns 8 q .. 8 q + 3 of register
// group q, lane l + 32 columns 8 q + 4 .. 8 q + 7.  Exchanging group 2 u + 1 of lane l with
// group 2 u of lane l + 32 (gfx950's v_permlane32_swap) leaves lane l with columns 16 u .. 16 u + 7
// and lane l + 32 with 16 u + 8 .. 16 u + 15, in order: one 16-byte store per lane.  lo and hi
// are this lane's groups 2 u and 2 u + 1 as packed bf16; every lane must take part.
__device__ __forceinline__ uint4 lane_pair(uint2 lo, uint2 hi) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t a = __builtin_amdgcn_permlane32_swap(lo.x, hi.x, false, false);
  const u32x2_t b = __builtin_amdgcn_permlane32_swap(lo.y, hi.y, false, false);
  return make_uint4(a[0], b[0], a[1], b[1]);
}
// (W8) 64-byte weight rows: chunk c of row r sits in slot c ^ key4(r); a fragment read (32 rows,
// 8 bytes of one chunk per lane) then spreads over 16 of the 32 eight-byte bank pairs
__device__ __forceinline__ int key4(int r) { return (r >> 2) & 3; }

// f(std::integral_constant<int, I>{}) for I = 0 .. N-1, in order
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) { (f(std::integral_constant<int, I>{}), ...); }(
      std::make_integer_sequence<int, N>{});
}

// The tiles of one shape, from the XCD's counter: G = 0 the schedule's m-tiles (routed, then
// the shared segment's), G = 1 one tile per listed expert.  lds is the kernel's LDS array.
template <int MODE, bool W8, int G>
__device__ __forceinline__ void run_tiles(const GemmArgs& p, uint8_t* lds) {
  using S = Geo<G, W8>;
  constexpr int kTM = S::TM, kTN = S::TN, kMB = S::MB, kNB = S::NB;
  constexpr int kWRowB = S::WRowB, kPartA = S::PartA, kWPart = S::WPart, kWS = S::WS;
  constexpr int kLdA = S::LdA, kLdW = S::LdW, kStageLd = S::StageLd;
  constexpr int kWBase = S::WBase, kSBase = S::SBase;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_byte*)lds));

  // the 1 x 4 layout for 256 x 256 gate/up tiles only: the down GEMM's epilogue would need the
  // gates of twice the rows per lane, and the extra registers cost its K loop more than the
  // layout saves
  constexpr bool kLay1 = MODE == MODE_GATE_UP && G != 1 && !W8;   // (W8: the scales are read per 2 x 2 block)
  // row blocks a wave holds in the 1 x 4 layout: 5 (256 x 256 tiles), 10 (320 x 256 tiles,
  // which always run 1 x 4: a 9-block expert then costs 18 MFMAs per k-step and wave, not 20)
  constexpr int kMBL = G == 2 ? 2 * kMB : kMB1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS bases stay scalar
  const int wm = wave >> 1, wn = wave & 1;
  // loads: wave w moves the 8-row groups w, w + 4, ... of a part; lane l fills LDS slot l % 8
  // of row l / 8 of the group, so it loads chunk (l % 8) ^ key(row).  Bit 3 of every row of
  // such a group is the wave's parity.

  const int n_cols = MODE == MODE_GATE_UP ? p.I : p.n_out;
  const int tile_cols = MODE == MODE_GATE_UP ? kTN / 2 : kTN;
  const int nN = (n_cols + tile_cols - 1) / tile_cols;
  // router: m-tiles of the single segment [0, rows); tiles ordered part -> n-block -> m-tile,
  // so with k_split = 8 each XCD's range is one column part (its slice of W_r stays in L2)
  const int mt_r = MODE == MODE_ROUTER ? (p.rows + kTM - 1) / kTM : 0;
  // routed tiles (expert -> n-block -> m-tile), then the shared segment's (m-tile -> n-block);
  // G = 1: listed expert -> n-block
  // (tile numbers are 32-bit: the launcher keeps 8 x the tile count below 2^31)
  const int n_r = MODE == MODE_ROUTER ? p.k_split * mt_r * nN
                  : G ? p.tall_list[0] * nN
                      : p.tile_prefix[p.E] * nN;
  const int n_s = G == 0 && MODE != MODE_ROUTER && p.shared_rows > 0
                            ? (p.tile_prefix[p.E + 1] - p.tile_prefix[p.E]) * nN
                            : 0;
  int32_t* const counter = G ? p.tall_counter : p.tile_counter;
  const int xcd = blockIdx.x % kNumXcd;
  const int slot = blockIdx.x / kNumXcd;
  const int per_xcd = gridDim.x / kNumXcd;
  // each XCD takes a contiguous range of the routed tiles and one of the shared segment's
  // (4 m-tiles x all n-blocks for an 8192-row shared expert: its rows are read once per XCD)
  const int r_beg = n_r * xcd / kNumXcd, r_cnt = n_r * (xcd + 1) / kNumXcd - r_beg;
  const int s_beg = n_s * xcd / kNumXcd, s_cnt = n_s * (xcd + 1) / kNumXcd - s_beg;
  const int v_end = r_cnt + s_cnt;   // this XCD's tiles, numbered 0 .. v_end - 1
  auto tile_of = [&](int v) __attribute__((always_inline)) {
    return v < r_cnt ? r_beg + v : n_r + s_beg + (v - r_cnt);
  };
  // tile v of XCD x's range
  auto tile_of_x = [&](int x, int v) __attribute__((always_inline)) {
    const int rb0 = n_r * x / kNumXcd, rc0 = n_r * (x + 1) / kNumXcd - rb0;
    return v < rc0 ? rb0 + v : n_r + n_s * x / kNumXcd + (v - rc0);
  };
  const int kspan = MODE == MODE_ROUTER ? p.K / p.k_split : p.K;   // K of one tile
  const int nk = kspan / 64;                                // even: kspan % 128 == 0
  const uint32_t rb = static_cast<uint32_t>(p.K) * 2;       // row bytes of the activations
  const uint32_t rbw = W8 ? static_cast<uint32_t>(p.K) : rb;   // row bytes of the weights
  const uint32_t kblk = static_cast<uint32_t>(p.K) / 128;      // (W8) scale blocks per weight row

  // first row of the wave's activation block m and weight block n, per layout (gate/up in
  // the 2 x 2 layout: the first NB / 2 weight blocks are W_gate rows, the rest the same W_up
  // rows; in the 1 x 4 layout wave w holds weight rows 64 w .. 64 w + 63, gate/up: W_gate
  // rows 32 w .. 32 w + 31 and the same W_up rows)
  auto a_row = [&](int lay, int m) __attribute__((always_inline)) { return lay ? m * 32 : (2 * m + wm) * 32; };
  auto b_row = [&](int lay, int n) __attribute__((always_inline)) {
    if (MODE == MODE_GATE_UP)
      return lay ? n * (kTN / 2) + wave * 32
                 : (n / (kNB / 2)) * (kTN / 2) + wn * (kNB / 2) * 32 + (n % (kNB / 2)) * 32;
    return lay ? wave * 64 + n * 32 : wn * kNB * 32 + n * 32;
  };

  // Tiles: from the XCD's counter (dynamic), or every per_xcd-th of the XCD's range.  With
  // the counter, tiles adjacent in the order (the m-tiles sharing a weight panel, the
  // n-blocks sharing activation rows) start close together in time whatever the earlier
  // tiles cost.  Wave 0 takes the next index early in the tile's second-to-last stage (late
  // enough that the take is still close to the start, early enough to hide its latency) and
  // hands it to the other waves at the tile boundary through the last word of the LDS array
  // (in the last weight ring slot, or the last scale slot with W8; no load writes that slot
  // between a boundary and the first stage).
  int32_t* const tile_word = reinterpret_cast<int32_t*>(lds + kLdsBytes<W8> - 4);
  const bool dynamic = counter != nullptr;
  // The end of a launch: every XCD's range takes about the same time, but not exactly, and a
  // workgroup whose range runs out would wait for the slowest XCD.  The last kTailT tiles of
  // every range (G = 0, the launch's last tiles) form a tail shared by all XCDs: a workgroup
  // takes its own range's tiles from its XCD's counter and then tail tiles from one shared
  // counter, which deals them XCD by XCD in turn.  kTailT: one tile per workgroup of an XCD,
  // two when K < 4096 (shorter tiles); none when a range is shorter than that.
  int32_t* const tail_ctr = p.tile_counter + kNumXcd;
  const int tail_per = G == 0 && MODE != MODE_ROUTER && dynamic ? per_xcd * (p.K < 4096 ? 2 : 1) : 0;
  const int kTailT = n_r / kNumXcd + n_s / kNumXcd >= tail_per ? tail_per : 0;
  constexpr int32_t kTailBit = 1 << 30, kTileMask = kTailBit - 1;   // (tile numbers < 2^28)
  // (lane 0 of wave 0) the tile word for a counter value g taken from the tail counter (tail) or
  // this XCD's: the tile's number, with kTailBit for a tail tile, or -1 when none is left
  auto resolve = [&](int g, bool tail) __attribute__((always_inline)) -> int32_t {
    if (!tail && g >= v_end - kTailT) {   // (this XCD's own tiles are all taken)
      if (kTailT == 0) return -1;
      tail = true;
      g = atomicAdd(tail_ctr, 1);
    }
    if (!tail) return tile_of(g);
    if (g >= kNumXcd * kTailT) return -1;
    const int x = g % kNumXcd;   // tail tile g / kNumXcd of XCD x's range
    const int v_end_x = (n_r * (x + 1) / kNumXcd - n_r * x / kNumXcd) + (n_s * (x + 1) / kNumXcd - n_s * x / kNumXcd);
    return kTailBit | tile_of_x(x, v_end_x - kTailT + g / kNumXcd);
  };
  int v = slot;
  int L = 0, tail_mode = 0;   // (the current tile is a tail tile: the next take is the tail's)
  if (dynamic) {
    __syncthreads();   // (after a previous shape's tiles: every wave has read the word)
    if (tid == 0) *tile_word = resolve(atomicAdd(counter + xcd, 1), false);
    __syncthreads();
    const int32_t word = __builtin_amdgcn_readfirstlane(*tile_word);
    if constexpr (G == 2) block_barrier();   // (its prologue writes the slot that holds the word)
    if (word < 0) return;
    L = word & kTileMask;
    tail_mode = word >> 30;
  } else {
    if (v >= v_end) return;
    L = tile_of(v);
  }

  struct Tile {
    int m0, mend, mlast, c0, kp;   // (kp: the router's column part)
    const uint8_t* a;
    const uint8_t* b;
    const uint8_t* sc;             // (W8) the expert's scales [n_out, K / 128]
    uint32_t a_src[kLdA], b_src[kLdW];
    uint32_t s_src;                // (W8) this lane's scale row offset
  };
  auto setup = [&](int L, Tile& t) __attribute__((always_inline)) {
    // the lane's load row and chunk, rebuilt here from the lane id: values kept across the
    // tile loop are spilled, and their reloads' count waits would also wait for the
    // epilogue's stores and the first loads of the tile
    const uint32_t ln = opaque_lane();
    const int lrow = static_cast<int>(ln >> 3);
    const int lchunk = static_cast<int>(ln & 7) ^ slot_key(lrow + (wave & 1) * 8);
    int e, mt_e, nblk, mtile, seg_lo, seg_hi, kp = 0;
    if (MODE == MODE_ROUTER) {
      e = 0;
      mt_e = mt_r;
      const int per = mt_r * nN;
      kp = static_cast<int>(L / per);
      const int local = L - kp * per;
      nblk = local / mt_r;
      mtile = local % mt_r;
      seg_lo = 0;
      seg_hi = p.rows;
    } else if (G != 0) {   // one tile per listed expert: all of its rows
      e = p.tall_list[1 + L / nN];
      mt_e = 1;
      nblk = L % nN;
      mtile = 0;
      expert_segment(p, e, seg_lo, seg_hi);
    } else if (L < n_r) {
      e = p.tile_expert[L / nN];
      const int pe = p.tile_prefix[e];
      mt_e = p.tile_prefix[e + 1] - pe;
      const int local = L - pe * nN;
      nblk = local / mt_e;
      mtile = local % mt_e;
      expert_segment(p, e, seg_lo, seg_hi);
    } else {   // the shared segment [rows, rows + shared_rows), weights shared_b
      e = p.E;
      mt_e = p.tile_prefix[p.E + 1] - p.tile_prefix[p.E];
      const int local = L - n_r;
      mtile = local / nN;
      nblk = local % nN;
      seg_lo = p.rows;
      seg_hi = p.rows + p.shared_rows;
    }
    int rpt = ((seg_hi - seg_lo + mt_e - 1) / mt_e + 31) / 32 * 32;
    rpt = rpt < kTM ? rpt : kTM;   // (G = 1: the list holds experts of at most kTM rows)
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
    t.b = e < p.E ? p.b + static_cast<size_t>(e) * p.b_rows * rbw : p.shared_b;
    // (W8) the weight row holding tile weight row r (gate/up: W_gate rows, then the same W_up
    // rows; columns past the output re-read the last one)
    auto w_row = [&](int r) __attribute__((always_inline)) -> uint32_t {
      if (MODE == MODE_GATE_UP) {
        const int c = r % (kTN / 2);
        return (r < kTN / 2 ? 0u : static_cast<uint32_t>(p.I)) + static_cast<uint32_t>(t.c0 + (c < clast ? c : clast));
      }
      return static_cast<uint32_t>(t.c0 + (r < clast ? r : clast));
    };
    if constexpr (W8) {
      t.sc = reinterpret_cast<const uint8_t*>(e < p.E ? p.b_scale + static_cast<size_t>(e) * p.b_rows * kblk
                                                      : p.shared_b_scale);
      // scale gather: wave w's lane l fetches the scale of tile weight row 64 w + l
      t.s_src = w_row(wave * 64 + static_cast<int>(ln)) * kblk * 4;
    }
    if (MODE == MODE_ROUTER) {
      t.a += static_cast<size_t>(kp) * kspan * 2;
      t.b += static_cast<size_t>(kp) * kspan * 2;
    }
    int ra[kLdA];   // operand row of each of this lane's loads
#pragma unroll
    for (int j = 0; j < kLdA; ++j) {
      const int r = (wave + 4 * j) * 8 + lrow;   // tile row of this lane's loads
      ra[j] = r < t.mlast ? r : t.mlast;
    }
    if (p.a_rows) {   // (the shared segment's row r is token r - rows)
      int tok[kLdA];
      if (e < p.E) {
        // every index load issued before the first is used: one memory latency, not kLdA
#pragma unroll
        for (int j = 0; j < kLdA; ++j) tok[j] = p.a_rows[t.m0 + ra[j]];
#pragma unroll
        for (int j = 0; j < kLdA; ++j) tok[j] /= p.a_div;
      } else {
#pragma unroll
        for (int j = 0; j < kLdA; ++j) tok[j] = t.m0 + ra[j] - p.rows;
      }
#pragma unroll
      for (int j = 0; j < kLdA; ++j) ra[j] = tok[j] < 0 ? 0 : (tok[j] < p.a_nrows ? tok[j] : p.a_nrows - 1);
    }
#pragma unroll
    for (int j = 0; j < kLdA; ++j) t.a_src[j] = row_off(static_cast<uint32_t>(ra[j]), rb, lchunk * 16);
#pragma unroll
    for (int j = 0; j < kLdW; ++j) {
      if constexpr (W8) {
        // 64-byte rows: load j fills the 16-row group wave + 4 j; lane l fills LDS slot l % 4
        // of row l / 4 of the group, so it loads chunk (l % 4) ^ key4(row)
        const int r8 = (wave + 4 * j) * 16 + static_cast<int>(ln >> 2);
        t.b_src[j] = row_off(w_row(r8), rbw, static_cast<uint32_t>((ln & 3) ^ key4(r8)) * 16);
      } else if constexpr (G == 2) {
        // half-stage rows of 64 bytes, laid out like the e4m3 rows; gate/up row mapping
        const int r8 = (wave + 4 * j) * 16 + static_cast<int>(ln >> 2);
        const int c = r8 % (kTN / 2);
        const int cc = c < clast ? c : clast;
        const uint32_t wr = (r8 < kTN / 2 ? 0u : static_cast<uint32_t>(p.I)) + static_cast<uint32_t>(t.c0 + cc);
        t.b_src[j] = row_off(wr, rb, static_cast<uint32_t>((ln & 3) ^ key4(r8)) * 16);
      } else {
        const int r = (wave + 4 * j) * 8 + lrow;   // tile weight row of this lane's loads
        uint32_t wr;
        if (MODE == MODE_GATE_UP) {
          const int c = r % (kTN / 2);
          const int cc = c < clast ? c : clast;
          wr = (r < kTN / 2 ? 0u : static_cast<uint32_t>(p.I)) + static_cast<uint32_t>(t.c0 + cc);
        } else {
          wr = static_cast<uint32_t>(t.c0 + (r < clast ? r : clast));
        }
        t.b_src[j] = row_off(wr, rb, lchunk * 16);
      }
    }
  };
  // activation rows of stage ks into buffer buf; weight rows of stage ks into ring slot ws.
  // Load J of a part fills its 8-row group wave + 4 J: LDS part base + wave * 1 KB, plus J * 4 KB
  // as a constant of the instruction.
  const uint32_t lds_wave = lds0 + static_cast<uint32_t>(wave) * 1024;
  auto load_a = [&]<int J>(const Tile& t, int ks, int buf) __attribute__((always_inline)) {
    dma16s<J * 4096>(t.a + static_cast<size_t>(ks) * kRowB, t.a_src[J], lds_wave + buf * kPartA);
  };
  auto load_w = [&]<int J>(const Tile& t, int ks, int ws) __attribute__((always_inline)) {
    dma16s<J * 4096>(t.b + static_cast<size_t>(ks) * kWRowB, t.b_src[J], lds_wave + kWBase + ws * kWPart);
  };
  // (W8) the scales of stage ks (block ks / 2) of the tile's 256 weight rows into scale slot ws
  auto load_s = [&](const Tile& t, int ks, int ws) __attribute__((always_inline)) {
    dma4s<0>(t.sc + static_cast<size_t>(ks >> 1) * 4, t.s_src,
             lds0 + static_cast<uint32_t>(kSBase + ws * 1024 + wave * 256));
  };
  // prologue loads of a tile: activation rows of stage 0, weight rows of stages 0 .. kWS - 2
  // (those that exist), activation rows of stage 1
  auto prologue_loads = [&](const Tile& t) __attribute__((always_inline)) {
    if constexpr (G == 2) {
      // activation rows of stage 0, weight halves 0-3 (stages 0 and 1), activation rows of
      // stage 1, weight half 4 (when K holds it: nk is even, so nk >= 4)
      static_for<kLdA>([&](auto j) __attribute__((always_inline)) { load_a.template operator()<j>(t, 0, 0); });
      static_for<4>([&](auto hc) __attribute__((always_inline)) {
        constexpr int h = decltype(hc)::value;
        static_for<kLdW>([&](auto j) __attribute__((always_inline)) { load_w.template operator()<j>(t, h, h); });
      });
      static_for<kLdA>([&](auto j) __attribute__((always_inline)) { load_a.template operator()<j>(t, 1, 1); });
      if (nk >= 4)
        static_for<kLdW>([&](auto j) __attribute__((always_inline)) { load_w.template operator()<j>(t, 4, 4); });
      return;
    }
    static_for<kLdA>([&](auto j) __attribute__((always_inline)) { load_a.template operator()<j>(t, 0, 0); });
    static_for<kLdW>([&](auto j) __attribute__((always_inline)) { load_w.template operator()<j>(t, 0, 0); });
    if constexpr (W8) load_s(t, 0, 0);
    static_for<kWS - 2>([&](auto ic) __attribute__((always_inline)) {
      constexpr int st = decltype(ic)::value + 1;
      if (G == 0 || st < nk) {   // (256 x 256: nk >= 2)
        static_for<kLdW>([&](auto j) __attribute__((always_inline)) { load_w.template operator()<j>(t, st, st); });
        if constexpr (W8) load_s(t, st, st);
      }
    });
    static_for<kLdA>([&](auto j) __attribute__((always_inline)) { load_a.template operator()<j>(t, 1, 1); });
  };
  // then the wait for stage 0 and the barrier: stage 0 landed once at most the later stages'
  // loads and the AFTER memory instructions issued behind them remain
  auto prologue_wait = [&]<int AFTER>() __attribute__((always_inline)) {
    if constexpr (G == 2) {   // (halves 2, 3, stage 1's activations and half 4 may remain)
      if (nk >= 4) wait_vmcnt<3 * kLdW + kLdA + AFTER>();
      else wait_vmcnt<2 * kLdW + kLdA + AFTER>();
    }
    else if (G == 0 || nk >= kWS - 1) wait_vmcnt<(kWS - 2) * kStageLd + kLdA + AFTER>();
    else wait_vmcnt<0>();
    block_barrier();
  };

  Tile cur;
  setup(L, cur);
  prologue_loads(cur);
  prologue_wait.template operator()<0>();

  for (;;) {
    const Tile& t = cur;   // (rewritten at the boundary, after the epilogue's last use)
    // (lane 0 of wave 0) the counter value taken for the next tile; per tile, so that it is
    // live only from the take to the boundary (carried across tiles it was spilled, and the
    // take's pending result made the compiler wait for memory inside the next K loop)
    int32_t grabbed;
    f32x16_t acc[kMB][kNB];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
      for (int j = 0; j < kNB; ++j) acc[i][j] = f32x16_t{};
    if constexpr (G == 2) {
      // the VGPR accumulators' first reader is an MFMA in inline assembly, which the compiler's
      // hazard checks do not see: two wait states after their VALU writes
      __asm__ volatile("s_nop 1" : "+v"(acc[4][0]), "+v"(acc[4][1]), "+v"(acc[4][2]), "+v"(acc[4][3]));
    }

    const int nblk = (t.mlast + 32) / 32;   // 32-row blocks that hold rows
    const bool lay1 = G == 2 || (kLay1 && (nblk & 1) != 0 && nblk <= kMB1);
    int act = lay1 ? nblk : (nblk - wm + 1) / 2;   // row blocks of this wave that hold rows
    act = lay1 ? act : (act < 0 ? 0 : (act > kMB ? kMB : act));

    auto k_loop = [&](auto act_c, auto lay_c) __attribute__((always_inline)) {
      constexpr int ACT = decltype(act_c)::value;
      constexpr int LAY = decltype(lay_c)::value;      // 1: the 1 x 4 layout
      constexpr int MB = LAY ? kMBL : kMB, NB = LAY ? kNB1 : kNB;
      constexpr int kReads = ACT > 0 ? ACT + NB : 0;   // fragment reads per k-step
      constexpr int kSlots = kMB * kNB;                // MFMA slots of a k-step
      uint4 f0a[MB], f0b[NB], f1a[MB], f1b[NB];
      // fragment reads: lane l reads row l % 32 of a 32-row block, chunk 2 s + l / 32 of k-step
      // s (swizzled).  fb[s] is the lane's part of the LDS offset; the block's first row
      // (uniform) is the rest.  Computed here from the lane index, so that they live only
      // through the K loop: kept across the epilogue they would be spilled, and the reload's
      // wait before their first use would sit inside the loop.
      const uint32_t ln = opaque_lane();
      uint32_t fb[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) fb[s] = (ln & 31) * kRowB + ((2 * s + (ln >> 5)) ^ slot_key(ln & 31)) * 16;
      // (W8) weight fragments: 8 codes at chunk s, half l / 32, of the 64-byte row; read raw,
      // then converted with the row's block scale (sc_cur: this stage's, sc_nxt: the next one's)
      uint32_t fbw[4];
      // (G = 2) weight fragments from 64-byte half-stage rows: k-step s reads chunk
      // 2 (s & 1) + l / 32 of its half
      uint32_t fbh[2];
      if constexpr (G == 2) {
#pragma unroll
        for (int j = 0; j < 2; ++j) fbh[j] = (ln & 31) * 64 + (((2 * j + (ln >> 5)) ^ key4(ln & 31)) * 16);
      }
      uint2 wraw[NB];
      float sc_cur[NB], sc_nxt[NB];
      if constexpr (W8) {
#pragma unroll
        for (int s = 0; s < 4; ++s) fbw[s] = (ln & 31) * 64 + ((s ^ key4(ln & 31)) * 16) + (ln >> 5) * 8;
      }
      auto read_scales = [&](int ws, float(&sc)[NB]) __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < NB; ++n)
          sc[n] = *reinterpret_cast<const float*>(lds + kSBase + ws * 1024 + (b_row(0, n) + (ln & 31)) * 4);
      };
      // fragment read r of a k-step, in the order the MFMAs use them: a0, b0 .. b(NB-1), a1, ..
      auto read_frag = [&](int r, int aoff, int boff, int s, uint4(&fa)[MB], uint4(&fw)[NB])
          __attribute__((always_inline)) {
        if (r == 0) fa[0] = *reinterpret_cast<const uint4*>(lds + fb[s] + (aoff + a_row(LAY, 0) * kRowB));
        else if (r <= NB) {
          if constexpr (W8)
            wraw[r - 1] = *reinterpret_cast<const uint2*>(lds + fbw[s] + (boff + b_row(LAY, r - 1) * kWRowB));
          else if constexpr (G == 2)
            fw[r - 1] = *reinterpret_cast<const uint4*>(lds + fbh[s & 1] + (boff + b_row(LAY, r - 1) * kWRowB));
          else
            fw[r - 1] = *reinterpret_cast<const uint4*>(lds + fb[s] + (boff + b_row(LAY, r - 1) * kRowB));
        }
        else
          fa[r - NB] = *reinterpret_cast<const uint4*>(lds + fb[s] + (aoff + a_row(LAY, r - NB) * kRowB));
      };
      // the MFMAs of a k-step on (ca, cb), kSlots slots: MFMA i is row block i / NB and
      // column block i % NB.  After slot i come a fragment read of the next k-step (into na,
      // nb, when READ: read i / 2 after even slots in the 2 x 2 layout of 256 x 256 tiles,
      // read i otherwise) and then between(i), all held in place by scheduling fences: the
      // wave never stalls on a burst of LDS or memory instructions while the matrix pipe has
      // nothing queued.  In the 1 x 4 layout, row block m and column block n accumulate in
      // acc[m / 2][m % 2 + 2 n].
      auto mfma_step = [&]<bool READ>(uint4(&ca)[MB], uint4(&cb)[NB], uint4(&na)[MB], uint4(&nb)[NB],
                                      int aoff, int boff, int s, const float(&scn)[NB], auto&& between)
          __attribute__((always_inline)) {
        static_for<kSlots>([&](auto ic) __attribute__((always_inline)) {
          constexpr int i = decltype(ic)::value;
          constexpr int m = i / NB, n = i % NB;
          if constexpr (m < ACT) {
            f32x16_t& c = LAY ? acc[m / 2][(m & 1) + 2 * n] : acc[m][n];
            if constexpr (G == 2 && (LAY ? m / 2 : m) == 4) {
              // (the 320 x 256 tile's fifth row block: accumulators in VGPRs)
              __asm__ volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                               : "+v"(c)
                               : "v"(__builtin_bit_cast(u32x4_t, cb[n])), "v"(__builtin_bit_cast(u32x4_t, ca[m])));
            } else {
              c = mma_bf16(cb[n], ca[m], c);
              // (an ordered use of the result: instruction selection otherwise may sink the
              // MFMA, which reads no memory, past the slot's scheduling fence)
              __asm__ volatile("" : "+a"(c));
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (G == 2) {
            // (one buffer of activation fragments: a[m] of the next k-step is read after this
            // k-step's last MFMA on a[m], slot NB m + NB - 1; the weight fragments, which every
            // row block uses, are read into the other buffer at slots 0 .. NB - 1)
            if constexpr (READ && i < NB) read_frag(1 + i, aoff, boff, s, na, nb);
            if constexpr (READ && i % NB == NB - 1 && i / NB < ACT)
              read_frag(i / NB == 0 ? 0 : NB + i / NB, aoff, boff, s, na, nb);
          } else {
            constexpr int rd = (LAY || G == 1) ? i : ((i & 1) == 0 ? i / 2 : kReads);
            if constexpr (READ && rd < kReads) read_frag(rd, aoff, boff, s, na, nb);
          }
          // (W8) weight fragment n of the next k-step, read at slot 2 + 2 n (320 x 128 tiles: slot
          // 1 + n), converted over slots c + 2 n (codes 0-3) and c + 2 n + 1 (codes 4-7), c = 8
          // (5): 8 VALU instructions a slot, no more than the slot's MFMA takes, so the matrix
          // pipe never waits for a conversion
          constexpr int kCv = G == 0 ? 8 : 5;
          if constexpr (W8 && READ && ACT > 0 && i >= kCv && (i - kCv) / 2 < NB) {
            constexpr int n = (i - kCv) / 2;
            if constexpr (((i - kCv) & 1) == 0) {
              nb[n].x = e4m3x2_scaled_to_bf16x2<false>(wraw[n].x, scn[n]);
              nb[n].y = e4m3x2_scaled_to_bf16x2<true>(wraw[n].x, scn[n]);
            } else {
              nb[n].z = e4m3x2_scaled_to_bf16x2<false>(wraw[n].y, scn[n]);
              nb[n].w = e4m3x2_scaled_to_bf16x2<true>(wraw[n].y, scn[n]);
            }
          }
          between(ic);
          __builtin_amdgcn_sched_barrier(0);
        });
      };
      auto nothing = [](auto) __attribute__((always_inline)) {};
      // the next tile's index, taken during k-step 0 of the second-to-last stage: that stage's
      // wait for all loads (before its k-step 3) then also covers the take, so its result is
      // never pending past the stage (a pending result makes the compiler add waits for memory
      // inside later K loops), and three k-steps of MFMAs hide its latency
      auto take_next = [&]() __attribute__((always_inline)) {
        if (dynamic && tid == 0) grabbed = atomicAdd(tail_mode ? tail_ctr : counter + xcd, 1);
      };

#pragma unroll
      for (int r = 0; r < kReads; ++r) read_frag(r, 0, kWBase, 0, f0a, f0b);
      if constexpr (W8 && ACT > 0) {
        read_scales(0, sc_cur);
#pragma unroll
        for (int n = 0; n < NB; ++n) f0b[n] = e4m3x8_scaled_to_bf16x8(wraw[n], sc_cur[n]);
      }
      // stage ks: activation rows in buffer PAR = ks & 1, weight rows in ring slot ws = ks % kWS.
      // FULL: stage ks+2 exists; NEXT: stage ks+1 exists; WN: stage ks + kWS - 1 exists, and its
      // weight rows load during stage ks, into the slot stage ks-1 used.
      auto stage = [&]<bool FULL, bool NEXT, int PAR, bool WN>(int ks, int ws) __attribute__((always_inline)) {
        constexpr int buf = PAR, nbuf = PAR ^ 1;
        const int ws1 = ws == kWS - 1 ? 0 : ws + 1;
        const int wsl = ws == 0 ? kWS - 1 : ws - 1;
        const int aoff = buf * kPartA, boff = kWBase + ws * kWPart;
        mfma_step.template operator()<true>(f0a, f0b, f1a, f1b, aoff, boff, 1, sc_cur, [&](auto ic) __attribute__((always_inline)) {
          constexpr int i = decltype(ic)::value;
          constexpr int jw = G == 0 ? ((i & 3) == 1 ? (i >> 2) : kLdW) : ((i & 1) == 1 ? (i >> 1) : kLdW);
          if constexpr (WN && jw < kLdW) load_w.template operator()<jw>(t, ks + kWS - 1, wsl);
          if constexpr (!FULL && NEXT && i == 0) take_next();
        });
        mfma_step.template operator()<true>(f1a, f1b, f0a, f0b, aoff, boff, 2, sc_cur, [&](auto ic) __attribute__((always_inline)) {
          constexpr int i = decltype(ic)::value;
          if constexpr (G == 0 && WN && (i & 3) == 1 && 4 + (i >> 2) < kLdW)
            load_w.template operator()<4 + (i >> 2)>(t, ks + kWS - 1, wsl);
          if constexpr (W8 && WN && i == 1) load_s(t, ks + kWS - 1, wsl);
        });
        mfma_step.template operator()<true>(f0a, f0b, f1a, f1b, aoff, boff, 3, sc_cur, nothing);
        if constexpr (NEXT) {
          // stage ks+1 (activation rows from k-step 3 of stage ks-1, weight rows (and scales)
          // from k-steps 0-1 of an earlier stage) has landed once at most this stage's
          // weight-side loads remain
          wait_lgkmcnt_all();
          if constexpr (WN) wait_vmcnt<kStageLd>();
          else wait_vmcnt<0>();
          block_barrier();
          if constexpr (W8 && ACT > 0) read_scales(ws1, sc_nxt);
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_step.template operator()<NEXT>(f1a, f1b, f0a, f0b, nbuf * kPartA, kWBase + ws1 * kWPart, 0, sc_nxt,
                                            [&](auto ic) __attribute__((always_inline)) {
          constexpr int i = decltype(ic)::value;
          constexpr int ja = G == 0 ? ((i & 1) == 1 ? (i >> 1) : kLdA) : i;   // activation load of slot i
          if constexpr (FULL && ja < kLdA) load_a.template operator()<ja>(t, ks + 2, buf);
        });
        if constexpr (W8 && NEXT && ACT > 0) {
#pragma unroll
          for (int n = 0; n < NB; ++n) sc_cur[n] = sc_nxt[n];
        }
      };
      // (G = 2) stage ks: activation rows in buffer PAR, weight halves 2 ks and 2 ks + 1 in ring
      // slots wh = 2 ks mod 5 and the next.  After the barrier that ends k-step 2 every wave is
      // past both halves, and k-step 3 loads, in this order, half 2 ks + 5 into slot wh
      // (FULL: stage ks + 2 exists), the activation rows of stage ks + 2 into buffer PAR (FULL)
      // and half 2 ks + 6 into the next slot (W6: stage ks + 3 exists).  The barrier's wait
      // leaves only the most recent half in flight (FULL: it exists).
      auto stage2 = [&]<bool FULL, bool NEXT, int PAR, bool W6>(int ks, int wh) __attribute__((always_inline)) {
        constexpr int buf = PAR, nbuf = PAR ^ 1;
        const int h1 = wh == kWS - 1 ? 0 : wh + 1;   // slot of half 2 ks + 1
        const int h2 = h1 == kWS - 1 ? 0 : h1 + 1;   // slot of half 2 ks + 2 (the next stage's first)
        const int aoff = buf * kPartA;
        const int b0 = kWBase + wh * kWPart, b1 = kWBase + h1 * kWPart;
        mfma_step.template operator()<true>(f0a, f0b, f0a, f1b, aoff, b0, 1, sc_cur, [&](auto ic) __attribute__((always_inline)) {
          if constexpr (!FULL && NEXT && decltype(ic)::value == 0) take_next();
        });
        mfma_step.template operator()<true>(f0a, f1b, f0a, f0b, aoff, b1, 2, sc_cur, nothing);
        mfma_step.template operator()<true>(f0a, f0b, f0a, f1b, aoff, b1, 3, sc_cur, nothing);
        if constexpr (NEXT) {
          wait_lgkmcnt_all();
          if constexpr (FULL) wait_vmcnt<kLdW>();
          else wait_vmcnt<0>();
          block_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_step.template operator()<NEXT>(f0a, f1b, f0a, f0b, nbuf * kPartA, kWBase + h2 * kWPart, 0, sc_nxt,
                                            [&](auto ic) __attribute__((always_inline)) {
          constexpr int i = decltype(ic)::value;
          constexpr int jw5 = i < kLdW ? i : kLdW;
          constexpr int ja = i >= kLdW && i - kLdW < kLdA ? i - kLdW : kLdA;
          constexpr int jw6 = i >= kLdW + kLdA && i - kLdW - kLdA < kLdW ? i - kLdW - kLdA : kLdW;
          if constexpr (FULL && jw5 < kLdW) load_w.template operator()<jw5>(t, 2 * ks + 5, wh);
          if constexpr (FULL && ja < kLdA) load_a.template operator()<ja>(t, ks + 2, buf);
          if constexpr (W6 && jw6 < kLdW) load_w.template operator()<jw6>(t, 2 * ks + 6, h1);
        });
      };
      static_assert(G != 2 || kSlots >= 2 * kLdW + kLdA, "k-step 3 has a slot for each load");
      // stages in pairs (nk is even): with weight loads, then (five-slot ring) the pair whose
      // weight stages lie past the end, then the last two
      constexpr int kAhead = G == 2 ? 0 : kWS - 3;   // stages the weight ring runs ahead of the activations
      // (nk through volatile assembly: the loop guards are then compared per tile, in scalar
      // registers; hoisted out of the tile loop they were kept in a spilled register whose
      // reload waited on every load of the tile's first stages)
      int nkt;
      __asm__ volatile("s_mov_b32 %0, %1" : "=s"(nkt) : "s"(nk));
      if constexpr (G == 2) {
        int ks = 0, wh = 0;
        auto adv2 = [&]() __attribute__((always_inline)) { wh = wh >= kWS - 2 ? wh - (kWS - 2) : wh + 2; };
        for (; ks < nkt - 4; ks += 2) {
          stage2.template operator()<true, true, 0, true>(ks, wh);
          adv2();
          stage2.template operator()<true, true, 1, true>(ks + 1, wh);
          adv2();
        }
        if (ks < nkt - 2) {   // stages nk - 4 and nk - 3: the second has no half 2 ks + 6
          stage2.template operator()<true, true, 0, true>(ks, wh);
          adv2();
          stage2.template operator()<true, true, 1, false>(ks + 1, wh);
          adv2();
        }
        stage2.template operator()<false, true, 0, false>(nkt - 2, wh);
        adv2();
        stage2.template operator()<false, false, 1, false>(nkt - 1, wh);
        return;
      }
      int ks = 0, ws = 0;
      auto adv = [&]() __attribute__((always_inline)) { ws = ws == kWS - 1 ? 0 : ws + 1; };
      for (; ks < nkt - 2 - kAhead; ks += 2) {
        stage.template operator()<true, true, 0, true>(ks, ws);
        adv();
        stage.template operator()<true, true, 1, true>(ks + 1, ws);
        adv();
      }
      static_assert(kAhead == 0 || kAhead == 2, "one pair without weight loads");
      if constexpr (kAhead == 2) {
        if (ks < nkt - 2) {
          stage.template operator()<true, true, 0, false>(ks, ws);
          adv();
          stage.template operator()<true, true, 1, false>(ks + 1, ws);
          adv();
        }
      }
      stage.template operator()<false, true, 0, false>(nkt - 2, ws);
      adv();
      stage.template operator()<false, false, 1, false>(nkt - 1, ws);
    };
    if constexpr (G == 2) {
      // (the listed experts have 9 or 10 row blocks, every wave all of them)
      if (act >= 10) k_loop(std::integral_constant<int, 10>{}, std::integral_constant<int, 1>{});
      else k_loop(std::integral_constant<int, 9>{}, std::integral_constant<int, 1>{});
      // results of the inline-assembly MFMAs (8 passes) are read by VALU instructions next:
      // 11 wait states are required, 16 are given
      __asm__ volatile("s_nop 7\n\ts_nop 7" : "+v"(acc[4][0]), "+v"(acc[4][1]), "+v"(acc[4][2]), "+v"(acc[4][3]));
    } else if constexpr (G == 1) {
      // (the listed experts have 9 or 10 row blocks: 4 or 5 per wave; a wave with fewer
      // would compute rows past the tile, which the epilogue does not store)
      if (act >= 5) k_loop(std::integral_constant<int, 5>{}, std::integral_constant<int, 0>{});
      else k_loop(std::integral_constant<int, 4>{}, std::integral_constant<int, 0>{});
    } else if (kLay1 && lay1) {
      [&]<int... A>(std::integer_sequence<int, A...>) {
        ((act == 2 * A + 1 ? k_loop(std::integral_constant<int, 2 * A + 1>{}, std::integral_constant<int, 1>{})
                           : void()),
         ...);
      }(std::make_integer_sequence<int, (kMB1 + 1) / 2>{});
    } else {
      [&]<int... A>(std::integer_sequence<int, A...>) {
        ((act == A ? k_loop(std::integral_constant<int, A>{}, std::integral_constant<int, 0>{}) : void()), ...);
      }(std::make_integer_sequence<int, kMB + 1>{});
    }

    // ---- tile boundary: every wave is past its last LDS reads; the next tile is known
    block_barrier();
    const int vn = v + per_xcd;
    bool more;
    int Ln, tail_next = 0;
    if (dynamic) {
      if (tid == 0) *tile_word = resolve(grabbed, tail_mode != 0);
      wait_lgkmcnt_all();
      block_barrier();
      const int32_t word = __builtin_amdgcn_readfirstlane(*tile_word);
      if constexpr (G == 2) block_barrier();   // (its prologue writes the slot that holds the word)
      more = word >= 0;
      Ln = word & kTileMask;
      tail_next = word >> 30;
    } else {
      more = vn < v_end;
      Ln = more ? tile_of(vn) : 0;
    }
    // the finished tile's rows and columns (cur is rewritten by the next tile's set-up)
    const int em0 = t.m0, emend = t.mend, ec0 = t.c0, ekp = t.kp;

    // ---- epilogue: block acc[mb][nb] holds, in lane l, token row rblk * 32 + l % 32 of the
    // tile and, in registers 4q .. 4q+3, output columns cblk + 8q + 4 (l / 32) + 0..3 (2 x 2:
    // rblk = 2 mb + wm, cblk = 32 nb of the wave's 32 NB columns; 1 x 4: rblk = 2 mb + nb % 2,
    // cblk = 32 (nb / 2) of the wave's 64).  bf16 outputs: the runs of groups 2u and 2u + 1
    // are exchanged between the lane halves, one 16-byte store per lane and pair (n_cols % 8
    // == 0, so a lane's 8 columns are all in or all out); fp32 router sums: one 16-byte store
    // per run (n_cols % 4 == 0).  Gate/up pairs the gate block nb < NB / 2 with the up block
    // nb + NB / 2 of the same rows and columns.
    // (the lane's row and column half are derived here from the lane id: kept from before the
    // K loop they would be spilled, and their reloads' waits would also wait for the next
    // tile's first loads, issued ahead of them)
    const int eln = static_cast<int>(opaque_lane());
    const int erow = eln & 31, ehk = eln >> 5;
    auto row_in = [&](int mb, int h) __attribute__((always_inline)) {   // row within the tile
      return (kLay1 && lay1 ? 2 * mb + h : 2 * mb + wm) * 32 + erow;
    };
    // down with gates: a routed row carries the gate of its slot (the shared rows gate 1),
    // loaded and waited for before anything else is issued
    float gsv[kMB];   // (only the down GEMM has gates, and it runs the 2 x 2 layout)
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) gsv[mb] = 1.0f;
    if (MODE == MODE_DOWN && p.row_gate != nullptr) {
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        const int r = em0 + row_in(mb, 0);
        if (r < p.rows && r < emend) {
          int sl = p.row_slot[r];
          sl = sl < 0 ? 0 : (sl < p.rows ? sl : p.rows - 1);
          gsv[mb] = p.row_gate[sl];
        }
      }
      wait_vmcnt<0>();
    }
    // bf16 outputs go out as buffer stores over the tile's rows, a fixed number per wave (a
    // lane outside the tile's rows or the output's columns gets an offset past the window and
    // writes nothing), so the next tile's set-up and first loads are issued before them and
    // its wait for stage 0 leaves exactly these stores in flight
    constexpr bool kEarly = MODE != MODE_ROUTER;
    constexpr int kStores = MODE == MODE_GATE_UP ? kMB * (kNB / 2) * 2 : kMB * kNB * 2;
    if (kEarly && more) {
      setup(Ln, cur);
      prologue_loads(cur);
    }
    const uint32_t orow = static_cast<uint32_t>(n_cols) * 2;   // bytes of an output row
    constexpr uint32_t kNoWrite = 0x80000000u;                   // past every tile's window
    if constexpr (MODE == MODE_ROUTER) {
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) {
            const int r = em0 + row_in(mb, nb & 1);
            const int col = ec0 + (lay1 ? wave * 64 + (nb >> 1) * 32 : wn * kNB * 32 + nb * 32) + 8 * q + 4 * ehk;
            if (r >= emend || col >= n_cols) continue;
            const f32x16_t& a = acc[mb][nb];
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) +
                                       (static_cast<size_t>(ekp) * p.rows + r) * p.n_out + col) =
                make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
          }
    } else {
      const uint32_t nrow = static_cast<uint32_t>(emend - em0);
      const buf_rsrc_t out_w = make_window(reinterpret_cast<uint8_t*>(p.out) + static_cast<size_t>(em0) * orow, nrow * orow);
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        // bf16 rows: register groups 2 u and 2 u + 1 are paired across the lane halves, so a
        // lane stores 8 adjacent columns (16 bytes) at column 16 u + 8 hk of its block
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          if constexpr (MODE == MODE_GATE_UP) {
#pragma unroll
            for (int nb = 0; nb < kNB / 2; ++nb) {
              const int ri = row_in(mb, nb);
              const int col = ec0 + (lay1 ? wave * 32 : wn * (kNB / 2) * 32 + nb * 32) + 16 * u + 8 * ehk;
              const bool in = ri < static_cast<int>(nrow) && col < n_cols;
              const f32x16_t& ga = acc[mb][nb];
              const f32x16_t& ua = acc[mb][nb + kNB / 2];
              uint2 hq[2];
#pragma unroll
              for (int g = 0; g < 2; ++g) {
                const int b0 = 8 * u + 4 * g;
                hq[g] = make_uint2(pack_bf16x2(silu_f32(ga[b0]) * ua[b0], silu_f32(ga[b0 + 1]) * ua[b0 + 1]),
                                   pack_bf16x2(silu_f32(ga[b0 + 2]) * ua[b0 + 2], silu_f32(ga[b0 + 3]) * ua[b0 + 3]));
              }
              store16(out_w, in ? static_cast<uint32_t>(ri) * orow + static_cast<uint32_t>(col) * 2 : kNoWrite,
                      lane_pair(hq[0], hq[1]));   // (every lane: the exchange reads both halves)
              if (p.au != nullptr) {   // the pre-activations, for the backward pass
                const uint32_t arow = static_cast<uint32_t>(p.I) * 4;
                const buf_rsrc_t au_w =
                    make_window(reinterpret_cast<uint8_t*>(p.au) + static_cast<size_t>(em0) * arow, nrow * arow);
                const uint32_t ao = in ? static_cast<uint32_t>(ri) * arow + static_cast<uint32_t>(col) * 2 : kNoWrite;
                store16(au_w, ao,
                        lane_pair(make_uint2(pack_bf16x2(ga[8 * u], ga[8 * u + 1]), pack_bf16x2(ga[8 * u + 2], ga[8 * u + 3])),
                                  make_uint2(pack_bf16x2(ga[8 * u + 4], ga[8 * u + 5]), pack_bf16x2(ga[8 * u + 6], ga[8 * u + 7]))));
                store16(au_w, in ? ao + static_cast<uint32_t>(p.I) * 2 : kNoWrite,
                        lane_pair(make_uint2(pack_bf16x2(ua[8 * u], ua[8 * u + 1]), pack_bf16x2(ua[8 * u + 2], ua[8 * u + 3])),
                                  make_uint2(pack_bf16x2(ua[8 * u + 4], ua[8 * u + 5]), pack_bf16x2(ua[8 * u + 6], ua[8 * u + 7]))));
              }
            }
          } else {
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) {
              const int ri = row_in(mb, nb & 1);
              const int col = ec0 + (lay1 ? wave * 64 + (nb >> 1) * 32 : wn * kNB * 32 + nb * 32) + 16 * u + 8 * ehk;
              const bool in = ri < static_cast<int>(nrow) && col < n_cols;
              const float gs = gsv[mb];
              const f32x16_t& a = acc[mb][nb];
              const uint4 ov = lane_pair(
                  make_uint2(pack_bf16x2(a[8 * u] * gs, a[8 * u + 1] * gs), pack_bf16x2(a[8 * u + 2] * gs, a[8 * u + 3] * gs)),
                  make_uint2(pack_bf16x2(a[8 * u + 4] * gs, a[8 * u + 5] * gs), pack_bf16x2(a[8 * u + 6] * gs, a[8 * u + 7] * gs)));
              store16(out_w, in ? static_cast<uint32_t>(ri) * orow + static_cast<uint32_t>(col) * 2 : kNoWrite, ov);
            }
          }
        }
      }
    }
    if (!more) break;
    if constexpr (kEarly) {
      // stage 0 of the next tile has landed once at most its later stages' loads and this
      // tile's stores (issued after them) remain: the stores drain under the next K loop
      prologue_wait.template operator()<kStores>();
    } else {
      setup(Ln, cur);
      prologue_loads(cur);
      prologue_wait.template operator()<0>();
    }
    v = vn;
    L = Ln;
    tail_mode = tail_next;
  }
}

// bf16 (or W8) grouped GEMM: the experts the schedule lists for 320-row tiles first (bf16 only:
// one 320 x 256 gate/up tile or 320 x 128 down tile per expert and n-block), then the 256 x 256
// tiles.  A workgroup that runs out of the first shape's tiles moves on to the second's without
// waiting for the others.
template <int MODE, bool W8>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_wide_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes<W8>];
  if constexpr (MODE == MODE_DOWN) {
    if (p.tall_list != nullptr) run_tiles<MODE, W8, 1>(p, lds);
  }
  if constexpr (MODE == MODE_GATE_UP && !W8) {
    if (p.tall_list != nullptr) run_tiles<MODE, W8, 2>(p, lds);
  }
  run_tiles<MODE, W8, 0>(p, lds);
}

}  // namespace

hipError_t launch_grouped_gemm_wide(int mode, const GemmArgs& p, hipStream_t s, bool w8) {
  const dim3 grid(256), block(kThreads);   // persistent: one workgroup per CU, a multiple of the 8 XCDs
  if (w8 && mode == MODE_ROUTER) return hipErrorNotSupported;
  if (((w8 && mode != MODE_DOWN) || mode == MODE_ROUTER) && p.tall_list != nullptr) return hipErrorNotSupported;
  if (mode == MODE_GATE_UP && w8)
    hipLaunchKernelGGL((grouped_gemm_wide_kernel<MODE_GATE_UP, true>), grid, block, 0, s, p);
  else if (mode == MODE_GATE_UP)
    hipLaunchKernelGGL((grouped_gemm_wide_kernel<MODE_GATE_UP, false>), grid, block, 0, s, p);
  else if (mode == MODE_DOWN && w8)
    hipLaunchKernelGGL((grouped_gemm_wide_kernel<MODE_DOWN, true>), grid, block, 0, s, p);
  else if (mode == MODE_DOWN)
    hipLaunchKernelGGL((grouped_gemm_wide_kernel<MODE_DOWN, false>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((grouped_gemm_wide_kernel<MODE_ROUTER, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
