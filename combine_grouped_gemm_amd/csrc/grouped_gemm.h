// Arguments shared by the grouped expert GEMM kernels and their launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum { CT_F32 = 0, CT_BF16 = 1, CT_FP8 = 2 };
enum { MODE_GATE_UP = 0, MODE_DOWN = 1, MODE_ROUTER = 2 };

constexpr int kNumXcd = 8;

struct GemmArgs {
  const uint8_t* a;            // [rows, K] compute-type elements (e4m3 codes for CT_FP8)
  const float* a_scale;        // [rows, K / 128]            (CT_FP8)
  const uint8_t* b;            // [E, b_rows, K]: compute type, or e4m3 codes when B8
  const float* b_scale;        // [E, b_rows, K / 128]       (CT_FP8, B8)
  void* out;                   // gate/up: h [rows, I]; down: out [rows, H]
  const int32_t* offsets;      // [E + 1]
  const int32_t* tile_prefix;  // [E + 1]  m-tiles before each expert
  const int32_t* tile_expert;  // [tile_cap]  m-tile -> expert
  const int32_t* a_rows;       // [rows] or null: row r of the operand is row a_rows[r] / a_div of a
  int a_div, a_nrows;          // (gathered operand: a has a_nrows rows)
  int E, K, rows, I, n_out, tile_cap;
  long long b_rows;
  int out_f32;
  int32_t* tile_counter;       // [kNumXcd + 1] next tile of each XCD's range, then the next tile
                               // of the shared tail (zeroed by the schedule prologue), or null:
                               // tiles dealt round-robin
  const uint8_t* shared_b;     // shared expert's weights [b_rows, K] (segment E), or null
  int shared_rows;             // rows of the shared segment [rows, rows + shared_rows); 0: none
  const int32_t* row_slot;     // down: routed output row r is scaled by row_gate[row_slot[r]]
  const float* row_gate;       //   (slots clamped into [0, rows)), or both null
  int k_split;                 // router: K is cut into k_split equal parts; part s of every
                               // output goes to out + s * rows * n_out (fp32)
  void* au;                    // gate/up (256 x 256 kernel): also the pre-activations [rows, 2I]
                               // bf16 (gate in columns 0..I-1, up in I..2I-1), or null
  const int32_t* tall_list = nullptr;   // (bf16 down, 256 x 256 kernel) [E + 1]: count T, then
                               // the T experts with kWideTileRows < n_e <= kWideTallRows, which the
                               // prefix gives no m-tiles and which run as one 320-row tile; or null
  int32_t* tall_counter = nullptr;      // [kNumXcd] the counters of those tiles (zeroed by the prologue)
  const float* shared_b_scale = nullptr;  // (B8) the shared expert's block scales [b_rows, K / 128]
};

// Segment [lo, hi) of expert e, clamped into [0, rows] so that malformed offsets cannot
// index out of range.
__device__ __forceinline__ void expert_segment(const GemmArgs& p, int e, int& lo, int& hi) {
  lo = p.offsets[e];
  hi = p.offsets[e + 1];
  lo = lo < 0 ? 0 : (lo > p.rows ? p.rows : lo);
  hi = hi < lo ? lo : (hi > p.rows ? p.rows : hi);
}

// Weight-streaming kernel for few rows per expert (grouped_gemm_stream.hip); the tile
// schedule in `p` must have been built with 16-row m-tiles.
constexpr int kStreamTileRows = 16;
hipError_t launch_grouped_gemm_stream(int mode, const GemmArgs& p, hipStream_t s);

// bf16 kernel on 256 x 256 tiles (grouped_gemm_wide.hip); the tile schedule in `p` must
// have been built with 256-row m-tiles, K must be a multiple of 128, and every operand
// offset (b_rows * K * 2 per expert; a_nrows * K * 2 when gathered) must fit in 32 bits.
constexpr int kWideTileRows = 256;
constexpr int kWideTallRows = 320;   // an expert of 257..320 rows: one tile of 320 x 128
// MODE_ROUTER (one segment [0, rows), no tile schedule, static tile order): tile
// (part s, n-block, m-tile) multiplies columns [s K/k_split, (s+1) K/k_split) of a and b
// (K / k_split a multiple of 128) and stores its fp32 sums, 16 bytes per run (n_out % 4 == 0).
hipError_t launch_grouped_gemm_wide(int mode, const GemmArgs& p, hipStream_t s, bool w8 = false);

}  // namespace moe
