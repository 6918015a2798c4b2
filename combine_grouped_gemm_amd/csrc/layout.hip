// Dispatch layout: expert histogram, exclusive scan and the stable scatter that builds the
// send-position and return maps ("EP / DeepEP explanation" page, sections 2, 3 and 6).
//
// Deterministic counting sort of the N*k slots by expert id, in three launches:
//   1. count:   per chunk of slots, an LDS histogram -> counts[chunk][e]
//   2. scan:    per expert, exclusive prefix over chunks (in place) and n_e; then the
//               exclusive prefix over experts -> offsets
//   3. scatter: per chunk, each wave ranks its slots within equal-expert groups with
//               ballots (lanes in slot order), so a slot's row is
//               offsets[e] + (earlier chunks) + (earlier waves of the chunk) + (earlier
//               steps of the wave) + (earlier lanes of the step).
// LDS atomics only build counts, whose value does not depend on their order, so every
// output is a pure function of topk_idx.
#include <mutex>

#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

constexpr int kLayoutThreads = 256;

int layout_chunk_slots(long long nk) {
  // 1024 slots per chunk, grown so there are at most 4096 chunks
  long long ch = 1024;
  while ((nk + ch - 1) / ch > 4096) ch *= 2;
  return static_cast<int>(ch);
}

int layout_num_chunks(long long nk) {
  const long long ch = layout_chunk_slots(nk);
  return static_cast<int>((nk + ch - 1) / ch);
}

__global__ __launch_bounds__(kLayoutThreads) void layout_count_kernel(
    const int32_t* __restrict__ idx, int nk, int E, int chunk, int32_t* __restrict__ counts) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += kLayoutThreads) hist[e] = 0;
  __syncthreads();
  const long long base = static_cast<long long>(blockIdx.x) * chunk;
  for (int i = threadIdx.x; i < chunk; i += kLayoutThreads) {
    const long long s = base + i;
    if (s >= nk) break;
    const int e = idx[s];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  int32_t* out = counts + static_cast<size_t>(blockIdx.x) * E;
  for (int e = threadIdx.x; e < E; e += kLayoutThreads) out[e] = hist[e];
}

__global__ __launch_bounds__(1024) void layout_scan_kernel(int32_t* __restrict__ counts, int nchunks,
                                                           int E, int32_t* __restrict__ n_e,
                                                           int32_t* __restrict__ offsets) {
  __shared__ int32_t tot[1024];
  const int e = threadIdx.x;
  int32_t run = 0;
  if (e < E) {
    // 16 chunks' counts loaded before any is replaced by its exclusive prefix, so the loads
    // are in flight together instead of one latency per chunk
    constexpr int kBatch = 16;
    for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
      int32_t v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        v[j] = c0 + j < nchunks ? counts[static_cast<size_t>(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (c0 + j < nchunks) counts[static_cast<size_t>(c0 + j) * E + e] = run;
        run += v[j];
      }
    }
    n_e[e] = run;
  }
  tot[e] = e < E ? run : 0;
  __syncthreads();
  // inclusive Hillis-Steele scan over 1024 entries
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = e >= off ? tot[e - off] : 0;
    __syncthreads();
    tot[e] += v;
    __syncthreads();
  }
  if (e < E) offsets[e] = tot[e] - run;
  if (e == E - 1) offsets[E] = tot[e];
}

__global__ __launch_bounds__(kLayoutThreads) void layout_scatter_kernel(
    const int32_t* __restrict__ idx, int nk, int E, int chunk, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ send_pos,
    int32_t* __restrict__ src_slot) {
  extern __shared__ int32_t wbase[];  // [4][E]
  constexpr int kWaves = kLayoutThreads / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  for (int i = threadIdx.x; i < kWaves * E; i += kLayoutThreads) wbase[i] = 0;
  __syncthreads();

  const long long cbase = static_cast<long long>(blockIdx.x) * chunk;
  const int quarter = chunk / kWaves;
  const long long qbeg = cbase + static_cast<long long>(w) * quarter;
  const long long qend_raw = qbeg + quarter;
  const long long qend = qend_raw < nk ? qend_raw : nk;

  // 1. per-wave histogram of its quarter
  for (long long s = qbeg + lane; s < qend; s += kWave) {
    const int e = idx[s];
    if (e >= 0 && e < E) atomicAdd(&wbase[w * E + e], 1);
  }
  __syncthreads();
  // 2. turn the per-wave counts into per-wave starting rows
  const int32_t* cnt = counts + static_cast<size_t>(blockIdx.x) * E;
  for (int e = threadIdx.x; e < E; e += kLayoutThreads) {
    int32_t b = offsets[e] + cnt[e];
    for (int q = 0; q < kWaves; ++q) {
      const int32_t v = wbase[q * E + e];
      wbase[q * E + e] = b;
      b += v;
    }
  }
  __syncthreads();
  // 3. walk the quarter in 64-slot steps, in slot order
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  for (long long s0 = qbeg; s0 < qend; s0 += kWave) {
    const long long s = s0 + lane;
    const bool in = s < qend;
    const int e = in ? idx[s] : -1;
    const bool ok = in && e >= 0 && e < E;
    uint64_t same = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = ok && ((e >> b) & 1);
      const uint64_t bal = __ballot(bit);
      same &= ((e >> b) & 1) ? bal : ~bal;
    }
    int32_t row = -1;
    int32_t base = 0;
    if (ok) {
      base = wbase[w * E + e];
      row = base + __popcll(same & lt_mask);
    }
    // every lane has read its base before the last lane of each group advances it
    __builtin_amdgcn_wave_barrier();
    if (ok && (63 - __clzll(same)) == lane) wbase[w * E + e] = base + __popcll(same);
    __builtin_amdgcn_wave_barrier();
    if (in) send_pos[s] = row;
    if (ok) src_slot[row] = static_cast<int32_t>(s);
  }
}

hipError_t launch_dispatch_layout(const int32_t* topk_idx, int nk, int E, int32_t* n_e,
                                  int32_t* offsets, int32_t* send_pos, int32_t* src_slot,
                                  int32_t* counts, hipStream_t s) {
  const int chunk = layout_chunk_slots(nk);
  const int nchunks = layout_num_chunks(nk);
  hipLaunchKernelGGL(layout_count_kernel, dim3(nchunks), dim3(kLayoutThreads), E * sizeof(int32_t),
                     s, topk_idx, nk, E, chunk, counts);
  hipLaunchKernelGGL(layout_scan_kernel, dim3(1), dim3(1024), 0, s, counts, nchunks, E, n_e,
                     offsets);
  hipLaunchKernelGGL(layout_scatter_kernel, dim3(nchunks), dim3(kLayoutThreads),
                     4 * E * sizeof(int32_t), s, topk_idx, nk, E, chunk, counts, offsets, send_pos,
                     src_slot);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// Scratch of the allocation-free entry point: the per-chunk counts live in a fixed device
// array instead of a caller's workspace.  Each device holds its own copy at its own address
// for the life of the process.  The count launch writes every entry that the scan and the
// scatter read, so no call needs the array cleared; calls that overlap on one device share
// the array and race.
// ------------------------------------------------------------------------------------

constexpr size_t kScratchInts = MOE_LAYOUT_SCRATCH_BYTES / sizeof(int32_t);
static __device__ __align__(256) int32_t scratch[kScratchInts];

constexpr int kMaxDevices = 64;

hipError_t layout_scratch(int32_t** out) {
  // the device address of the current device's copy, looked up once per device (host code
  // never passes the array's own name: on the host it is a stand-in, not a device address)
  static std::mutex mu;
  static int32_t* ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = ptr[dev];
  return hipSuccess;
}

}  // namespace moe
