// Group the T*k (token, rank) slots by expert: counts, exclusive offsets, and a stable
// permutation (review of the from-scratch gpt-oss-20B at pomoai.com, section 3.4: only the
// picked experts compute). One workgroup of 16 waves performs a stable counting sort:
//   1. each wave histograms a contiguous range of slots into its own LDS row;
//   2. per-expert totals -> exclusive scan -> expert_offsets, and each wave's base offset
//      per expert = offset[e] + counts of the same expert in the waves before it;
//   3. each wave walks its range again in slot order, 64 slots at a time, ranking equal
//      experts among the lanes with ballots, and scatters.
// Deterministic: positions depend only on slot order, never on atomics' timing.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kPermWaves = 16;
constexpr int kPermThreads = kPermWaves * kWave;
constexpr int kMaxExperts = 256;

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t *__restrict__ topk_idx,
                                                               int64_t S, int E,
                                                               int32_t *__restrict__ offsets,
                                                               int32_t *__restrict__ sorted_slot,
                                                               int32_t *__restrict__ slot_row) {
  __shared__ int hist[kPermWaves][kMaxExperts];
  __shared__ int scan[kMaxExperts + 1];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  for (int i = tid; i < kPermWaves * kMaxExperts; i += kPermThreads) (&hist[0][0])[i] = 0;
  __syncthreads();

  const int64_t per_wave = (((S + kPermWaves - 1) / kPermWaves) + kWave - 1) / kWave * kWave;
  const int64_t beg = (int64_t)wave * per_wave;
  const int64_t end = (beg + per_wave < S) ? beg + per_wave : S;
  // ids outside [0, E) are skipped (their slots get no position), never indexed
  for (int64_t s = beg + lane; s < end; s += kWave) {
    const int e = topk_idx[s];
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[wave][e], 1);
  }
  __syncthreads();

  // totals and exclusive scan over experts (E <= 256 fits in 4 waves' worth of threads)
  if (tid < kMaxExperts) {
    int tot = 0;
    if (tid < E)
      for (int w = 0; w < kPermWaves; ++w) tot += hist[w][tid];
    scan[tid + 1] = tot;
  }
  __syncthreads();
  if (wave == 0) {
    int carry = 0;
    for (int base = 0; base < kMaxExperts; base += kWave) {
      const int v = scan[base + lane + 1];
      const int inc = wave_inclusive_scan(v);
      scan[base + lane + 1] = inc + carry;
      carry += wave_read(inc, kWave - 1);
    }
    if (lane == 0) scan[0] = 0;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += kPermThreads) offsets[e] = scan[e];
  if (tid < E) {
    int run = scan[tid];
    for (int w = 0; w < kPermWaves; ++w) {
      const int c = hist[w][tid];
      hist[w][tid] = run;
      run += c;
    }
  }
  __syncthreads();

  // stable scatter: lanes of a batch are in slot order; equal experts are ranked by lane
  for (int64_t s0 = beg; s0 < end; s0 += kWave) {
    const int64_t s = s0 + lane;
    const int e = (s < end) ? topk_idx[s] : -1;
    const bool active = (unsigned)e < (unsigned)E;
    uint64_t same = __ballot(active);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const uint64_t ones = __ballot(active && ((e >> bit) & 1));
      same &= ((e >> bit) & 1) ? ones : ~ones;
    }
    if (active) {
      const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
      const int rank = __popcll(same & below);
      const int pos = hist[wave][e] + rank;
      sorted_slot[pos] = (int32_t)s;
      slot_row[s] = pos;
      // the lowest lane of each group advances the group's base after everyone has read it
      __builtin_amdgcn_wave_barrier();
      if (rank == 0) hist[wave][e] += __popcll(same);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

hipError_t launch_permute(const int32_t *topk_idx, int64_t S, int E, int32_t *offsets,
                          int32_t *sorted_slot, int32_t *slot_row, hipStream_t stream) {
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, stream, topk_idx, S, E, offsets,
                     sorted_slot, slot_row);
  return hipGetLastError();
}

}  // namespace moe
