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
#include "topk.h"

namespace moe {

constexpr int kPermWaves = 16;
constexpr int kPermThreads = kPermWaves * kWave;
constexpr int kMaxExperts = 256;
constexpr int64_t kPermSingleMax = 8192;  // up to this many slots one workgroup sorts them all

// The single-workgroup sort by NW waves (NW * 64 >= 256 threads); idx(s) yields slot s's
// expert id.
template <int NW, typename Idx>
__device__ __forceinline__ void permute_block(Idx idx, int64_t S, int E, int32_t *__restrict__ offsets,
                                              int32_t *__restrict__ sorted_slot, int32_t *__restrict__ slot_row,
                                              int (&hist)[NW][kMaxExperts], int (&scan)[kMaxExperts + 1]) {
  static_assert(NW * kWave >= kMaxExperts, "one thread per expert for the totals");
  constexpr int kThreads = NW * kWave;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  for (int i = tid; i < NW * kMaxExperts; i += kThreads) (&hist[0][0])[i] = 0;
  __syncthreads();

  const int64_t per_wave = (((S + NW - 1) / NW) + kWave - 1) / kWave * kWave;
  const int64_t beg = (int64_t)wave * per_wave;
  const int64_t end = (beg + per_wave < S) ? beg + per_wave : S;
  // ids outside [0, E) are skipped (their slots get no position), never indexed
  for (int64_t s = beg + lane; s < end; s += kWave) {
    const int e = idx(s);
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[wave][e], 1);
  }
  __syncthreads();

  // totals and exclusive scan over experts (E <= 256 fits in 4 waves' worth of threads)
  if (tid < kMaxExperts) {
    int tot = 0;
    if (tid < E)
      for (int w = 0; w < NW; ++w) tot += hist[w][tid];
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
  for (int e = tid; e <= E; e += kThreads) offsets[e] = scan[e];
  if (tid < E) {
    int run = scan[tid];
    for (int w = 0; w < NW; ++w) {
      const int c = hist[w][tid];
      hist[w][tid] = run;
      run += c;
    }
  }
  __syncthreads();

  // stable scatter: lanes of a batch are in slot order; equal experts are ranked by lane
  for (int64_t s0 = beg; s0 < end; s0 += kWave) {
    const int64_t s = s0 + lane;
    const int e = (s < end) ? idx(s) : -1;
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

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t *__restrict__ topk_idx,
                                                               int64_t S, int E,
                                                               int32_t *__restrict__ offsets,
                                                               int32_t *__restrict__ sorted_slot,
                                                               int32_t *__restrict__ slot_row) {
  __shared__ int hist[kPermWaves][kMaxExperts];
  __shared__ int scan[kMaxExperts + 1];
  permute_block<kPermWaves>([&](int64_t s) { return topk_idx[s]; }, S, E, offsets, sorted_slot, slot_row, hist, scan);
}

// Many slots: the same counting sort over several workgroups. Chunk c of kPermChunk
// consecutive slots belongs to workgroup c; wave w of it to the w-th sixteenth of the chunk.
// Pass 1 writes every (chunk, wave) histogram; pass 2 has every workgroup add up, for each
// expert, the totals (-> offsets) and the counts of all (chunk, wave) ranges before each of
// its waves (-> that wave's base), then scatter its chunk exactly as above. Slot order is
// chunk order, then wave order, then batch order, so the permutation stays stable.
constexpr int kPermChunk = kPermWaves * 256;

__global__ __launch_bounds__(kPermThreads) void permute_hist_kernel(const int32_t *__restrict__ topk_idx,
                                                                    int64_t S, int E, int32_t *__restrict__ whist) {
  __shared__ int hist[kPermWaves][kMaxExperts];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  for (int i = tid; i < kPermWaves * kMaxExperts; i += kPermThreads) (&hist[0][0])[i] = 0;
  __syncthreads();
  const int64_t beg = (int64_t)blockIdx.x * kPermChunk + wave * 256;
  const int64_t end = (beg + 256 < S) ? beg + 256 : S;
  for (int64_t s = beg + lane; s < end; s += kWave) {
    const int e = topk_idx[s];
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[wave][e], 1);
  }
  __syncthreads();
  for (int i = tid; i < kPermWaves * E; i += kPermThreads)
    whist[((int64_t)blockIdx.x * kPermWaves + i / E) * E + i % E] = hist[i / E][i % E];
}

__global__ __launch_bounds__(kPermThreads) void permute_scatter_kernel(const int32_t *__restrict__ topk_idx,
                                                                       int64_t S, int E, int nchunks,
                                                                       const int32_t *__restrict__ whist,
                                                                       int32_t *__restrict__ offsets,
                                                                       int32_t *__restrict__ sorted_slot,
                                                                       int32_t *__restrict__ slot_row) {
  __shared__ int base[kPermWaves][kMaxExperts];
  __shared__ int scan[kMaxExperts + 1];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int nranges = nchunks * kPermWaves;
  const int mine = blockIdx.x * kPermWaves;  // this workgroup's first (chunk, wave) range
  // thread e: the expert's total and its count in the ranges before each of this chunk's waves
  if (tid < kMaxExperts) {
    int tot = 0;
    if (tid < E) {
      // ranges come in groups of kPermWaves (one chunk); load a group, then add in order
      for (int g0 = 0; g0 < nranges; g0 += kPermWaves) {
        int c[kPermWaves];
#pragma unroll
        for (int w = 0; w < kPermWaves; ++w) c[w] = whist[(int64_t)(g0 + w) * E + tid];
#pragma unroll
        for (int w = 0; w < kPermWaves; ++w) {
          if (g0 == mine) base[w][tid] = tot;
          tot += c[w];
        }
      }
    }
    scan[tid + 1] = tot;
  }
  __syncthreads();
  if (wave == 0) {
    int carry = 0;
    for (int b = 0; b < kMaxExperts; b += kWave) {
      const int v = scan[b + lane + 1];
      const int inc = wave_inclusive_scan(v);
      scan[b + lane + 1] = inc + carry;
      carry += wave_read(inc, kWave - 1);
    }
    if (lane == 0) scan[0] = 0;
  }
  __syncthreads();
  if (blockIdx.x == 0)
    for (int e = tid; e <= E; e += kPermThreads) offsets[e] = scan[e];
  if (tid < E)
    for (int w = 0; w < kPermWaves; ++w) base[w][tid] += scan[tid];
  __syncthreads();
  const int64_t beg = (int64_t)blockIdx.x * kPermChunk + wave * 256;
  const int64_t end = (beg + 256 < S) ? beg + 256 : S;
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
      const int pos = base[wave][e] + rank;
      sorted_slot[pos] = (int32_t)s;
      slot_row[s] = pos;
      __builtin_amdgcn_wave_barrier();
      if (rank == 0) base[wave][e] += __popcll(same);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Decode-sized batches: the router's top-k step (one wave per token, as router_topk_kernel
// on token-major partials) and, in the workgroup that finishes last, the permutation (the
// counting sort above on 4 waves), in one launch. Every workgroup publishes its picks
// (device-scope fence) before counting itself in; the last one to count in reads all picks
// back at device scope. No workgroup waits for another. The counter is zeroed by
// router_partial_kernel of the same call.
constexpr int64_t kTopkPermMaxSlots = 2048;
constexpr int64_t kTopkSmallMaxT = kPermWaves;  // one wave per token in one workgroup

__global__ __launch_bounds__(256) void router_topk_permute_kernel(
    const float *__restrict__ partial, int nsplit, const float *__restrict__ bias, int64_t T, int E, int k,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, int *__restrict__ counter,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_slot, int32_t *__restrict__ slot_row) {
  __shared__ int hist[4][kMaxExperts];
  __shared__ int scan[kMaxExperts + 1];
  __shared__ int last;
  const int lane = threadIdx.x % kWave;
  const int64_t t = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (t < T) {
    float v[4];
    router_logits_wave<false>(partial, nsplit, bias, t, T, E, lane, v);
    topk_softmax_wave(v, E, k, lane, topk_idx + t * k, topk_w + t * k);
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) last = atomicAdd(counter, 1) == (int)gridDim.x - 1;
  __syncthreads();
  if (!last) return;
  __threadfence();
  permute_block<4>(
      [&](int64_t s) { return __hip_atomic_load(topk_idx + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); },
      T * k, E, offsets, sorted_slot, slot_row, hist, scan);
}

// Batches of at most kTopkSmallMaxT tokens: one workgroup of 16 waves; wave t picks token t's
// experts (the same top-k and softmax as above) and leaves its picks in LDS, then the counting
// sort runs on them there. No hand-off between workgroups, so no arrival counter and no
// device-scope fences: at these sizes those round trips, not the work, set the kernel's time.
__global__ __launch_bounds__(kPermThreads) void router_topk_permute_small_kernel(
    const float *__restrict__ partial, int nsplit, const float *__restrict__ bias, int64_t T, int E, int k,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, int32_t *__restrict__ offsets,
    int32_t *__restrict__ sorted_slot, int32_t *__restrict__ slot_row) {
  __shared__ int hist[kPermWaves][kMaxExperts];
  __shared__ int scan[kMaxExperts + 1];
  __shared__ int picks[kTopkSmallMaxT * 8];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  if (wave < T) {  // wave-uniform
    float v[4];
    router_logits_wave<false>(partial, nsplit, bias, wave, T, E, lane, v);
    topk_softmax_wave(v, E, k, lane, topk_idx + (int64_t)wave * k, topk_w + (int64_t)wave * k, picks + wave * k);
  }
  __syncthreads();
  permute_block<kPermWaves>([&](int64_t s) { return picks[s]; }, T * k, E, offsets, sorted_slot, slot_row, hist,
                            scan);
}

bool topk_permute_fits(int64_t T, int E, int k) {
  return T * k <= kTopkPermMaxSlots && T < 1024 && E <= kMaxExperts && k <= 8;
}

hipError_t launch_router_topk_permute(const float *partial, int nsplit, const float *bias, int64_t T, int E, int k,
                                      int32_t *topk_idx, float *topk_w, int *counter, int32_t *offsets,
                                      int32_t *sorted_slot, int32_t *slot_row, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  if (T <= kTopkSmallMaxT) {
    hipLaunchKernelGGL(router_topk_permute_small_kernel, dim3(1), dim3(kPermThreads), 0, stream, partial, nsplit, bias,
                       T, E, k, topk_idx, topk_w, offsets, sorted_slot, slot_row);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(router_topk_permute_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream, partial, nsplit,
                     bias, T, E, k, topk_idx, topk_w, counter, offsets, sorted_slot, slot_row);
  return hipGetLastError();
}

int64_t permute_scratch_ints(int64_t S, int E) {
  return S > kPermSingleMax ? ((S + kPermChunk - 1) / kPermChunk) * kPermWaves * (int64_t)E : 0;
}

hipError_t launch_permute(const int32_t *topk_idx, int64_t S, int E, int32_t *offsets,
                          int32_t *sorted_slot, int32_t *slot_row, int32_t *scratch, hipStream_t stream) {
  if (S <= kPermSingleMax || scratch == nullptr) {
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, stream, topk_idx, S, E, offsets,
                       sorted_slot, slot_row);
    return hipGetLastError();
  }
  const int nchunks = (int)((S + kPermChunk - 1) / kPermChunk);
  hipLaunchKernelGGL(permute_hist_kernel, dim3(nchunks), dim3(kPermThreads), 0, stream, topk_idx, S, E, scratch);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(nchunks), dim3(kPermThreads), 0, stream, topk_idx, S, E, nchunks,
                     scratch, offsets, sorted_slot, slot_row);
  return hipGetLastError();
}

}  // namespace moe
