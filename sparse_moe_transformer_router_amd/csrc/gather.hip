// Expert-sorted copy of the layer input for the prefill GEMM: row r of the copy is the input
// row of the token that sorted slot r belongs to (slot s = token * k + rank, so the token
// is s / k). The copy makes every GEMM tile's slot rows one contiguous block, so the GEMM
// needs no per-row index loads while its LDS DMA stream is in flight.
#include "common.h"
#include "kernels.h"

namespace moe {

// One wave per sorted row, four rows per workgroup; each lane moves 16-byte pieces.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t *__restrict__ x,
                                                          const int32_t *__restrict__ sorted_slot, int k, int64_t S,
                                                          int H, uint16_t *__restrict__ xs) {
  const int64_t r = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (r >= S) return;
  const int lane = threadIdx.x % kWave;
  const int64_t t = sorted_slot[r] / k;
  const u32x4_t *src = reinterpret_cast<const u32x4_t *>(x + t * H);
  u32x4_t *dst = reinterpret_cast<u32x4_t *>(xs + r * H);
  for (int c = lane; c < H / 8; c += kWave) dst[c] = src[c];
}

hipError_t launch_gather_rows(const uint16_t *x, const int32_t *sorted_slot, int k, int64_t S, int H,
                              uint16_t *xs, hipStream_t stream) {
  if (S <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)((S + 3) / 4)), dim3(256), 0, stream, x, sorted_slot, k, S, H,
                     xs);
  return hipGetLastError();
}

}  // namespace moe
