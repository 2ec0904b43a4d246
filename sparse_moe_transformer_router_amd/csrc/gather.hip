// Expert-sorted copy of the layer input for the prefill GEMM: row r of the copy is the input
// row of the token that sorted slot r belongs to (slot s = token * k + rank, so the token
// is s / k). The copy makes every GEMM tile's slot rows one contiguous block, so the GEMM
// needs no per-row index loads while its LDS DMA stream is in flight.
#include "common.h"
#include "kernels.h"
#include "mx_act.h"

namespace moe {

// One wave per sorted row, four rows per workgroup; each lane moves 16-byte pieces.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t *__restrict__ x,
                                                          const int32_t *__restrict__ sorted_slot, int k, int64_t S,
                                                          int H, uint16_t *__restrict__ xs) {
  const int64_t r = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (r >= S) return;
  const int lane = threadIdx.x % kWave;
  const int64_t t = sorted_slot != nullptr ? sorted_slot[r] / k : r;
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

// Gather into the two-term MXFP8 form. One wave per sorted row; a lane takes 8 consecutive
// elements (16 bytes of bf16), so a lane quad holds one 32-element block and 16 lanes one
// 128-element record (mx_store_piece); a wave covers 4 records per pass. Elements past H are
// zeros (the quad reads nothing there).
__global__ __launch_bounds__(256) void gather_rows_mx_kernel(const uint16_t *__restrict__ x,
                                                             const int32_t *__restrict__ sorted_slot, int k, int64_t S,
                                                             int H, uint8_t *__restrict__ rec,
                                                             uint8_t *__restrict__ scales) {
  const int64_t r = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (r >= S) return;  // wave-uniform
  const int lane = threadIdx.x % kWave;
  const int nrec = mx_records(H);
  const int64_t t = sorted_slot != nullptr ? sorted_slot[r] / k : r;
  const uint16_t *src = x + t * H;
  uint8_t *drow = rec + r * nrec * kMxRecBytes;
  uint8_t *srow = scales + r * nrec * kMxScBytes;
  for (int c0 = 0; c0 < nrec; c0 += 4) {
    const int c = c0 + lane / 16, j = lane % 16;
    const int e0 = c * kMxRecElems + 8 * j;  // H % 32 == 0: a piece is wholly inside or past H
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (c < nrec && e0 < H) v = *reinterpret_cast<const u32x4_t *>(src + e0);
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
    mx_store_piece(f, c, j, nrec, drow, srow);
  }
}

hipError_t launch_gather_rows_mx(const uint16_t *x, const int32_t *sorted_slot, int k, int64_t S, int H,
                                 uint8_t *rec, uint8_t *scales, hipStream_t stream) {
  if (S <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_mx_kernel, dim3((unsigned)((S + 3) / 4)), dim3(256), 0, stream, x, sorted_slot, k, S,
                     H, rec, scales);
  return hipGetLastError();
}

}  // namespace moe
