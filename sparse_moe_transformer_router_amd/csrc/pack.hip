// Re-order a row-major MXFP4 matrix into the tiled layout the expert kernels stream.
//
// Tile (g, c) of expert e: rows 16g..16g+15, elements 128c..128c+127 (MX blocks 4c..4c+3).
// Codes: 64 lanes x 16 bytes, lane l = r + 16q; for MFMA step j (= block 4c + j) the lane's
// bytes 4j..4j+3 are the 8 elements 32j + 8q .. 32j + 8q + 7 of row 16g + r. Scales: 16
// rows x 4 bytes. So one 16x16x32 MFMA step consumes exactly one MX block, one wave-wide
// 16-byte load reads a whole 1 KB tile, and a lane's four block scales are one dword.
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void pack_kernel(const uint8_t *__restrict__ codes,
                                                   const uint8_t *__restrict__ scales, int64_t ntiles, int NG,
                                                   int nchunk, int K, uint8_t *__restrict__ pcodes,
                                                   uint8_t *__restrict__ pscales) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t tile = tid / kWave;  // (e * NG + g) * nchunk + c
  if (tile >= ntiles) return;
  const int lane = (int)(tid % kWave);
  const int r = lane % 16, q = lane / 16;
  const int c = (int)(tile % nchunk);
  const int64_t eg = tile / nchunk;  // e * NG + g
  const int64_t row = eg * 16 + r;   // global row index over all experts (n rows per expert)
  const int KB = K / 32;
  const int64_t row_bytes = K / 2;
  u32x4_t v;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = 4 * c + j;
    v[j] = (b < KB) ? *reinterpret_cast<const uint32_t *>(codes + row * row_bytes + 16 * b + 4 * q) : 0u;
  }
  *reinterpret_cast<u32x4_t *>(pcodes + tile * 1024 + lane * 16) = v;
  if (q == 0) {
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = 4 * c + j;
      const uint32_t sb = (b < KB) ? scales[row * KB + b] : 127u;
      s |= sb << (8 * j);
    }
    *reinterpret_cast<uint32_t *>(pscales + tile * 64 + r * 4) = s;
  }
}

hipError_t launch_pack(const uint8_t *codes, const uint8_t *scales, int E, int N, int K, uint8_t *pcodes,
                       uint8_t *pscales, hipStream_t stream) {
  const int NG = N / 16;
  const int nchunk = (K / 32 + 3) / 4;
  const int64_t ntiles = (int64_t)E * NG * nchunk;
  const int64_t threads = ntiles * kWave;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, codes, scales,
                     ntiles, NG, nchunk, K, pcodes, pscales);
  return hipGetLastError();
}

}  // namespace moe
