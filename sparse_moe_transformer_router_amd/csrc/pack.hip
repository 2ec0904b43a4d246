// Re-order a row-major MXFP4 matrix into the tiled layout the expert kernels stream.
//
// Tile (G, c) of expert e: rows 32G..32G+31, elements 128c..128c+127 (MX blocks 4c..4c+3).
// Codes: 2 KB = two 1 KB halves p = 0, 1; in half p, lane l (0..63) holds the 16 code bytes of
// MX block 4c + 2p + l/32 of row 32G + l%32. Scales: 32 rows x 4 bytes (blocks 4c..4c+3).
// So a wave-wide 16-byte load reads a contiguous 1 KB, a lane's two loads give the A operand
// of four 32x32x16 bf16 MFMA steps per half (or one 32x32x64 FP4 step), and a lane's four
// block scales are one dword. Elements past k: zero codes with scale 127.
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void pack_kernel(const uint8_t *__restrict__ codes,
                                                   const uint8_t *__restrict__ scales, int64_t ntiles, int nchunk,
                                                   int K, uint8_t *__restrict__ pcodes,
                                                   uint8_t *__restrict__ pscales) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t tile = tid / (2 * kWave);  // (e * NG + G) * nchunk + c
  if (tile >= ntiles) return;
  const int p = (int)(tid / kWave) & 1;
  const int lane = (int)(tid % kWave);
  const int r = lane % 32, kh = lane / 32;
  const int c = (int)(tile % nchunk);
  const int64_t eg = tile / nchunk;  // e * NG + G
  const int64_t row = eg * 32 + r;   // global row over all experts (n rows per expert)
  const int KB = K / 32;
  const int64_t row_bytes = K / 2;
  const int b = 4 * c + 2 * p + kh;
  const u32x4_t v = (b < KB) ? *reinterpret_cast<const u32x4_t *>(codes + row * row_bytes + 16 * b)
                             : u32x4_t{0u, 0u, 0u, 0u};
  *reinterpret_cast<u32x4_t *>(pcodes + tile * 2048 + p * 1024 + lane * 16) = v;
  if (p == 0 && kh == 0) {
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int bj = 4 * c + j;
      const uint32_t sb = (bj < KB) ? scales[row * KB + bj] : 127u;
      s |= sb << (8 * j);
    }
    *reinterpret_cast<uint32_t *>(pscales + tile * 128 + r * 4) = s;
  }
}

hipError_t launch_pack(const uint8_t *codes, const uint8_t *scales, int E, int N, int K, uint8_t *pcodes,
                       uint8_t *pscales, hipStream_t stream) {
  const int NG = N / 32;
  const int nchunk = (K / 32 + 3) / 4;
  const int64_t ntiles = (int64_t)E * NG * nchunk;
  const int64_t threads = ntiles * 2 * kWave;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, codes, scales,
                     ntiles, nchunk, K, pcodes, pscales);
  return hipGetLastError();
}

}  // namespace moe
