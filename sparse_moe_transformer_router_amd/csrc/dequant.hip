// MXFP4 -> fp32 decode, exported for tests of the decode step (OCP MX v1.0 element and
// scale encodings; the gpt-oss walkthrough at pnsm.cn, sections 1 and 4, names the format).
// Exact for every code and scale byte: built from the bit fields with ldexpf, so fp32
// subnormal results are kept, overflow gives +-inf and scale 0xFF gives NaN.
#include "common.h"
#include "kernels.h"

namespace moe {

// One thread decodes one 32-element block: 16 code bytes and one scale byte.
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ codes,
                                                      const uint8_t *__restrict__ scales,
                                                      int64_t nblocks, float *__restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const u32x4_t c = *reinterpret_cast<const u32x4_t *>(codes + b * 16);
  const uint32_t s = scales[b];
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t code = (c[i >> 3] >> ((i & 7) * 4)) & 0xFu;
    const uint32_t e = (code >> 1) & 3u, m = code & 1u;
    // magnitude = (e == 0 ? m/2 : (1 + m/2) * 2^(e-1)) = (2*[e>0] + m) * 2^(max(e,1) - 2)
    const float mag = (float)((e ? 2u : 0u) + m);
    float val = ldexpf(mag, (int)(e ? e : 1u) - 2 + (int)s - 127);
    val = (code & 8u) ? -val : val;
    v[i] = (s == 255u) ? __uint_as_float(0x7fc00000u) : val;
  }
  f32x4_t *o = reinterpret_cast<f32x4_t *>(out + b * 32);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    f32x4_t t = {v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
    o[q] = t;
  }
}

hipError_t launch_dequant(const uint8_t *codes, const uint8_t *scales, int64_t n, float *out,
                          hipStream_t stream) {
  const int64_t nb = n / 32;
  const int threads = 256;
  const int64_t grid = (nb + threads - 1) / threads;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)grid), dim3(threads), 0, stream, codes, scales,
                     nb, out);
  return hipGetLastError();
}

}  // namespace moe
