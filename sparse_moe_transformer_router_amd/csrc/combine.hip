// Weighted combine: out[t] = sum_j w[t][j] * y[slot_row[t*k + j]], the routing-weighted sum
// of the picked experts' outputs (review of the from-scratch gpt-oss-20B at pomoai.com,
// section 3.4). A gather in rank order with fp32 accumulation, so no atomics and a
// deterministic result; the output is rounded to nearest-even bf16 or kept in fp32. With a
// residual (the block's input row, review section 3.3: a residual path joins the FFN's
// output and its input), it is added to the sum last, before the one rounding.
#include "common.h"
#include "kernels.h"

namespace moe {

// Every load is issued unconditionally from an in-bounds address and the unused values are
// dropped at their use (a pick outside [0, S) reads row 0 and is skipped; without a residual
// the residual load reads y's first bytes and is ignored): with loads under branches the
// compiler waited for the rows two at a time, one memory round trip per pair. K = k.
template <int K, bool BY_SLOT>
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y,
                                                      const int32_t *__restrict__ slot_row,
                                                      const float *__restrict__ topk_w, int64_t T, int H,
                                                      const uint16_t *__restrict__ residual,
                                                      void *__restrict__ out, int out_f32) {
  const int chunks = (H / 4 + blockDim.x - 1) / blockDim.x;
  const int64_t t = blockIdx.x / chunks;
  const int h = ((blockIdx.x % chunks) * blockDim.x + threadIdx.x) * 4;
  if (h >= H) return;
  const int64_t S = T * K;
  int32_t r[K];
  float w[K];
  bool ok[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    r[j] = slot_row[t * K + j];
    w[j] = topk_w[t * K + j];
    ok[j] = (uint32_t)r[j] < (uint64_t)S;
  }
  f32x4_t v[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    // slot order: the row is the slot itself, so this load does not wait for slot_row's
    const int64_t row = BY_SLOT ? t * K + j : (int64_t)(ok[j] ? r[j] : 0);
    v[j] = *reinterpret_cast<const f32x4_t *>(y + row * H + h);
  }
  // y holds S >= T rows of H floats, so its first T H halves cover the dummy residual read
  const uint2 res = *reinterpret_cast<const uint2 *>(
      (residual != nullptr ? residual : reinterpret_cast<const uint16_t *>(y)) + t * H + h);
  // the residual's value is taken here, with the rows' (else the compiler sinks its load into
  // the residual branch, a second round trip after the rows)
  asm volatile("" ::"v"(res.x), "v"(res.y));
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < K; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = ok[j] ? fmaf(w[j], v[j][i], acc[i]) : acc[i];
  if (residual != nullptr) {
    acc[0] += __uint_as_float(res.x << 16);
    acc[1] += __uint_as_float(res.x & 0xffff0000u);
    acc[2] += __uint_as_float(res.y << 16);
    acc[3] += __uint_as_float(res.y & 0xffff0000u);
  }
  if (out_f32) {
    *reinterpret_cast<f32x4_t *>(reinterpret_cast<float *>(out) + t * H + h) = acc;
  } else {
    const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
    uint32_t *o = reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(out) + t * H + h);
    o[0] = lo;
    o[1] = hi;
  }
}

hipError_t launch_combine(const float *y, const int32_t *slot_row, const float *topk_w, int64_t T,
                          int k, int H, void *out, bool out_f32, hipStream_t stream, const uint16_t *residual,
                          bool by_slot) {
  const int threads = 256;
  const int64_t chunks = (H / 4 + threads - 1) / threads;
  dim3 grid((unsigned)(T * chunks));
#define MOE_COMBINE(K)                                                                                          \
  do {                                                                                                          \
    if (by_slot)                                                                                                \
      hipLaunchKernelGGL((combine_kernel<K, true>), grid, dim3(threads), 0, stream, y, slot_row, topk_w, T, H,  \
                         residual, out, out_f32 ? 1 : 0);                                                       \
    else                                                                                                        \
      hipLaunchKernelGGL((combine_kernel<K, false>), grid, dim3(threads), 0, stream, y, slot_row, topk_w, T, H, \
                         residual, out, out_f32 ? 1 : 0);                                                       \
  } while (0)
  switch (k) {
    case 1: MOE_COMBINE(1); break;
    case 2: MOE_COMBINE(2); break;
    case 3: MOE_COMBINE(3); break;
    case 4: MOE_COMBINE(4); break;
    case 5: MOE_COMBINE(5); break;
    case 6: MOE_COMBINE(6); break;
    case 7: MOE_COMBINE(7); break;
    case 8: MOE_COMBINE(8); break;
    default: return hipErrorInvalidValue;
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// The smallest-batch path's expert outputs arrive as nslice partial rows per slot (one per
// 32-activation block of the expert's hidden layer, part[s][row][H]). Their sum has one fixed
// order, shared by the combine below and by launch_slice_sum: thread group g (of kSlGroups)
// adds slices g and g + kSlGroups, then the groups meet in LDS by halving, group g taking
// group g + 32, then g + 16, ..., g + 1. A workgroup of 256 threads covers kSlQuads column
// quads of up to 8 rows (a token's picks); every load a thread makes (at most 2 per row) is
// issued before its first add, so the sum costs one memory round trip.
constexpr int kSlGroups = 64;
constexpr int kSlQuads = 256 / kSlGroups;
constexpr int kSlRows = 8;
static_assert(2 * kSlGroups == kSmallMaxSlices, "the sliced combine's limit");

// red[0][j][q] = the slices' sum for row rows(j), columns h .. h + 3, j < nrows (a workgroup-wide
// call: every thread takes part, the result is valid after it returns).
template <typename Rows>
__device__ __forceinline__ void sliced_rows_sum(const float *__restrict__ part, int nslice, int64_t stride, int H,
                                                Rows rows, int nrows, int h, bool h_ok, int q, int g,
                                                f32x4_t (*red)[kSlRows][kSlQuads]) {
  // every load is issued from an in-bounds address (unused ones read part[0] and are zeroed at
  // their use), so all of them are in flight together
  f32x4_t u[kSlRows][2];
#pragma unroll
  for (int j = 0; j < kSlRows; ++j) {
    const int64_t r = rows(j < nrows ? j : 0);
    const bool ok = j < nrows && h_ok && r >= 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int sl = g + kSlGroups * i;
      const bool use = ok && sl < nslice;
      const f32x4_t x = *reinterpret_cast<const f32x4_t *>(part + (use ? sl * stride + r * H + h : 0));
      u[j][i] = use ? x : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int j = 0; j < kSlRows; ++j) {
    if (j >= nrows) break;
    f32x4_t v = u[j][0];
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] += u[j][1][c];
    red[g][j][q] = v;
  }
  __syncthreads();
#pragma unroll
  for (int off = kSlGroups / 2; off >= 1; off /= 2) {
    if (g < off) {
#pragma unroll
      for (int j = 0; j < kSlRows; ++j) {
        if (j >= nrows) break;
        f32x4_t v = red[g][j][q];
        const f32x4_t w = red[g + off][j][q];
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] += w[c];
        red[g][j][q] = v;
      }
    }
    __syncthreads();
  }
}

// out[t] = sum_j w[t][j] y_j (+ residual), y_j the slices' sum for slot (t, j), then the one
// rounding as combine_kernel.
__global__ __launch_bounds__(256) void combine_sliced_kernel(const float *__restrict__ part, int nslice,
                                                             const int32_t *__restrict__ slot_row,
                                                             const float *__restrict__ topk_w, int64_t T, int k,
                                                             int H, const uint16_t *__restrict__ residual,
                                                             void *__restrict__ out, int out_f32) {
  __shared__ f32x4_t red[kSlGroups][kSlRows][kSlQuads];
  const int nq = (H / 4 + kSlQuads - 1) / kSlQuads;
  const int64_t t = blockIdx.x / nq;
  const int q = threadIdx.x % kSlQuads, g = threadIdx.x / kSlQuads;
  const int h = ((blockIdx.x % nq) * kSlQuads + q) * 4;
  const int64_t S = T * k;
  const bool h_ok = h < H;
  sliced_rows_sum(
      part, nslice, S * H, H,
      [&](int j) -> int64_t {
        const int32_t r = slot_row[t * k + j];
        return (uint32_t)r < (uint64_t)S ? (int64_t)r : -1;
      },
      k, h, h_ok, q, g, red);
  if (g != 0 || !h_ok) return;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int32_t r = slot_row[t * k + j];
    if ((uint32_t)r >= (uint64_t)S) continue;
    const f32x4_t y = red[0][j][q];
    const float w = topk_w[t * k + j];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, y[i], acc[i]);
  }
  if (residual != nullptr) {
    const uint2 res = *reinterpret_cast<const uint2 *>(residual + t * H + h);
    acc[0] += __uint_as_float(res.x << 16);
    acc[1] += __uint_as_float(res.x & 0xffff0000u);
    acc[2] += __uint_as_float(res.y << 16);
    acc[3] += __uint_as_float(res.y & 0xffff0000u);
  }
  if (out_f32) {
    *reinterpret_cast<f32x4_t *>(reinterpret_cast<float *>(out) + t * H + h) = acc;
  } else {
    const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
    uint32_t *o = reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(out) + t * H + h);
    o[0] = lo;
    o[1] = hi;
  }
}

hipError_t launch_combine_sliced(const float *part, int nslice, const int32_t *slot_row, const float *topk_w,
                                 int64_t T, int k, int H, void *out, bool out_f32, hipStream_t stream,
                                 const uint16_t *residual) {
  if (nslice < 1 || nslice > kSmallMaxSlices || k > kSlRows) return hipErrorInvalidValue;
  const int nq = (H / 4 + kSlQuads - 1) / kSlQuads;
  hipLaunchKernelGGL(combine_sliced_kernel, dim3((unsigned)(T * nq)), dim3(256), 0, stream, part, nslice, slot_row,
                     topk_w, T, k, H, residual, out, out_f32 ? 1 : 0);
  return hipGetLastError();
}

// y[r] = the slices' sum in the order above (the step API's expert outputs on the
// smallest-batch path): a workgroup covers kSlQuads column quads of one row.
__global__ __launch_bounds__(256) void slice_sum_kernel(const float *__restrict__ part, int nslice, int64_t S, int H,
                                                        float *__restrict__ y) {
  __shared__ f32x4_t red[kSlGroups][kSlRows][kSlQuads];
  const int nq = (H / 4 + kSlQuads - 1) / kSlQuads;
  const int64_t r = blockIdx.x / nq;
  const int q = threadIdx.x % kSlQuads, g = threadIdx.x / kSlQuads;
  const int h = ((blockIdx.x % nq) * kSlQuads + q) * 4;
  const bool h_ok = h < H;
  sliced_rows_sum(part, nslice, S * H, H, [&](int) -> int64_t { return r; }, 1, h, h_ok, q, g, red);
  if (g != 0 || !h_ok) return;
  *reinterpret_cast<f32x4_t *>(y + r * H + h) = red[0][0][q];
}

hipError_t launch_slice_sum(const float *part, int nslice, int64_t S, int H, float *y, hipStream_t stream) {
  if (S <= 0) return hipSuccess;
  if (nslice < 1 || nslice > kSmallMaxSlices) return hipErrorInvalidValue;
  const int nq = (H / 4 + kSlQuads - 1) / kSlQuads;
  hipLaunchKernelGGL(slice_sum_kernel, dim3((unsigned)(S * nq)), dim3(256), 0, stream, part, nslice, S, H, y);
  return hipGetLastError();
}

}  // namespace moe
