// Row-major -> tiled conversion of weight and MX32 scale matrices (the tiled
// layout is defined in include/moe.h at moe_layout).  One-time, load-time
// work: one thread per destination 16-byte chunk (weights) or 4-byte word
// (scales), coalesced writes, gathered reads.
#include "kernels.hpp"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void pack_weights_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                           int64_t n_chunks, int32_t row_chunks) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= n_chunks) return;
  // destination chunk q = ((tile * 2 + half) * 64 + lane), tile = rb * nkt + kt
  const int lane = (int)(q & 63);
  const int64_t half_idx = q >> 6;
  const int half = (int)(half_idx & 1);
  const int64_t tile = half_idx >> 1;
  const int nkt = row_chunks / 8;
  const int64_t rb = tile / nkt;
  const int kt = (int)(tile - rb * nkt);
  const int64_t row = rb * 16 + (lane & 15);
  const int chunk = kt * 8 + half * 4 + (lane >> 4);
  dst[q] = src[row * row_chunks + chunk];
}

__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t* __restrict__ src, uint32_t* __restrict__ dst,
                                                          int64_t n_words, int32_t scale_bytes) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= n_words) return;
  // destination word q holds bytes 4q..4q+3 = (tile, qq, rows 4w..4w+3)
  const int64_t tile = q >> 4;
  const int within = (int)(q & 15);  // 4-byte word inside the 64-byte tile
  const int qq = within >> 2;        // scale index inside the tile's K slice
  const int r0 = (within & 3) * 4;   // first tile row of this word
  const int nkt = scale_bytes / 4;
  const int64_t rb = tile / nkt;
  const int kt = (int)(tile - rb * nkt);
  uint32_t v = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = rb * 16 + r0 + i;
    v |= (uint32_t)src[row * scale_bytes + kt * 4 + qq] << (8 * i);
  }
  dst[q] = v;
}

}  // namespace

hipError_t launch_pack_weights(const void* src, void* dst, int64_t rows, int32_t row_bytes, hipStream_t s) {
  const int64_t n = rows * (row_bytes / 16);
  if (n == 0) return hipSuccess;
  const int64_t grid = (n + 255) / 256;
  hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const uint4*>(src),
                     static_cast<uint4*>(dst), n, row_bytes / 16);
  return hipGetLastError();
}

hipError_t launch_pack_scales(const void* src, void* dst, int64_t rows, int32_t scale_bytes, hipStream_t s) {
  const int64_t n = rows * scale_bytes / 4;
  if (n == 0) return hipSuccess;
  const int64_t grid = (n + 255) / 256;
  hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const uint8_t*>(src),
                     static_cast<uint32_t*>(dst), n, scale_bytes);
  return hipGetLastError();
}

}  // namespace moe
