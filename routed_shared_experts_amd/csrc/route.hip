// Routing prologue for gfx950 (the per-token body is route_token in
// prologue.hpp): one wave64 per token does the routing with the fused
// shared-expert gate dot and the fused MX-32 quantisation of bf16 x; extra
// workgroups may clear a region (the stage-2 arrival counters when no sort
// launch follows).  The standalone gate dot kernel serves any H.
#include "prologue.hpp"

namespace moe {

constexpr int kRouteWaves = 4;

// NPL: experts per lane, the smallest of 1, 2, 4, 8 with E <= 64 NPL
template <int NPL>
__global__ __launch_bounds__(kWave* kRouteWaves) void route_kernel(RouteParams p) {
  __shared__ float s_sel[kRouteWaves][kWave * NPL];
  __shared__ float s_val[kRouteWaves][kWave * NPL];
  const int nroute = (p.T + kRouteWaves - 1) / kRouteWaves;
  if ((int)blockIdx.x >= nroute) {
    clear_region(p.zero_ptr, p.zero_vec, nroute);
    return;
  }
  const int wv = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * kRouteWaves + wv;
  if (t >= p.T) return;
  route_token<NPL>(p, t, lane, s_sel[wv], s_val[wv], p.logits + (size_t)t * p.E);
}

// Standalone gate dot: one workgroup of 256 threads per token, any H.
__global__ __launch_bounds__(256) void gate_dot_kernel(const void* x, int x_f32, const void* g, int H,
                                                      int apply_sigmoid, float* out) {
  __shared__ float red[256 / kWave];
  const int t = blockIdx.x;
  float sum = 0.f;
  if (x_f32) {
    const float* xr = static_cast<const float*>(x) + (size_t)t * H;
    const float* gr = static_cast<const float*>(g);
    for (int i = threadIdx.x * 4; i < H; i += 256 * 4) {
      float4 a = *reinterpret_cast<const float4*>(xr + i);
      float4 b = *reinterpret_cast<const float4*>(gr + i);
      sum += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
    }
  } else {
    const uint16_t* xr = static_cast<const uint16_t*>(x) + (size_t)t * H;
    const uint16_t* gr = static_cast<const uint16_t*>(g);
    for (int i = threadIdx.x * 8; i < H; i += 256 * 8) {
      uint4 a = *reinterpret_cast<const uint4*>(xr + i);
      uint4 b = *reinterpret_cast<const uint4*>(gr + i);
      uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sum += bf16_to_f32(av[q] & 0xFFFFu) * bf16_to_f32(bv[q] & 0xFFFFu);
        sum += bf16_to_f32(av[q] >> 16) * bf16_to_f32(bv[q] >> 16);
      }
    }
  }
  sum = wave_sum(sum);
  if ((threadIdx.x % kWave) == 0) red[threadIdx.x / kWave] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = red[0] + red[1] + red[2] + red[3];
    out[t] = apply_sigmoid ? spec_sigmoid(s) : s;
  }
}

hipError_t launch_route(const RouteParams& p, hipStream_t s) {
  const dim3 grid((unsigned)((p.T + kRouteWaves - 1) / kRouteWaves + clear_blocks(p.zero_vec, kWave * kRouteWaves)));
  const dim3 block(kWave * kRouteWaves);
  if (p.E <= kWave)
    hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, s, p);
  else if (p.E <= 2 * kWave)
    hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, s, p);
  else if (p.E <= 4 * kWave)
    hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, s, p);
  else
    hipLaunchKernelGGL(route_kernel<kMaxE / kWave>, grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gate_dot(const void* x, int x_f32, const void* g, int T, int H, int apply_sigmoid,
                           float* out, hipStream_t s) {
  hipLaunchKernelGGL(gate_dot_kernel, dim3(T), dim3(256), 0, s, x, x_f32, g, H, apply_sigmoid, out);
  return hipGetLastError();
}

}  // namespace moe
