// Routing prologue for gfx950: one wave64 per token does
//  * the shared-expert gate gamma_t = sigmoid(x_t . g) as a K-length dot
//    product with the sigmoid folded in (vLLM PR 56789, "Commits": the 1x1xK
//    GEMM becomes a dot product; fp32 accumulation);
//  * the in-layer MX-32 quantisation of bf16 x (OCP MX v1.0 rule; AITER PR
//    6106, "Technical Details": 32-element K blocks);
//  * top-k / biased grouped top-k routing with the routed scaling factor
//    folded into the weights (vLLM PR 65207, "Purpose", commit 1), with
//    deterministic tie-breaks (equal scores -> lower index).
// Selection keys are (order-preserving score bits << 32 | ~index), so one
// 64-bit wave max per round (two DPP reductions) picks the winner and applies
// the tie rule.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kRouteWaves = 4;
constexpr int kMaxE = 512;

__device__ void gate_dot_wave(const RouteParams& p, int t, int lane, float* gamma_out_val) {
  float sum = 0.f;
  if (p.x_f32) {
    const float4* xr = reinterpret_cast<const float4*>(static_cast<const float*>(p.x) + (size_t)t * p.H);
    const float4* gr = reinterpret_cast<const float4*>(p.gate_w);
    for (int c = lane; c < p.H / 4; c += kWave) {
      float4 a = xr[c], b = gr[c];
      sum += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
    }
  } else {
    const uint4* xr = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.x) + (size_t)t * p.H);
    const uint4* gr = reinterpret_cast<const uint4*>(p.gate_w);
    for (int c = lane; c < p.H / 8; c += kWave) {
      uint4 a = xr[c], b = gr[c];
      uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sum += bf16_to_f32(av[q] & 0xFFFFu) * bf16_to_f32(bv[q] & 0xFFFFu);
        sum += bf16_to_f32(av[q] >> 16) * bf16_to_f32(bv[q] >> 16);
      }
    }
  }
  sum = dpp_wave_sum(sum);
  *gamma_out_val = spec_sigmoid(sum);
}

// MX-32 quantisation of one bf16 row: 4 lanes per 32-element block.
__device__ void mx_quant_row(const uint16_t* xr, int H, uint8_t* qr, uint8_t* sr, int lane) {
  for (int base = 0; base < H; base += 8 * kWave) {
    int c0 = base + lane * 8;  // first element of this lane's 8
    bool active = c0 < H;
    uint4 v = active ? *reinterpret_cast<const uint4*>(xr + c0) : make_uint4(0, 0, 0, 0);
    float f[8];
    uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[2 * q] = bf16_to_f32(vv[q] & 0xFFFFu);
      f[2 * q + 1] = bf16_to_f32(vv[q] >> 16);
    }
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(f[q]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
    // shared exponent floor(log2 amax) - 8, clamped to [-127, 127]; zero block -> -127
    uint32_t ab = __float_as_uint(amax);
    int eb = (int)((ab >> 23) & 0xFF);
    int X = (eb == 0) ? -127 : (eb - 127 - 8);
    X = X < -127 ? -127 : (X > 127 ? 127 : X);
    float mul = __builtin_ldexpf(1.0f, -X);
    uint32_t w0 = pack4_e4m3(f[0] * mul, f[1] * mul, f[2] * mul, f[3] * mul);
    uint32_t w1 = pack4_e4m3(f[4] * mul, f[5] * mul, f[6] * mul, f[7] * mul);
    if (active) {
      *reinterpret_cast<uint2*>(qr + c0) = make_uint2(w0, w1);
      if ((lane & 3) == 0) sr[c0 / 32] = (uint8_t)(X + 127);
    }
  }
}

__global__ __launch_bounds__(kWave* kRouteWaves) void route_kernel(RouteParams p) {
  __shared__ float s_sel[kRouteWaves][kMaxE];
  __shared__ float s_val[kRouteWaves][kMaxE];
  const int wv = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * kRouteWaves + wv;
  if (t >= p.T) return;

  float gamma = 1.0f;
  if (p.gate_w != nullptr) {
    gate_dot_wave(p, t, lane, &gamma);
    if (lane == 0 && p.gamma_out != nullptr) p.gamma_out[t] = gamma;
  } else if (p.gamma_in != nullptr) {
    gamma = p.gamma_in[t];
  }
  if (p.xq != nullptr) {
    mx_quant_row(static_cast<const uint16_t*>(p.x) + (size_t)t * p.H, p.H, p.xq + (size_t)t * p.H,
                 p.xs + (size_t)t * (p.H / 32), lane);
  }
  if (!p.do_route) return;

  const int E = p.E;
  float* sel = s_sel[wv];
  float* val = s_val[wv];
  const float* lrow = p.logits + (size_t)t * E;
  float lmax = -INFINITY;
  for (int e = lane; e < E; e += kWave) {
    float l = lrow[e];
    lmax = fmaxf(lmax, l);
    if (p.score == 0) {
      sel[e] = l;
      val[e] = l;
    } else {
      float sg = spec_sigmoid(l);
      float b = p.bias ? p.bias[e] : 0.0f;
      sel[e] = __fadd_rn(sg, b);
      val[e] = sg;
    }
  }
  lmax = wave_max(lmax);
  wave_lds_sync();

  // ---- group selection ----
  uint64_t kept = ~0ull;  // bit g set: group g eligible
  int eg = E;
  if (p.n_group > 1) {
    eg = E / p.n_group;
    uint64_t gkey = 0;
    if (lane < p.n_group) {
      float t1 = -INFINITY, t2 = -INFINITY;
      for (int i = 0; i < eg; ++i) {
        float v = sel[lane * eg + i];
        if (v > t1) {
          t2 = t1;
          t1 = v;
        } else if (v > t2) {
          t2 = v;
        }
      }
      float gs = (p.gtopk == 2) ? __fadd_rn(t1, t2) : t1;
      gkey = ((uint64_t)float_key(gs) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)lane);
    }
    kept = 0;
    for (int r = 0; r < p.topk_group; ++r) {
      uint64_t m = dpp_wave_max_key(gkey);
      int g = (int)(0xFFFFFFFFu - (uint32_t)(m & 0xFFFFFFFFu));
      kept |= 1ull << g;
      if (lane == g) gkey = 0;
    }
  }

  // ---- top-k ----
  constexpr int NPL = kMaxE / kWave;
  uint64_t cand[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    int e = lane + i * kWave;
    bool ok = e < E && ((kept >> (e / eg)) & 1ull);
    cand[i] = ok ? (((uint64_t)float_key(sel[e]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e)) : 0ull;
  }
  int my_id = 0;
  float my_v = 0.f;
  for (int j = 0; j < p.topk; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) best = cand[i] > best ? cand[i] : best;
    uint64_t m = dpp_wave_max_key(best);
    int e = (int)(0xFFFFFFFFu - (uint32_t)(m & 0xFFFFFFFFu));
    if ((e % kWave) == lane) {
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        if (lane + i * kWave == e) cand[i] = 0;
    }
    if (lane == j) {
      my_id = e;
      my_v = val[e];
    }
  }

  // ---- weights ----
  float wgt = 0.f;
  if (p.score == 0) {
    float ex = (lane < p.topk) ? __expf(my_v - lmax) : 0.f;
    float denom;
    if (p.renorm) {
      denom = dpp_wave_sum(ex);
    } else {
      float part = 0.f;
      for (int e = lane; e < E; e += kWave) part += __expf(val[e] - lmax);
      denom = dpp_wave_sum(part);
    }
    wgt = ex / denom;
  } else {
    float sg = (lane < p.topk) ? my_v : 0.f;
    float denom = p.renorm ? dpp_wave_sum(sg) : 1.0f;
    wgt = sg / denom;
  }
  wgt *= p.scale;
  const int kt = p.topk + p.n_pseudo;
  if (lane < p.topk) {
    p.ids[(size_t)t * kt + lane] = my_id;
    p.w[(size_t)t * kt + lane] = wgt;
  } else if (lane < kt) {
    p.ids[(size_t)t * kt + lane] = E + (lane - p.topk);
    p.w[(size_t)t * kt + lane] = gamma;
  }
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
  dim3 grid((p.T + kRouteWaves - 1) / kRouteWaves);
  hipLaunchKernelGGL(route_kernel, grid, dim3(kWave * kRouteWaves), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gate_dot(const void* x, int x_f32, const void* g, int T, int H, int apply_sigmoid,
                           float* out, hipStream_t s) {
  hipLaunchKernelGGL(gate_dot_kernel, dim3(T), dim3(256), 0, s, x, x_f32, g, H, apply_sigmoid, out);
  return hipGetLastError();
}

}  // namespace moe
