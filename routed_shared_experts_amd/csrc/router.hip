// Fused layer prologue with the router-logit GEMM (gfx950): the logits
// l = x . Wr^T of a block of tokens are computed on the matrix cores, kept in
// LDS, and the same workgroup then routes those tokens from LDS with the
// shared-expert gate dot and the MX-32 quantisation of x folded in
// (route_token).  This extends the folding the pages describe for the small
// dot products next to the MoE -- the shared-expert gate's 1 x 1 x K GEMM
// turned into a dot product with its sigmoid fused (vLLM PR 56789,
// "Commits") and the routing bias / scaling applied inside the kernel (vLLM
// PR 65207, "Purpose", commit 1) -- to the router projection itself, so the
// logits never travel through HBM between two launches.
//
// Mapping.  A workgroup of four waves owns 64 consecutive tokens, wave w the
// 16 tokens 16 w ..; every wave computes all E_pad = 16 NT experts of its
// tokens (NT 16x16 MFMA tiles, experts = rows of the A operand, tokens =
// columns).  Per K tile (128 bytes of a router-weight row: 64 bf16 or 32
// fp32 elements), the E_pad weight rows are staged once in LDS
// (XOR-swizzled 16-byte chunks, rows past E read as zero) and shared by the
// four waves; each wave reads its 16 token rows straight into B-operand
// registers (e4m3 activations are widened to bf16 on the way, exactly).  The
// fp32 accumulators are multiplied by the token's scale (e4m3 input), written
// to the logits output and to LDS, and route_token reads them from there.
#include "gemm_common.hpp"
#include "prologue.hpp"

namespace moe {

constexpr int kRtTokens = 64;
constexpr int kRtThreads = 256;

template <int NT>
struct RouterSmem {
  static constexpr int EP = 16 * NT;
  static constexpr int kTile = EP * 128;            // one K tile of the router weights
  static constexpr int kLogits = kRtTokens * EP * 4;  // the block's logits, fp32
  union {
    uint8_t w[kTile];
    float logit[kRtTokens * EP];
    uint8_t raw[kTile > kLogits ? kTile : kLogits];
  };
  float sel[kRtThreads / kWave][EP];
  float val[kRtThreads / kWave][EP];
};

// Eight e4m3 codes (two dwords) -> eight bf16 values (exact: every e4m3 value
// is a bf16 value).
__device__ __forceinline__ uint4 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  uint32_t out[4];
  const uint32_t in[2] = {lo, hi};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const auto lo2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)in[h], false);  // bytes 0, 1
    const auto hi2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)in[h], true);   // bytes 2, 3
    out[2 * h] = (__float_as_uint(lo2[0]) >> 16) | (__float_as_uint(lo2[1]) & 0xFFFF0000u);
    out[2 * h + 1] = (__float_as_uint(hi2[0]) >> 16) | (__float_as_uint(hi2[1]) & 0xFFFF0000u);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// XF: x format (0 fp32 with fp32 router weights; 1 bf16; 2 e4m3 with an fp32
// scale per token; router weights bf16 for 1 and 2).  NPL: experts per lane
// of the routing (E <= 64 NPL).
template <int XF, int NT, int NPL>
__global__ __launch_bounds__(kRtThreads) void router_kernel(RouterParams g, RouteParams rp) {
  constexpr int EP = 16 * NT;
  constexpr int FMT = XF == 0 ? FMT_F32 : FMT_BF16;
  constexpr int XB = XF == 0 ? 4 : (XF == 1 ? 2 : 1);  // bytes per x element
  constexpr int KE = XF == 0 ? 32 : 64;                // elements per K tile
  __shared__ __attribute__((aligned(16))) RouterSmem<NT> sm;

  const int nblk = (g.T + kRtTokens - 1) / kRtTokens;
  if ((int)blockIdx.x >= nblk) {
    clear_region(rp.zero_ptr, rp.zero_vec, nblk);
    return;
  }
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int g4 = lane / 16, r = lane % 16;
  const int t0 = blockIdx.x * kRtTokens;
  const int tok = t0 + 16 * wv + r;
  const bool tok_ok = tok < g.T;
  const size_t wrow = (size_t)g.H * (XF == 0 ? 4 : 2);  // bytes per router-weight row
  const uint8_t* xrow = static_cast<const uint8_t*>(g.x) + (size_t)(tok_ok ? tok : 0) * g.H * XB;

  f32x4 acc[NT];
#pragma unroll
  for (int et = 0; et < NT; ++et) acc[et] = f32x4{0, 0, 0, 0};
  const int nk = g.H / KE;
  for (int kt = 0; kt < nk; ++kt) {
    // the E_pad weight rows of this K tile -> LDS
#pragma unroll 4
    for (int i = tid; i < EP * 8; i += kRtThreads) {
      const int row = i / 8, c = i % 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row < g.E) v = ld16(static_cast<const uint8_t*>(g.w) + (size_t)row * wrow + (size_t)kt * 128 + 16 * c);
      *reinterpret_cast<uint4*>(sm.w + swz(row, c)) = v;
    }
    // this lane's B operand: token tok, chunks g4 and 4 + g4 of the K tile
    uint4 b0 = make_uint4(0, 0, 0, 0), b1 = make_uint4(0, 0, 0, 0);
    if (tok_ok) {
      if constexpr (XF == 2) {
        const uint8_t* xp = xrow + (size_t)kt * 64;
        const uint2 c0 = *reinterpret_cast<const uint2*>(xp + 8 * g4);
        const uint2 c1 = *reinterpret_cast<const uint2*>(xp + 32 + 8 * g4);
        b0 = e4m3x8_to_bf16(c0.x, c0.y);
        b1 = e4m3x8_to_bf16(c1.x, c1.y);
      } else {
        const uint8_t* xp = xrow + (size_t)kt * 128;
        b0 = ld16(xp + 16 * g4);
        b1 = ld16(xp + 64 + 16 * g4);
      }
    }
    __syncthreads();
#pragma unroll
    for (int et = 0; et < NT; ++et) {
      const uint4 a0 = *reinterpret_cast<const uint4*>(sm.w + swz(16 * et + r, g4));
      const uint4 a1 = *reinterpret_cast<const uint4*>(sm.w + swz(16 * et + r, 4 + g4));
      mfma_tile<FMT>(acc[et], a0, a1, b0, b1, 0, 0);
    }
    __syncthreads();  // the next tile rewrites the weights
  }

  // logits of token 16 wv + r: experts 16 et + 4 g4 + v
  const float xs = (XF == 2 && tok_ok) ? g.x_scale[tok] : 1.0f;
#pragma unroll
  for (int et = 0; et < NT; ++et)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = 16 * et + 4 * g4 + v;
      const float l = acc[et][v] * xs;
      sm.logit[(16 * wv + r) * EP + e] = l;
      if (tok_ok && e < g.E) g.logits[(size_t)tok * g.E + e] = l;
    }
  if (!rp.do_route) return;
  __syncthreads();
  // routing (+ gate dot, + MX quantisation of x) of the wave's 16 tokens
  for (int i = 0; i < 16; ++i) {
    const int t = t0 + 16 * wv + i;
    if (t >= g.T) break;
    route_token<NPL>(rp, t, lane, sm.sel[wv], sm.val[wv], &sm.logit[(16 * wv + i) * EP]);
  }
}

template <int XF>
static hipError_t launch_router_xf(const RouterParams& g, const RouteParams& rp, hipStream_t s) {
  const int nblk = (g.T + kRtTokens - 1) / kRtTokens;
  const dim3 grid((unsigned)(nblk + (rp.do_route ? clear_blocks(rp.zero_vec, kRtThreads) : 0)));
  const dim3 block(kRtThreads);
  if (g.E <= 64)
    hipLaunchKernelGGL((router_kernel<XF, 4, 1>), grid, block, 0, s, g, rp);
  else if (g.E <= 128)
    hipLaunchKernelGGL((router_kernel<XF, 8, 2>), grid, block, 0, s, g, rp);
  else if (g.E <= 256)
    hipLaunchKernelGGL((router_kernel<XF, 16, 4>), grid, block, 0, s, g, rp);
  else
    hipLaunchKernelGGL((router_kernel<XF, 32, kMaxE / kWave>), grid, block, 0, s, g, rp);
  return hipGetLastError();
}

hipError_t launch_router(const RouterParams& g, const RouteParams& rp, hipStream_t s) {
  switch (g.x_fmt) {
    case 0: return launch_router_xf<0>(g, rp, s);
    case 1: return launch_router_xf<1>(g, rp, s);
    case 2: return launch_router_xf<2>(g, rp, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
