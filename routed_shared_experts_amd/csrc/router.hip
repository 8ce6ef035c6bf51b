// Fused layer prologue with the router-logit GEMM (gfx950): the logits
// l = x . Wr^T of a block of tokens are computed on the matrix cores, kept in
// LDS, and the same workgroup then routes those tokens from LDS with the
// shared-expert gate dot and the MX-32 quantisation of x folded in
// (route_token).  This extends the folding the pages describe for the small
// dot products next to the MoE -- the shared-expert gate's 1 x 1 x K GEMM
// turned into a dot product with its sigmoid fused (vLLM PR 56789,
// "Commits") and the routing bias / scaling applied inside the kernel (vLLM
// PR 65207, "Purpose", commit 1) -- to the router projection itself, so the
// logits never travel through HBM between two launches.  It serves fp32
// activations; bf16 and e4m3 activations take a tiled GEMM instead
// (router_gemm_kernel below) and route in a second launch, which measured
// faster at every batch size on MI355X (decode 33 -> 23 us, T = 512 103 -> 53
// us, T = 8192 with H = 7168, E = 256 236 -> 96 us): the fused kernel reads
// the whole router projection once per 16 tokens and routes its 16 tokens
// with four waves, where the routing launch has a wave per token.
//
// Mapping.  A workgroup of four waves owns 16 consecutive tokens and all
// E_pad = 16 NT experts: wave w computes the tokens against every fourth
// 16-expert MFMA tile starting at w (experts = rows of the A operand, tokens
// = columns).
// Per K tile (128 bytes of a router-weight row: 64 bf16 or 32 fp32
// elements) the E_pad weight rows are staged once in LDS (XOR-swizzled
// 16-byte chunks, rows past E read as zero) for the four waves, in two
// buffers: the next tile's rows and token fragments are loaded into
// registers while the current one is multiplied, so one barrier per tile
// remains and the load latency is hidden.  Token rows go straight into
// B-operand registers (e4m3 activations are widened to bf16 on the way,
// exactly).  The fp32 accumulators are multiplied by the token's scale (e4m3
// input), written to the logits output and to LDS, and route_token then
// routes the workgroup's tokens from there, four per wave.  (Measured on
// MI355X: 64-token workgroups read the router weights a quarter as often
// but were slower -- 187 against 158 us for the logits alone at T = 8192,
// H = 7168, E = 256 -- and route 16 tokens per wave in sequence.)
#include "prologue.hpp"
#include "tile_common.hpp"

namespace moe {

constexpr int kRtThreads = 256;
constexpr int kRtTokens = 16;  // tokens per workgroup

template <int NT>
struct RouterSmem {
  static constexpr int EP = 16 * NT;
  static constexpr int kTiles = 2 * EP * 128;            // two K tiles of the router weights
  static constexpr int kLogits = kRtTokens * EP * 4;     // the block's logits, fp32
  union {
    uint8_t w[2][EP * 128];
    float logit[kRtTokens * EP];
    uint8_t raw[kTiles > kLogits ? kTiles : kLogits];
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
  constexpr int BT = kRtTokens;
  constexpr int NTW = NT / 4;            // expert tiles per wave
  constexpr int CPT = EP * 8 / kRtThreads;  // weight chunks per thread per K tile
  constexpr int FMT = XF == 0 ? FMT_F32 : FMT_BF16;
  constexpr int XB = XF == 0 ? 4 : (XF == 1 ? 2 : 1);  // bytes per x element
  constexpr int KE = XF == 0 ? 32 : 64;                // elements per K tile
  static_assert(NT % 4 == 0 && CPT >= 1, "expert tiles must split over the waves");
  __shared__ __attribute__((aligned(16))) RouterSmem<NT> sm;

  const int nblk = (g.T + BT - 1) / BT;
  if ((int)blockIdx.x >= nblk) {
    clear_region(rp.zero_ptr, rp.zero_vec, nblk);
    return;
  }
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int g4 = lane / 16, r = lane % 16;
  const int t0 = blockIdx.x * BT;
  const int tok = t0 + r;
  const bool tok_ok = tok < g.T;
  const size_t wrow = (size_t)g.H * (XF == 0 ? 4 : 2);  // bytes per router-weight row
  const uint8_t* xrow = static_cast<const uint8_t*>(g.x) + (size_t)(tok_ok ? tok : 0) * g.H * XB;
  const uint8_t* wbase = static_cast<const uint8_t*>(g.w);

  uint4 wr[CPT];
  auto load_w = [&](int kt) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int i = tid + kRtThreads * u;
      const int row = i / 8, c = i % 8;
      wr[u] = row < g.E ? ld16(wbase + (size_t)row * wrow + (size_t)kt * 128 + 16 * c) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_w = [&](int buf) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int i = tid + kRtThreads * u;
      *reinterpret_cast<uint4*>(&sm.w[buf][swz(i / 8, i % 8)]) = wr[u];
    }
  };
  // this lane's B operand: token tok, chunks g4 and 4 + g4 of K tile kt
  auto load_x = [&](int kt, uint4& b0, uint4& b1) {
    b0 = make_uint4(0, 0, 0, 0);
    b1 = make_uint4(0, 0, 0, 0);
    if (!tok_ok) return;
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
  };

  f32x4 acc[NTW];
#pragma unroll
  for (int i = 0; i < NTW; ++i) acc[i] = f32x4{0, 0, 0, 0};
  const int nk = g.H / KE;
  uint4 b0, b1;
  load_w(0);
  load_x(0, b0, b1);
  store_w(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    uint4 n0, n1;
    if (more) {
      load_w(kt + 1);
      load_x(kt + 1, n0, n1);
    }
    const uint8_t* wt = sm.w[kt & 1];
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
      const int et = wv + 4 * i;
      const uint4 a0 = *reinterpret_cast<const uint4*>(wt + swz(16 * et + r, g4));
      const uint4 a1 = *reinterpret_cast<const uint4*>(wt + swz(16 * et + r, 4 + g4));
      mfma_tile<FMT>(acc[i], a0, a1, b0, b1, 0, 0);
    }
    if (more) {
      store_w((kt + 1) & 1);  // its buffer was last read before the previous barrier
      b0 = n0;
      b1 = n1;
    }
    __syncthreads();
  }

  // logits of token r: experts 16 et + 4 g4 + v (the weight buffers
  // are dead now: the union's logits overwrite them after the last barrier)
  const float xs = (XF == 2 && tok_ok) ? g.x_scale[tok] : 1.0f;
#pragma unroll
  for (int i = 0; i < NTW; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = 16 * (wv + 4 * i) + 4 * g4 + v;
      const float l = acc[i][v] * xs;
      sm.logit[r * EP + e] = l;
      if (tok_ok && e < g.E) g.logits[(size_t)tok * g.E + e] = l;
    }
  if (!rp.do_route) return;
  __syncthreads();
  // routing (+ gate dot, + MX quantisation of x): token i of the block by wave i % 4
  for (int i = wv; i < BT; i += kRtThreads / kWave) {
    const int t = t0 + i;
    if (t >= g.T) break;
    route_token<NPL>(rp, t, lane, sm.sel[wv], sm.val[wv], &sm.logit[i * EP]);
  }
}

// bf16 / e4m3 activations: the logits alone, as a tiled GEMM whose
// workgroups own 128 tokens x 64 experts, so each router-weight byte is read
// T / 128 times and each activation byte E / 64 times; the routing then runs
// as its own launch over the logits.
//
// Eight waves: wave w multiplies experts 32 (w & 1) .. + 31 of the tile by
// tokens 32 (w >> 1) .. + 31 on the 32x32x16 bf16 matrix cores, four K steps
// per 64-element K tile.  Within a K tile, lane half h of K step s holds
// elements 32 h + 8 s .. + 7 of its row (the A and B operands alike, so each
// step sums 16 distinct elements and the four steps all 64).  Both operands
// of a K tile are staged in LDS as bf16 rows of 128 bytes, XOR-swizzled by
// 16-byte chunk, in two buffers: every global load reads whole row segments
// (four or eight lanes per row), e4m3 activations are widened to bf16
// (exactly) on the way to LDS, and the loads run eight K tiles ahead in
// register rings.
constexpr int kRgThreads = 512;
constexpr int kRgTokens = 128;
constexpr int kRgExperts = 64;

template <int XF>
__global__ __launch_bounds__(kRgThreads) void router_gemm_kernel(RouterParams g) {
  static_assert(XF == 1 || XF == 2, "bf16 or e4m3 activations");
  constexpr int XB = XF == 1 ? 2 : 1;  // bytes per x element
  constexpr int XR = XF == 1 ? 2 : 1;  // 16-byte activation loads per thread and K tile
  constexpr int D = 8;                  // K tiles in flight (register rings)
  __shared__ __attribute__((aligned(16))) uint8_t wl[2][kRgExperts * 128];
  __shared__ __attribute__((aligned(16))) uint8_t xl[2][kRgTokens * 128];
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int eh = wv & 1, tq = wv >> 1;
  const int h = lane / 32, l32 = lane % 32;
  const int t0 = blockIdx.x * kRgTokens, e0 = blockIdx.y * kRgExperts;
  const int nk = g.H / 64;

  // Staging, as buffer offsets (tokens past T and rows past E read zeros, so
  // every load is unconditional and the compiler's load counting stays exact):
  // thread q stages router-weight chunk q % 8 of row q / 8, and activation
  // chunk(s) of token row q / 4 -- 16 elements at 16 (q % 4), as one e4m3 or
  // two bf16 loads.
  const int sr = tid / 8, sc = tid % 8;
  const __amdgpu_buffer_rsrc_t wrs = tile_rsrc(g.w, (uint32_t)((size_t)g.E * g.H * 2));
  const uint32_t woff = e0 + sr < g.E ? (uint32_t)((size_t)(e0 + sr) * g.H * 2) + 16 * sc : kTileOutOfRange;
  const int xrow = tid / 4, xq = tid % 4;
  const __amdgpu_buffer_rsrc_t xrs = tile_rsrc(g.x, (uint32_t)((size_t)g.T * g.H * XB));
  const uint32_t xoff =
      t0 + xrow < g.T ? (uint32_t)((size_t)(t0 + xrow) * g.H * XB) + 16 * xq * XB : kTileOutOfRange;

  uint4 xr[D][XR];
  uint4 wr[D];
  auto load = [&](int d, int kt) {
    kt = kt < nk ? kt : nk - 1;  // past the end: a harmless reload of the last tile
    wr[d] = tile_load16(wrs, woff, (uint32_t)kt * 128);
#pragma unroll
    for (int u = 0; u < XR; ++u) xr[d][u] = tile_load16(xrs, xoff, (uint32_t)(kt * 64 * XB + 16 * u));
  };
  auto store = [&](int buf, int d) {
    *reinterpret_cast<uint4*>(&wl[buf][swz(sr, sc)]) = wr[d];
    // the row's elements 16 xq .. + 15: bf16 chunks 2 xq and 2 xq + 1
    uint4 c0, c1;
    if constexpr (XF == 2) {
      c0 = e4m3x8_to_bf16(xr[d][0].x, xr[d][0].y);
      c1 = e4m3x8_to_bf16(xr[d][0].z, xr[d][0].w);
    } else {
      c0 = xr[d][0];
      c1 = xr[d][1];
    }
    *reinterpret_cast<uint4*>(&xl[buf][swz(xrow, 2 * xq)]) = c0;
    *reinterpret_cast<uint4*>(&xl[buf][swz(xrow, 2 * xq + 1)]) = c1;
  };

  // this lane's A row (expert) and B row (token) in the staged tiles
  const int ar = 32 * eh + l32, br = 32 * tq + l32;
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  auto compute = [&](int buf) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 a = *reinterpret_cast<const uint4*>(&wl[buf][swz(ar, 4 * h + s)]);
      const uint4 b = *reinterpret_cast<const uint4*>(&xl[buf][swz(br, 4 * h + s)]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   acc, 0, 0, 0);
    }
  };

  // K tile kt: loaded D tiles ahead into register set kt % D, staged into LDS
  // buffer kt & 1 one tile ahead (after the barrier that ends the reads of
  // that buffer); past the last tile the loads and the staging are repeats
#pragma unroll
  for (int d = 0; d < D; ++d) load(d, d);
  store(0, 0);
  __syncthreads();
  auto step = [&](int kt, int d) {
    compute(kt & 1);
    load(d, kt + D);              // its tile went to LDS one step ago
    store((kt + 1) & 1, (d + 1) % D);
    __syncthreads();
  };
  int kt = 0;
  for (; kt + D <= nk; kt += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) step(kt + d, d);
  }
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (kt + d < nk) step(kt + d, d);

  // acc[4 j + v] = expert 32 eh + 8 j + 4 h + v of the tile x token br
  const int t = t0 + br;
  if (t >= g.T) return;
  const float xs = XF == 2 ? g.x_scale[t] : 1.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = e0 + 32 * eh + 8 * j + 4 * h + v;
      if (e < g.E) g.logits[(size_t)t * g.E + e] = acc[4 * j + v] * xs;
    }
}

template <int XF>
static hipError_t launch_router_xf(const RouterParams& g, const RouteParams& rp, hipStream_t s) {
  if constexpr (XF != 0) {
    // (32-bit buffer offsets address the activations and the router weights;
    // larger operands take the fused kernel)
    if ((size_t)g.T * g.H * (XF == 1 ? 2 : 1) < 0x7FFFFFFFu && (size_t)g.E * g.H * 2 < 0x7FFFFFFFu) {
      const dim3 grid((unsigned)((g.T + kRgTokens - 1) / kRgTokens), (unsigned)((g.E + kRgExperts - 1) / kRgExperts));
      hipLaunchKernelGGL(router_gemm_kernel<XF>, grid, dim3(kRgThreads), 0, s, g);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess || !rp.do_route) return e;
      return launch_route(rp, s);
    }
  }
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
