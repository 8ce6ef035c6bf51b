// Grouped GEMM for 16-row sorted blocks, one wave per workgroup (gfx950).
//
// Decode-sized batches (a few tokens per expert) make both stages stream the
// expert weights once and do almost no arithmetic per byte (vLLM PR 65207's
// decode profile is this regime).  A workgroup here is a single wave that owns
// NCG consecutive 16-column groups of one block: stage 1 owns 2 groups = 32 h
// columns (one MX-32 block) and streams their gate and up rows, with bias and act-mul
// in registers; stage 2 owns 4 groups = one 64-column output tile and streams
// those 64 rows of W2.  The weight rows are the MFMA M dimension and the
// block's (at most 16) tokens the N dimension.  The K tile is the outer loop:
// each 128-byte activation tile is read once and feeds all NCG x (gate, up)
// weight tiles.  Weights are in the tiled layout, so the wave's 16 rows of one
// K tile are two contiguous 1024-byte non-temporal loads, which go from HBM
// straight into MFMA operand registers, D K-tiles ahead; the activation rows come from L2
// through a buffer descriptor (a padding row reads past the end of the
// buffer, i.e. zeros, with no branch and no fetch).  There is no LDS and no
// barrier: the many small independent workgroups hide each other's start-up
// latency.
//
// Stage 2 keeps the deterministic pair-row reduction: each wave stores the 64
// columns of its weighted pair rows, then counts one arrival per token on the
// (token, 64-column tile) counter; the last of the k_total arrivals sums the
// addend and the token's rows in slot order and rounds once into out.
//
// K order as in the other GEMM kernels: lane group g feeds chunks g and 4+g of
// each 128-byte K tile (the gfx950 16x16x128 f8f6f4 operand order); MX scales
// come from lane r + 16b for K block b.
#include "gemm_common.hpp"
#include "prologue.hpp"

namespace moe {

constexpr uint32_t kWvOutOfRange = 0x80000000u;  // buffer offset that reads as zero
// prefetch depth caps (K tiles): stage 1 already has 2 groups x gate/up = 4
// weight tiles per K tile in flight, stage 2 4 groups x W2
constexpr int kWaveMaxDepth1 = 1, kWaveMaxDepth2 = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t wv_rsrc(const void* base, uint32_t bytes) {
  // raw (untyped) buffer, dword 3 = 0x00020000 on gfx9-family parts
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 wv_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

// Whether expert e < E <= 64 (E a multiple of 4) is among token t's top-k
// under the routing's own rule (route_token with softmax scores and no
// groups): fewer than topk experts have a larger selection key (logit bits,
// then the lower index).
__device__ __forceinline__ bool expert_selected(const RouteParams& r, int t, int e) {
  const float* lr = r.logits + (size_t)t * r.E;
  const uint64_t ke = ((uint64_t)float_key(lr[e]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
  int above = 0;
#pragma unroll 4
  for (int f = 0; f < r.E; f += 4) {
    const float4 v = *reinterpret_cast<const float4*>(lr + f);
    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      above += (((uint64_t)float_key(vv[q]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(f + q))) > ke;
  }
  return above < r.topk;
}

// The routing workgroups of a fused stage-1 launch (E <= 64): workgroup
// w < T routes token w (ids, weights, gamma), the rest clear the stage-2
// counters.
__device__ __forceinline__ void fused_route_wave(const GemmParams& p, int first, int lane) {
  __shared__ float sel[kWave], val[kWave];
  const int w = (int)blockIdx.x - first;
  if (w >= p.route.T) {
    clear_region(p.route.zero_ptr, p.route.zero_vec, first + p.route.T);
    return;
  }
  route_token<1>(p.route, w, lane, sel, val, p.route.logits + (size_t)w * p.route.E);
}

template <int FMT, int STAGE, int D>
__global__ __launch_bounds__(64) void gemm_wave_kernel(GemmParams p) {
  constexpr int esz = FmtInfo<FMT>::esz;
  constexpr int BM = 16;
  constexpr int NW = (STAGE == 1) ? 2 : 1;    // weight rows per lane and group: gate + up, or W2
  constexpr int NCG = (STAGE == 1) ? 2 : 4;   // 16-column groups per wave (a multiple of 4 in stage 2)
  constexpr int CW = 16 * NCG;                // columns per wave

  const int lane = threadIdx.x;
  const int g = lane / 16, l16 = lane % 16;
  const int width_max = (STAGE == 1) ? (p.dense ? p.I_s : p.I) : p.H;
  const int ncw = width_max / CW;
  if (STAGE == 1 && p.route_fused && (int)blockIdx.x >= p.max_blocks * ncw) {
    fused_route_wave(p, p.max_blocks * ncw, lane);
    return;
  }
  const int b = blockIdx.x / ncw, c0 = (blockIdx.x % ncw) * CW;

  // block expert and this lane's token (sorted blocks: fetched together)
  const int slot_l = b * BM + l16;
  int e, sb = 0, pair_l = -1, tok_l = -1;
  if (p.dense) {
    if (b * BM >= p.T) return;
    e = -1;
    tok_l = slot_l < p.T ? slot_l : -1;
  } else if (p.self_sort) {
    // block b = sb * E' + e holds expert e's pairs of rank 16 sb .. 16 sb + 15
    const int Et = p.E + p.n_pseudo;
    e = b % Et;
    sb = b / Et;
  } else {
    e = p.block_expert[b];  // -1 past the last block
    const int pr = p.sorted[slot_l];
    if (e < 0) return;
    pair_l = pr < p.T * p.k_total ? pr : -1;
    tok_l = pair_l >= 0 ? pair_l / p.k_total : -1;
  }
  const ExpertView ev = resolve_expert<FMT, STAGE>(p, e);
  if (STAGE == 1 && c0 >= ev.width) return;
  const int kbytes = (STAGE == 1) ? p.H * esz : ev.width * esz;  // a multiple of 128
  const int nk = kbytes / 128;                                    // a multiple of D (launch)

  // ---- weights: lane row r = l16 of each group (clamped; rows past a narrow
  // chunk are never stored) ----
  const uint8_t* wbase[NW];
  const uint8_t* sbase[NW];
  wbase[0] = ev.wa + lane * 16;
  sbase[0] = ev.sa + lane;
  if constexpr (NW == 2) {
    wbase[1] = ev.wb + lane * 16;
    sbase[1] = ev.sb + lane;
  }
  // row block of group cgi (rows past a narrow chunk read row block 0 and are
  // never stored)
  auto group_rb = [&](int cgi) {
    const int r0 = c0 + cgi * 16;
    return (STAGE == 1 && r0 >= ev.width) ? 0 : r0 / 16;
  };
  // K tile outermost: one activation tile feeds every group of the wave;
  // D K tiles of all NCG * NW weight tiles in flight
  uint4 wb[D][NCG][NW][2];
  int wsc[D][NCG][NW];
  auto load_w = [&](int d, int kt) {
    kt = kt < nk ? kt : nk - 1;  // unconditional loads: no branch forces a full wait
#pragma unroll
    for (int cgi = 0; cgi < NCG; ++cgi) {
      const int rb = group_rb(cgi);
      const size_t off = tile_off(ev, rb, kt);
#pragma unroll
      for (int m = 0; m < NW; ++m) {
        wb[d][cgi][m][0] = ld16_stream(wbase[m] + off);
        // MXFP4: one 1 KiB half per tile (lane (g, r): 32 e2m1 values)
        wb[d][cgi][m][1] = FMT == FMT_MX4 ? make_uint4(0, 0, 0, 0) : ld16_stream(wbase[m] + off + 1024);
        if constexpr (fmt_mx(FMT)) wsc[d][cgi][m] = sbase[m][scale_tile_off(ev, rb, kt)];
        else wsc[d][cgi][m] = 127;
      }
    }
  };
  // Self-sorted blocks: the first block of an expert is almost always
  // occupied, so its weights start streaming before the token scan; later
  // blocks scan first (most of them are empty and leave).
  const bool early_w = p.self_sort && sb == 0;
  if (early_w) {
#pragma unroll
    for (int d = 0; d < D; ++d) load_w(d, d);
  }
  if (!p.dense && p.self_sort) {
    // the block's pairs: ranks 16 sb .. 16 sb + 15 of expert e among the
    // T * k_total ids in pair order (ascending pair index, as the sort orders them)
    __shared__ int s_pair[BM];
    const int P = p.T * p.k_total;
    int cum = 0;
    if (STAGE == 1 && p.route_fused) {
      // lane t: token t (T <= 64) selects expert e; pseudo experts take every
      // token.  Ranks in token order are ranks in pair order; stage 1 needs
      // only the token of a row (pair index with slot 0).
      const bool hit = lane < p.T && (e >= p.E || expert_selected(p.route, lane, e));
      const uint64_t m = __ballot(hit);
      const int r = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) - BM * sb;
      if (hit && r >= 0 && r < BM) s_pair[r] = lane * p.k_total;
      cum = (int)__popcll(m);
    }
    for (int base = 0; base < P && !(STAGE == 1 && p.route_fused); base += 4 * kWave) {
      int idv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = base + u * kWave + lane;
        idv[u] = i < P ? p.ids[i] : -1;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool hit = idv[u] == e;
        const uint64_t m = __ballot(hit);
        const int r = cum - BM * sb +
                      (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (hit && r >= 0 && r < BM) s_pair[r] = base + u * kWave + lane;
        cum += (int)__popcll(m);
      }
    }
    const int rows = cum - BM * sb;
    if (rows <= 0) return;
    wave_lds_sync();
    pair_l = l16 < rows ? s_pair[l16] : -1;
    tok_l = pair_l >= 0 ? pair_l / p.k_total : -1;
  }
  // ---- activations: this lane's token row through a buffer descriptor ----
  const bool xok = tok_l >= 0;
  const float wgt_pair = (STAGE == 2 && pair_l >= 0) ? p.pair_w[pair_l] : 0.f;  // ACCUMULATE weight
  __amdgpu_buffer_rsrc_t xr, xsr;
  uint32_t xoff, xsoff = 0;
  if constexpr (STAGE == 1) {
    xr = wv_rsrc(p.x, (uint32_t)((size_t)p.T * p.H * esz));
    xoff = xok ? (uint32_t)((size_t)tok_l * p.H * esz) + g * 16 : kWvOutOfRange;
    if constexpr (fmt_mx(FMT)) {
      xsr = wv_rsrc(p.x_s, (uint32_t)((size_t)p.T * (p.H / 32)));
      xsoff = xok ? (uint32_t)(tok_l * (p.H / 32)) + g : kWvOutOfRange;
    }
  } else {
    const size_t rows = (size_t)p.max_blocks * BM;
    xr = wv_rsrc(p.h, (uint32_t)(rows * h_row_bytes<FMT>(p)));
    xoff = xok ? (uint32_t)((size_t)slot_l * h_row_bytes<FMT>(p)) + g * 16 : kWvOutOfRange;
    if constexpr (fmt_mx(FMT)) {
      xsr = wv_rsrc(p.h_s, (uint32_t)(rows * (p.ld_h / 32)));
      xsoff = xok ? (uint32_t)(slot_l * (p.ld_h / 32)) + g : kWvOutOfRange;
    }
  }
  float rs = 1.0f;  // A8W8: stage 1 the token's x scale, stage 2 the row scale amax / 448
  if constexpr (FMT == FMT_A8W8) {
    if (STAGE == 1) {
      rs = xok ? static_cast<const float*>(p.x_s)[tok_l] : 0.f;
    } else {
      const float amax = xok ? static_cast<const float*>(p.h_s)[slot_l] : 0.f;
      if (amax > 0.f) rs = __fdiv_rn(amax, 448.0f);
    }
  }

  uint4 xb[D][2];
  int xsc[D];
  auto load_x = [&](int d, int kt) {
    const uint32_t o = xoff + (uint32_t)kt * 128;
    xb[d][0] = wv_load16(xr, o);
    xb[d][1] = wv_load16(xr, o + 64);
    if constexpr (fmt_mx(FMT))
      xsc[d] = (int)__builtin_amdgcn_raw_buffer_load_b8(xsr, (int)(xsoff + (uint32_t)kt * 4), 0, 0);
    else
      xsc[d] = 127;
  };

  // lane results: rows 4g..4g+3 of each group (columns c0 + 16 cgi + 4g + j),
  // token l16
  const float sc = rs * ev.wscale;
  float res[NCG][4];
  auto load = [&](int d, int kt) {
    load_w(d, kt);
    load_x(d, kt < nk ? kt : nk - 1);
  };
#pragma unroll
  for (int d = 0; d < D; ++d) {
    if (!early_w) load_w(d, d);
    load_x(d, d);
  }
  f32x4 acc[NCG][NW];
#pragma unroll
  for (int cgi = 0; cgi < NCG; ++cgi)
#pragma unroll
    for (int m = 0; m < NW; ++m) acc[cgi][m] = f32x4{0, 0, 0, 0};
  for (int kt0 = 0; kt0 < nk; kt0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
#pragma unroll
      for (int cgi = 0; cgi < NCG; ++cgi)
#pragma unroll
        for (int m = 0; m < NW; ++m)
          mfma_tile<FMT>(acc[cgi][m], wb[d][cgi][m][0], wb[d][cgi][m][1], xb[d][0], xb[d][1], wsc[d][cgi][m],
                         xsc[d]);
      load(d, kt0 + d + D);
    }
  }
#pragma unroll
  for (int cgi = 0; cgi < NCG; ++cgi)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = c0 + 16 * cgi + 4 * g + j;
      res[cgi][j] = (STAGE == 1) ? act_mul(acc[cgi][0][j] * sc + bias_at(ev.bg, col, ev.width),
                                           acc[cgi][NW - 1][j] * sc + bias_at(ev.bu, col, ev.width), p.act)
                                 : acc[cgi][0][j] * sc + bias_at(ev.b2, col);
    }

  if constexpr (STAGE == 1) {
    const size_t slot = (size_t)slot_l;
    if constexpr (fmt_mx(FMT)) {
      // one MX-32 block per token: the wave's 32 columns
      float v[8], amax = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        v[q] = bf16_to_f32(f32_to_bf16(res[q / 4][q % 4]));
        amax = fmaxf(amax, fabsf(v[q]));
      }
      amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
      amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
      const int eb = (int)((__float_as_uint(amax) >> 23) & 0xFF);
      int X = (eb == 0) ? -127 : (eb - 127 - 8);
      X = X < -127 ? -127 : (X > 127 ? 127 : X);
      const float mul = __builtin_ldexpf(1.0f, -X);
      if (xok && c0 < ev.width) {
        uint8_t* dst = p.h + slot * p.ld_h + c0 + 4 * g;
        *reinterpret_cast<uint32_t*>(dst) = pack4_e4m3(v[0] * mul, v[1] * mul, v[2] * mul, v[3] * mul);
        *reinterpret_cast<uint32_t*>(dst + 16) = pack4_e4m3(v[4] * mul, v[5] * mul, v[6] * mul, v[7] * mul);
        if (g == 0) static_cast<uint8_t*>(p.h_s)[slot * (p.ld_h / 32) + c0 / 32] = (uint8_t)(X + 127);
      }
    } else {
      float amax = 0.f;
#pragma unroll
      for (int cgi = 0; cgi < NCG; ++cgi) {
        const int col = c0 + cgi * 16 + 4 * g;
        const bool ok = xok && col < ev.width;
        if constexpr (FMT == FMT_F32) {
          if (ok) *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.h) + slot * p.ld_h + col) =
              make_float4(res[cgi][0], res[cgi][1], res[cgi][2], res[cgi][3]);
        } else {
          uint32_t bits[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            bits[j] = f32_to_bf16(res[cgi][j]);
            if (ok) amax = fmaxf(amax, fabsf(bf16_to_f32(bits[j])));
          }
          if (ok) *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.h) + slot * p.ld_h + col) =
              make_uint2(bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16));
        }
      }
      if constexpr (FMT == FMT_A8W8) {
        // row amax of the bf16-rounded values over the wave's columns
        amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
        amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
        if (g == 0 && xok) atomicMax(reinterpret_cast<unsigned int*>(p.h_s) + slot, __float_as_uint(amax));
      }
    }
  } else {
    if (p.mode == 0) {  // STORE: the dense shared expert's gamma * S(x) as the addend
      if (xok) {
        const float gm = p.gamma ? p.gamma[tok_l] : 1.0f;
#pragma unroll
        for (int cgi = 0; cgi < NCG; ++cgi)
          *reinterpret_cast<float4*>(p.acc + (size_t)tok_l * p.H + c0 + cgi * 16 + 4 * g) =
              make_float4(gm * res[cgi][0], gm * res[cgi][1], gm * res[cgi][2], gm * res[cgi][3]);
      }
      return;
    }
    // ACCUMULATE: this pair's CW columns with device-coherent stores
    if (pair_l >= 0) {
      const float wgt = wgt_pair;
      uint64_t* dst = reinterpret_cast<uint64_t*>(p.pair_out + (size_t)pair_l * p.H + c0 + 4 * g);
#pragma unroll
      for (int cgi = 0; cgi < NCG; ++cgi)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint64_t v = (uint64_t)__float_as_uint(wgt * res[cgi][2 * h]) |
                             ((uint64_t)__float_as_uint(wgt * res[cgi][2 * h + 1]) << 32);
          __hip_atomic_store(dst + cgi * 8 + h, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // count the arrivals (one per 64-column reduction tile) once the stores
    // are acknowledged (no agent-scope fence: on multi-XCD parts it would
    // write back and invalidate the whole L2)
    __builtin_amdgcn_s_waitcnt(0);
    constexpr int NT = NCG / 4;
    const int n_tiles = p.H / 64;
    const int t0 = c0 / 64;
    int old[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      old[tt] = -1;
      if (g == 0 && pair_l >= 0) old[tt] = atomicAdd(p.counters + (size_t)tok_l * n_tiles + t0 + tt, 1);
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      // broadcast to the token's 4 lanes
      const int done = __shfl(old[tt], l16, kWave) == p.expected - 1;
      if (done) last_arrival_sum16(p, tok_l, 64 * (t0 + tt) + 16 * g);
    }
  }
}

// Prefetch depth (2 or 1, within the stage's cap) dividing the K-tile count
// of every expert the launch can meet (routed width, shared width, last
// pseudo chunk).
static int wave_depth(const GemmParams& p, int stage, int fmt) {
  const int esz = fmt == FMT_F32 ? 4 : (fmt == FMT_BF16 ? 2 : 1);
  int g = 0;
  auto gcd = [](int a, int b) { while (b) { int t = a % b; a = b; b = t; } return a; };
  if (stage == 1) {
    g = p.H * esz / 128;
  } else if (p.dense) {
    g = p.I_s * esz / 128;
  } else {
    g = p.I * esz / 128;
    if (p.n_pseudo > 0) g = gcd(g, (p.I_s - (p.n_pseudo - 1) * p.I) * esz / 128);
  }
  const int cap = stage == 1 ? kWaveMaxDepth1 : kWaveMaxDepth2;
  return (g % 2 == 0 && cap >= 2) ? 2 : 1;
}

// (64 columns per stage-2 wave measured best for decode batches: 32 or 128
// columns per wave stream slower on MI355X)
template <int FMT, int STAGE>
static hipError_t launch_wv(const GemmParams& p, int depth, hipStream_t s) {
  constexpr int CW = (STAGE == 1) ? 32 : 64;
  const int width_max = (STAGE == 1) ? (p.dense ? p.I_s : p.I) : p.H;
  const long long route_wgs = (STAGE == 1 && p.route_fused) ? p.route.T + clear_blocks(p.route.zero_vec, 64) : 0;
  const dim3 grid((unsigned)(p.max_blocks * (width_max / CW) + route_wgs));
  if (depth >= 2) return launch_gemm_kernel(gemm_wave_kernel<FMT, STAGE, 2>, grid, dim3(64), s, p);
  return launch_gemm_kernel(gemm_wave_kernel<FMT, STAGE, 1>, grid, dim3(64), s, p);
}

// Activation buffers are addressed with 32-bit buffer offsets; widths must
// split into whole waves (32 columns in stage 1, 64 in stage 2).
bool wave_kernel_fits(const GemmParams& p, int stage, int fmt) {
  const size_t esz = fmt == FMT_F32 ? 4 : (fmt == FMT_BF16 ? 2 : 1);
  const size_t hsz = fmt == FMT_A8W8 ? 2 : esz;
  const size_t bytes = stage == 1 ? (size_t)p.T * p.H * esz : (size_t)p.max_blocks * 16 * p.ld_h * hsz;
  if (bytes >= 0x7FFFFFFFu) return false;
  if (stage == 1) return p.I % 32 == 0 && p.I_s % 32 == 0;
  return p.H % 64 == 0;
}

hipError_t launch_gemm_wave(const GemmParams& p, int stage, int fmt, hipStream_t s) {
  const int depth = wave_depth(p, stage, fmt);
  if (stage == 1) {
    switch (fmt) {
      case FMT_F32: return launch_wv<FMT_F32, 1>(p, depth, s);
      case FMT_BF16: return launch_wv<FMT_BF16, 1>(p, depth, s);
      case FMT_MX: return launch_wv<FMT_MX, 1>(p, depth, s);
      case FMT_MX4: return launch_wv<FMT_MX4, 1>(p, depth, s);
      case FMT_A8W8: return launch_wv<FMT_A8W8, 1>(p, depth, s);
    }
  } else {
    switch (fmt) {
      case FMT_F32: return launch_wv<FMT_F32, 2>(p, depth, s);
      case FMT_BF16: return launch_wv<FMT_BF16, 2>(p, depth, s);
      case FMT_MX: return launch_wv<FMT_MX, 2>(p, depth, s);
      case FMT_MX4: return launch_wv<FMT_MX4, 2>(p, depth, s);
      case FMT_A8W8: return launch_wv<FMT_A8W8, 2>(p, depth, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
