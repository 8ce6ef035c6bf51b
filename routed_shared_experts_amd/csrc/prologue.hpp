// Device bodies of the layer prologue (routing and sort kernels):
//  * route_token: one wave routes one token -- the shared-expert gate
//    gamma_t = sigmoid(x_t . g) as a K-length dot product with the sigmoid
//    folded in (vLLM PR 56789, "Commits": the 1x1xK GEMM becomes a dot
//    product; fp32 accumulation), the in-layer MX-32 quantisation of bf16 x
//    (OCP MX v1.0 rule; AITER PR 6106, "Technical Details": 32-element K
//    blocks), and top-k / biased grouped top-k routing with the routed scaling
//    factor folded into the weights (vLLM PR 65207, "Purpose", commit 1), with
//    deterministic tie-breaks (equal scores -> lower index).  Selection keys
//    are (order-preserving score bits << 32 | ~index), so one 64-bit wave max
//    per round (two DPP reductions) picks the winner and applies the tie rule.
//  * sort_wg: one 1024-thread workgroup sorts the (token, slot) pairs by
//    expert with per-expert padding (vLLM PR 65207, "Purpose", commit 2):
//      1. histogram of expert ids (LDS atomics; counts are order-independent);
//      2. exclusive scan of the counts padded to block_m, block -> expert map;
//      3. a stable scatter: pairs are taken in index order, 1024 per round;
//         the rank of a pair among equal experts of its wave comes from a
//         ballot match on the expert id bits, and the wave's base from the
//         per-wave counts of the waves before it, so the output order is
//         ascending pair index inside each expert independently of scheduling.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kMaxE = 512;  // routed experts a routing wave handles
constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / kWave;
constexpr int kMaxSortExperts = 576;

// gamma_t = sigmoid(x_t . g) by one wave: every lane issues its row loads four
// 16-byte chunks at a time before it accumulates them.
__device__ __forceinline__ float gate_dot_wave(const RouteParams& p, int t, int lane) {
  float sum = 0.f;
  if (p.x_f32) {
    const float4* xr = reinterpret_cast<const float4*>(static_cast<const float*>(p.x) + (size_t)t * p.H);
    const float4* gr = reinterpret_cast<const float4*>(p.gate_w);
    const int n = p.H / 4;
    for (int base = 0; base < n; base += 4 * kWave) {
      float4 a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = base + u * kWave + lane;
        a[u] = c < n ? xr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        b[u] = c < n ? gr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) sum += a[u].x * b[u].x + a[u].y * b[u].y + a[u].z * b[u].z + a[u].w * b[u].w;
    }
  } else {
    const uint4* xr = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.x) + (size_t)t * p.H);
    const uint4* gr = reinterpret_cast<const uint4*>(p.gate_w);
    const int n = p.H / 8;
    for (int base = 0; base < n; base += 4 * kWave) {
      uint4 a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = base + u * kWave + lane;
        a[u] = c < n ? xr[c] : make_uint4(0, 0, 0, 0);
        b[u] = c < n ? gr[c] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t av[4] = {a[u].x, a[u].y, a[u].z, a[u].w}, bv[4] = {b[u].x, b[u].y, b[u].z, b[u].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          sum += bf16_to_f32(av[q] & 0xFFFFu) * bf16_to_f32(bv[q] & 0xFFFFu);
          sum += bf16_to_f32(av[q] >> 16) * bf16_to_f32(bv[q] >> 16);
        }
      }
    }
  }
  return spec_sigmoid(dpp_wave_sum(sum));
}

// MX-32 quantisation of one bf16 row: 4 lanes per 32-element block.
__device__ __forceinline__ void mx_quant_row(const uint16_t* xr, int H, uint8_t* qr, uint8_t* sr, int lane) {
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

// Token t by one wave.  sel / val: this wave's LDS scratch of at least E
// floats; lrow: the token's E router logits (global memory or LDS).  NPL =
// experts per lane (E <= 64 * NPL).
template <int NPL>
__device__ __forceinline__ void route_token(const RouteParams& p, int t, int lane, float* sel, float* val,
                                            const float* lrow) {
  const int E = p.E;
  // the logits first: their loads overlap the gate dot
  float lg[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + i * kWave;
    lg[i] = (p.do_route && e < E) ? lrow[e] : 0.f;
  }

  float gamma = 1.0f;
  if (p.gate_w != nullptr) {
    gamma = gate_dot_wave(p, t, lane);
    if (lane == 0 && p.gamma_out != nullptr) p.gamma_out[t] = gamma;
  } else if (p.gamma_in != nullptr) {
    gamma = p.gamma_in[t];
  }
  if (p.xq != nullptr) {
    mx_quant_row(static_cast<const uint16_t*>(p.x) + (size_t)t * p.H, p.H, p.xq + (size_t)t * p.H,
                 p.xs + (size_t)t * (p.H / 32), lane);
  }
  if (!p.do_route) return;

  float lmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + i * kWave;
    if (e < E) {
      const float l = lg[i];
      lmax = fmaxf(lmax, l);
      if (p.score == 0) {
        sel[e] = l;
        val[e] = l;
      } else {
        const float sg = spec_sigmoid(l);
        const float b = p.bias ? p.bias[e] : 0.0f;
        sel[e] = __fadd_rn(sg, b);
        val[e] = sg;
      }
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
  int id = -1;
  if (lane < p.topk) {
    id = my_id;
    p.w[(size_t)t * kt + lane] = wgt;
  } else if (lane < kt) {
    id = E + (lane - p.topk);
    p.w[(size_t)t * kt + lane] = gamma;
  }
  if (lane < kt) p.ids[(size_t)t * kt + lane] = id;
}

struct SortSmem {
  int count[kMaxSortExperts];
  int off[kMaxSortExperts + 1];
  int run[kMaxSortExperts];
  int wave[kSortWaves][kMaxSortExperts];
};

// The whole sort by one workgroup of kSortThreads threads; ids may live in
// global memory or LDS.
__device__ __forceinline__ void sort_wg(const SortParams& p, const int32_t* ids, SortSmem& s) {
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wv = tid / kWave;
  const int nE = p.n_experts;
  const int BM = p.block_m;

  for (int e = tid; e < nE; e += kSortThreads) {
    s.count[e] = 0;
    s.run[e] = 0;
  }
  for (int i = tid; i < kSortWaves * kMaxSortExperts; i += kSortThreads) (&s.wave[0][0])[i] = 0;
  __syncthreads();
  for (int i = tid; i < p.P; i += kSortThreads) atomicAdd(&s.count[ids[i]], 1);
  __syncthreads();

  // padded exclusive scan by wave 0, 64 experts at a time
  if (wv == 0) {
    int carry = 0;
    for (int base = 0; base < nE; base += kWave) {
      int e = base + lane;
      int c = e < nE ? s.count[e] : 0;
      int pc = (c + BM - 1) / BM * BM;
      int incl = pc;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        int y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
      }
      if (e < nE) s.off[e] = carry + incl - pc;
      carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) s.off[nE] = carry;
  }
  __syncthreads();
  const int total = s.off[nE];
  const int nblk = total / BM;
  for (int e = tid; e < nE; e += kSortThreads) {
    p.counts[e] = s.count[e];
    p.offsets[e] = s.off[e];
  }
  if (tid == 0) {
    p.offsets[nE] = total;
    *p.num_blocks = nblk;
  }
  // block -> expert (upper bound search over the padded offsets)
  const int max_blocks = p.capacity / BM;
  for (int b = tid; b < max_blocks; b += kSortThreads) {
    int be = -1;
    if (b < nblk) {
      int row = b * BM, lo = 0, hi = nE - 1;
      while (lo < hi) {  // last e with off[e] <= row
        int mid = (lo + hi + 1) / 2;
        if (s.off[mid] <= row) lo = mid; else hi = mid - 1;
      }
      be = lo;
    }
    p.block_expert[b] = be;
  }
  // sentinels: padding slots of each expert, and the unused tail
  for (int e = tid; e < nE; e += kSortThreads)
    for (int i = s.off[e] + s.count[e]; i < s.off[e + 1]; ++i) p.sorted[i] = p.P;
  for (int i = total + tid; i < p.capacity; i += kSortThreads) p.sorted[i] = p.P;

  // stable scatter
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < p.P; base += kSortThreads) {
    const int pi = base + tid;
    const bool valid = pi < p.P;
    const int e = valid ? ids[pi] : 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 10; ++bit) {
      const bool b = (e >> bit) & 1;
      const uint64_t bal = __ballot(b);
      peers &= b ? bal : ~bal;
    }
    const int rank = __popcll(peers & lt_mask);
    const int leader = valid ? (__ffsll((unsigned long long)peers) - 1) : -1;
    if (valid && lane == leader) s.wave[wv][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int pos = s.off[e] + s.run[e] + rank;
      for (int w = 0; w < wv; ++w) pos += s.wave[w][e];
      p.sorted[pos] = pi;
    }
    __syncthreads();
    if (valid && lane == leader) {
      atomicAdd(&s.run[e], s.wave[wv][e]);
      s.wave[wv][e] = 0;
    }
    __syncthreads();
  }
}

// 16-byte clearing of [ptr, ptr + n) by the workgroups from first_block on.
__device__ __forceinline__ void clear_region(uint4* ptr, long long n, int first_block) {
  const long long stride = (long long)(gridDim.x - first_block) * blockDim.x;
  for (long long i = (long long)(blockIdx.x - first_block) * blockDim.x + threadIdx.x; i < n; i += stride)
    ptr[i] = make_uint4(0, 0, 0, 0);
}

// Workgroups that clear a region of n 16-byte vectors next to a launch's own
// (threads per workgroup: nt).
inline long long clear_blocks(long long n, int nt) {
  if (n <= 0) return 0;
  const long long b = (n + nt * 4LL - 1) / (nt * 4LL);
  return b > 1024 ? 1024 : b;
}

}  // namespace moe
