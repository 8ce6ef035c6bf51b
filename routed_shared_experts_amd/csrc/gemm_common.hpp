// Pieces shared by the grouped-GEMM kernels (gemm.hip: LDS-staged tiles, the
// general fallback; gemm_wave.hip: 16-row blocks, one wave per workgroup with
// weights streamed straight into MFMA operand registers; gemm_tile.hip: 32-128
// row blocks, weights in registers and token rows staged through LDS): operand
// formats, the MFMA wrapper, the expert/pseudo-expert resolution, the
// per-block row setup, the epilogues and the last-arrival reduction.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// esz: bytes per activation (and stage-2 input) element in the MFMA K order;
// wtile: bytes of one weight tile (16 rows x one K tile: 128 bytes of
// activation per row; MXFP4 weights pack that K range in 64 bytes)
template <int FMT>
struct FmtInfo;
template <>
struct FmtInfo<FMT_F32> { static constexpr int esz = 4, wtile = 2048; static constexpr bool fp8 = false; };
template <>
struct FmtInfo<FMT_BF16> { static constexpr int esz = 2, wtile = 2048; static constexpr bool fp8 = false; };
template <>
struct FmtInfo<FMT_MX> { static constexpr int esz = 1, wtile = 2048; static constexpr bool fp8 = true; };
template <>
struct FmtInfo<FMT_A8W8> { static constexpr int esz = 1, wtile = 2048; static constexpr bool fp8 = true; };
template <>
struct FmtInfo<FMT_MX4> { static constexpr int esz = 1, wtile = 1024; static constexpr bool fp8 = true; };

// Bytes of a weight matrix region of `rows` rows with K elements each.
template <int FMT>
__device__ __forceinline__ size_t wbytes(size_t rows, size_t K) {
  return rows * K * FmtInfo<FMT>::esz * FmtInfo<FMT>::wtile / 2048;
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
// Non-temporal load for data read exactly once (decode weight streams): it
// does not displace reusable lines from the caches.
__device__ __forceinline__ uint4 ld16_stream(const uint8_t* p) {
  const i32x4 v = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

template <int FMT>
__device__ __forceinline__ void mfma_tile(f32x4& acc, const uint4& a0, const uint4& a1, const uint4& b0,
                                          const uint4& b1, int sa, int sb) {
  if constexpr (FMT == FMT_F32) {
    const float* fa0 = reinterpret_cast<const float*>(&a0);
    const float* fa1 = reinterpret_cast<const float*>(&a1);
    const float* fb0 = reinterpret_cast<const float*>(&b0);
    const float* fb1 = reinterpret_cast<const float*>(&b1);
#pragma unroll
    for (int v = 0; v < 4; ++v) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa0[v], fb0[v], acc, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa1[v], fb1[v], acc, 0, 0, 0);
  } else if constexpr (FMT == FMT_BF16) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0), __builtin_bit_cast(bf16x8, b0),
                                                  acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1), __builtin_bit_cast(bf16x8, b1),
                                                  acc, 0, 0, 0);
  } else if constexpr (FMT == FMT_MX4) {
    // A: e2m1 weights, lane (g, r) holding K 32 g .. 32 g + 31 of row r in a0
    // (even elements in low nibbles; a1 unused); B: e4m3 as for FMT_MX
    i32x8 A = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, 0, 0, 0, 0};
    i32x8 B = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 4, 0, 0, sa, 0, sb);
  } else {
    i32x8 A = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    i32x8 B = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 0, 0, 0, sa, 0, sb);
  }
}

// Per-block problem description resolved from the expert index.  Weights
// and MX scales are in the tiled layout (16-row tiles of one K tile each,
// 2048 bytes, or 1024 for MXFP4 weights; row block major; 64-byte scale
// tiles), so a view is the base of its row block 0 plus the tile count of a
// full matrix row, a first K tile and the tile size.
struct ExpertView {
  const uint8_t* wa;   // stage 1: gate rows; stage 2: W2 rows
  const uint8_t* wb;   // stage 1: up rows
  const uint8_t* sa;   // MX scales of wa rows
  const uint8_t* sb;   // MX scales of wb rows
  int nkt;             // K tiles per row of the underlying matrix
  int kt0;             // first K tile of this view (shared W2 pseudo-expert chunk)
  int width;           // stage 1: valid h columns; stage 2: valid K (h columns)
  int tb;              // bytes of one weight tile
  float wscale;        // A8W8 per-expert scale
  const float* bg;     // stage 1: bias of the view's gate column 0 (or NULL)
  const float* bu;     // stage 1: bias of the view's up column 0 (or NULL)
  const float* b2;     // stage 2: bias of output column 0 (or NULL; pseudo-expert 0 only)
};

// Byte offset of tile (row block rb, K tile kt) of a view, and of its scales.
__device__ __forceinline__ size_t tile_off(const ExpertView& v, int rb, int kt) {
  return ((size_t)rb * v.nkt + v.kt0 + kt) * v.tb;
}
__device__ __forceinline__ size_t scale_tile_off(const ExpertView& v, int rb, int kt) {
  return ((size_t)rb * v.nkt + v.kt0 + kt) * 64;
}

template <int FMT, int STAGE>
__device__ __forceinline__ ExpertView resolve_expert(const GemmParams& p, int e) {
  constexpr int esz = FmtInfo<FMT>::esz;
  ExpertView v{};
  v.wscale = 1.0f;
  v.tb = FmtInfo<FMT>::wtile;
  const int H = p.H, I = p.I, Is = p.I_s;
  if (e >= 0 && e < p.E) {
    if (STAGE == 1) {
      v.wa = p.w13 + wbytes<FMT>((size_t)e * 2 * I, H);
      v.wb = v.wa + wbytes<FMT>(I, H);
      v.nkt = H * esz / 128;
      v.width = I;
      if (p.b13) {
        v.bg = p.b13 + (size_t)e * 2 * I;
        v.bu = v.bg + I;
      }
      if (fmt_mx(FMT)) {
        v.sa = static_cast<const uint8_t*>(p.w13_s) + (size_t)e * 2 * I * (H / 32);
        v.sb = v.sa + (size_t)I * (H / 32);
      }
      if (FMT == FMT_A8W8) v.wscale = static_cast<const float*>(p.w13_s)[e];
    } else {
      v.wa = p.w2 + wbytes<FMT>((size_t)e * H, I);
      v.nkt = I * esz / 128;
      v.width = I;
      if (p.b2) v.b2 = p.b2 + (size_t)e * H;
      if (fmt_mx(FMT)) v.sa = static_cast<const uint8_t*>(p.w2_s) + (size_t)e * H * (I / 32);
      if (FMT == FMT_A8W8) v.wscale = static_cast<const float*>(p.w2_s)[e];
    }
  } else {
    // shared expert: whole (e < 0, dense) or pseudo-expert chunk c = e - E
    const int c = (e < 0) ? 0 : e - p.E;
    const int col0 = (e < 0) ? 0 : c * I;
    const int w = (e < 0) ? Is : min(I, Is - col0);
    if (STAGE == 1) {
      // rows col0.. of the gate and up halves (col0 is a multiple of 16)
      v.wa = p.ws13 + wbytes<FMT>(col0, H);
      v.wb = p.ws13 + wbytes<FMT>(Is + col0, H);
      v.nkt = H * esz / 128;
      v.width = w;
      if (p.bs13) {
        v.bg = p.bs13 + col0;
        v.bu = p.bs13 + Is + col0;
      }
      if (fmt_mx(FMT)) {
        v.sa = static_cast<const uint8_t*>(p.ws13_s) + (size_t)col0 * (H / 32);
        v.sb = static_cast<const uint8_t*>(p.ws13_s) + (size_t)(Is + col0) * (H / 32);
      }
      if (FMT == FMT_A8W8) v.wscale = static_cast<const float*>(p.ws13_s)[0];
    } else {
      // K columns col0.. of W2: a K-tile offset into every row block
      v.wa = p.ws2;
      v.nkt = Is * esz / 128;
      v.kt0 = col0 * esz / 128;
      v.width = w;
      if (c == 0) v.b2 = p.bs2;
      if (fmt_mx(FMT)) v.sa = static_cast<const uint8_t*>(p.ws2_s);
      if (FMT == FMT_A8W8) v.wscale = static_cast<const float*>(p.ws2_s)[0];
    }
  }
  return v;
}


// Per-row description of a block of BM sorted slots (or dense tokens).
// Bytes per row of the stage-2 input h: A8W8 rows keep the size of stage 1's
// bf16 output and carry their e4m3 codes at the start (quantised in place by
// quant_rows_kernel before stage 2).
template <int FMT>
__device__ __forceinline__ size_t h_row_bytes(const GemmParams& p) {
  return (size_t)p.ld_h * (FMT == FMT_A8W8 ? 2 : FmtInfo<FMT>::esz);
}

template <int FMT, int STAGE, int BM>
__device__ __forceinline__ void setup_rows(const GemmParams& p, int b, int tid, int* s_tok, int* s_pair,
                                           float* s_rw, float* s_rs) {
  const int P = p.T * p.k_total;
  if (tid < BM) {
    const int slot = b * BM + tid;
    int tok = -1, pair = -1;
    float rw = 0.f;
    if (p.dense) {
      tok = slot < p.T ? slot : -1;
      rw = (tok >= 0 && p.gamma) ? p.gamma[tok] : 1.0f;
    } else {
      pair = p.sorted[slot];
      if (pair < P) {
        tok = pair / p.k_total;
        if (STAGE == 2) rw = p.pair_w[pair];
      } else {
        pair = -1;
      }
    }
    s_tok[tid] = tok;
    s_pair[tid] = pair;
    s_rw[tid] = rw;
    float rs = 1.0f;
    if (FMT == FMT_A8W8) {
      if (STAGE == 1) {
        rs = tok >= 0 ? static_cast<const float*>(p.x_s)[tok] : 0.f;
      } else {
        const float amax = static_cast<const float*>(p.h_s)[slot];
        if (amax > 0.f) rs = __fdiv_rn(amax, 448.0f);
      }
    }
    s_rs[tid] = rs;
  }
}

// Stage-1 epilogue: the fp32 h tile sT[BM][LDT] (SiLU-mul already applied) is
// rounded / quantised and stored as rows of h (columns n0.. of the block's
// slots), MX scales and the per-row amax (A8W8) included.
template <int FMT, int BM, int BN>
__device__ __forceinline__ void epilogue_stage1(const GemmParams& p, const float* sT, int LDT, int b, int n0,
                                                int ncol_valid, const int* s_tok, int tid) {
  if constexpr (FMT == FMT_F32 || FMT == FMT_BF16 || FMT == FMT_A8W8) {
    constexpr int VPC = (FMT == FMT_F32) ? 4 : 8;  // values per 16-byte chunk
    constexpr int CPR = BN / VPC;                  // chunks per row
    for (int cid = tid; cid < BM * CPR; cid += 256) {
      const int r = cid / CPR, cc = cid % CPR;
      const int c = cc * VPC;
      const bool ok = s_tok[r] >= 0 && c < ncol_valid;
      const size_t slot = (size_t)b * BM + r;
      float amax = 0.f;
      if (ok) {
        const float* src = sT + r * LDT + c;
        if constexpr (FMT == FMT_F32) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.h) + slot * p.ld_h + n0 + c) =
              make_float4(src[0], src[1], src[2], src[3]);
        } else {
          uint32_t wds[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint32_t lo = f32_to_bf16(src[2 * u]), hi = f32_to_bf16(src[2 * u + 1]);
            wds[u] = lo | (hi << 16);
            amax = fmaxf(amax, fmaxf(fabsf(bf16_to_f32(lo)), fabsf(bf16_to_f32(hi))));
          }
          *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.h) + slot * p.ld_h + n0 + c) =
              make_uint4(wds[0], wds[1], wds[2], wds[3]);
        }
      }
      if constexpr (FMT == FMT_A8W8) {
        // row amax of the bf16-rounded values: reduce over the CPR lanes of a row
#pragma unroll
        for (int o = 1; o < CPR; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
        if (cc == 0 && s_tok[r] >= 0)
          atomicMax(reinterpret_cast<unsigned int*>(p.h_s) + slot, __float_as_uint(amax));
      }
    }
  } else {  // MX: one thread per (row, 32-column block)
    constexpr int BPR = BN / 32;
    for (int task = tid; task < BM * BPR; task += 256) {
      const int r = task / BPR, blk = task % BPR;
      const int c = blk * 32;
      if (s_tok[r] < 0 || c >= ncol_valid) continue;
      const float* src = sT + r * LDT + c;
      float v[32];
      float amax = 0.f;
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        v[u] = bf16_to_f32(f32_to_bf16(src[u]));
        amax = fmaxf(amax, fabsf(v[u]));
      }
      const int eb = (int)((__float_as_uint(amax) >> 23) & 0xFF);
      int X = (eb == 0) ? -127 : (eb - 127 - 8);
      X = X < -127 ? -127 : (X > 127 ? 127 : X);
      const float mul = __builtin_ldexpf(1.0f, -X);
      uint32_t wds[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) wds[u] = pack4_e4m3(v[4 * u] * mul, v[4 * u + 1] * mul, v[4 * u + 2] * mul, v[4 * u + 3] * mul);
      const size_t slot = (size_t)b * BM + r;
      uint8_t* dst = p.h + slot * p.ld_h + n0 + c;
      *reinterpret_cast<uint4*>(dst) = make_uint4(wds[0], wds[1], wds[2], wds[3]);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(wds[4], wds[5], wds[6], wds[7]);
      static_cast<uint8_t*>(p.h_s)[slot * (p.ld_h / 32) + (n0 + c) / 32] = (uint8_t)(X + 127);
    }
  }
}

// Stage-2 epilogue: STORE writes gamma * o (dense addend); ACCUMULATE stores
// the weighted pair rows with device-coherent stores, counts arrivals per
// (token, column tile) and lets the last arrival sum addend + rows in slot
// order with a single rounding into out.
template <int BM, int BN>
__device__ __forceinline__ void epilogue_stage2(const GemmParams& p, const float* sT, int LDT, int n0, int nt,
                                                int n_tiles, const int* s_tok, const int* s_pair,
                                                const float* s_rw, int* s_done, int tid) {
  const int lane = tid % kWave, wv = tid / kWave;
  if (p.mode == 0) {
    for (int r = wv; r < BM; r += 4) {
      const int tok = s_tok[r];
      if (tok < 0) continue;
      const float wgt = s_rw[r];
      float* dst = p.acc + (size_t)tok * p.H + n0;
      for (int c = lane; c < BN; c += kWave) dst[c] = wgt * sT[r * LDT + c];
    }
    return;
  }
  // Each (token, slot) pair owns one row of the pair buffer; rows are written
  // with device-coherent stores so that whichever workgroup completes a
  // (token, column tile) last can read them from any XCD.
  for (int r = wv; r < BM; r += 4) {
    const int pair = s_pair[r];
    if (pair < 0) continue;
    const float wgt = s_rw[r];
    float* dst = p.pair_out + (size_t)pair * p.H + n0;
    for (int c = lane; c < BN; c += kWave)
      __hip_atomic_store(dst + c, wgt * sT[r * LDT + c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // The counter increment only has to wait until this workgroup's row stores
  // are acknowledged (they are coherent by themselves); an agent-scope fence
  // would also write back and invalidate the XCD's whole L2.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid < BM) {
    int done = 0;
    const int tok = s_tok[tid];
    if (tok >= 0) {
      const int old = atomicAdd(p.counters + (size_t)tok * n_tiles + nt, 1);
      done = (old == p.expected - 1);
    }
    s_done[tid] = done;
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  // last arrival: addend + the token's rows in slot order, one rounding
  for (int r = wv; r < BM; r += 4) {
    if (!s_done[r]) continue;
    const int tok = s_tok[r];
    const float* rows = p.pair_out + (size_t)tok * p.k_total * p.H + n0;
    for (int c = lane; c < BN; c += kWave) {
      float v = p.acc ? p.acc[(size_t)tok * p.H + n0 + c] : 0.0f;
      for (int j = 0; j < p.k_total; ++j)
        v += __hip_atomic_load(rows + (size_t)j * p.H + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (p.out_bf16)
        static_cast<uint16_t*>(p.out)[(size_t)tok * p.H + n0 + c] = (uint16_t)f32_to_bf16(v);
      else
        static_cast<float*>(p.out)[(size_t)tok * p.H + n0 + c] = v;
    }
  }
}

// Last arrival at a (token, 64-column tile): the addend plus the token's
// k_total weighted pair rows, summed in slot order in fp32 and rounded once
// into out.  The calling lane covers the 16 columns from cbase.  Pair rows
// are read with device-coherent loads (they were written from other XCDs),
// four rows per round trip.
__device__ __forceinline__ void last_arrival_sum16(const GemmParams& p, int tok, int cbase) {
  float v[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) v[q] = p.acc ? p.acc[(size_t)tok * p.H + cbase + q] : 0.0f;
  const uint64_t* rows = reinterpret_cast<const uint64_t*>(p.pair_out + (size_t)tok * p.k_total * p.H + cbase);
  const size_t rstride = (size_t)(p.H / 2);  // one pair row, in 8-byte words
  int jj = 0;
  for (; jj + 4 <= p.k_total; jj += 4) {
    uint64_t t[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < 8; ++q)
        t[r][q] = __hip_atomic_load(rows + (jj + r) * rstride + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        v[2 * q] += __uint_as_float((uint32_t)t[r][q]);
        v[2 * q + 1] += __uint_as_float((uint32_t)(t[r][q] >> 32));
      }
  }
  for (; jj < p.k_total; ++jj) {
    uint64_t t[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      t[q] = __hip_atomic_load(rows + jj * rstride + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      v[2 * q] += __uint_as_float((uint32_t)t[q]);
      v[2 * q + 1] += __uint_as_float((uint32_t)(t[q] >> 32));
    }
  }
  if (p.out_bf16) {
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) w[q] = f32_to_bf16(v[2 * q]) | (f32_to_bf16(v[2 * q + 1]) << 16);
    uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + (size_t)tok * p.H + cbase);
    o[0] = make_uint4(w[0], w[1], w[2], w[3]);
    o[1] = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
    float4* o = reinterpret_cast<float4*>(static_cast<float*>(p.out) + (size_t)tok * p.H + cbase);
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  }
}

}  // namespace moe
