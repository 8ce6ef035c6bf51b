// Device helpers shared by the tiled grouped-GEMM kernels (gemm_tile.hip:
// weights in registers, token rows through LDS; gemm_lds.hip: both operands
// through LDS by direct loads): XCD-aware placement, buffer loads, the
// expert-major work order, and the 16-bit block-scaled stage-2 pair rows with
// their last-arrival reduction.
#pragma once

#include "gemm_common.hpp"

namespace moe {

constexpr int kNumXcd = 8;
constexpr uint32_t kTileOutOfRange = 0x80000000u;  // buffer offset past every range: reads zero

// Bijection of [0, active) that gives each XCD (blockIdx % 8) a contiguous
// range of logical tile indices.
__device__ __forceinline__ int xcd_remap(int bid, int active) {
  const int q = active / kNumXcd, r = active % kNumXcd;
  const int x = bid % kNumXcd, i = bid / kNumXcd;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

// The XCD this wave runs on (HW_REG_XCC_ID, bits 2:0).
__device__ __forceinline__ int xcc_id() {
  return __builtin_amdgcn_s_getreg((15 << 11) | (0 << 6) | 20) & (kNumXcd - 1);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, uint32_t bytes) {
  // raw (untyped) buffer, dword 3 = 0x00020000 on gfx9-family parts
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 tile_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

// Expert-major order of a launch's work: the items of expert e (its blocks x
// n_per column tiles, a contiguous range in block-major order) are taken
// column tile by column tile, the blocks of one column tile side by side, so
// the concurrent workgroups of an expert share each weight tile through L2
// instead of streaming the expert's weights once per block.  In: the item
// index `it` of block-major order; out: block b and column tile c; returns
// the expert.
__device__ __forceinline__ int split_of(const GemmParams& p) { return p.bsplit > 1 ? p.bsplit : 1; }

__device__ __forceinline__ int expert_major(const GemmParams& p, int BM, int n_per, int it, int& b, int& c) {
  const int e = p.block_expert[it / n_per / split_of(p)];
  const int bs = p.offsets[e] / BM, nb = (p.offsets[e + 1] - p.offsets[e]) / BM;
  const int local = it - bs * n_per;
  c = local / nb;
  b = bs + local % nb;
  return e;
}

// Stage-2 pair rows in 16-bit block-scaled form.  The 64 values v of one
// (pair, 64-column tile) become one 128-byte line of 16-bit words
// 2 q + b: q = rint(v * 2^(14 - e)) saturated to +-16383, with e the frexp
// exponent of the tile's largest magnitude (|v| < 2^e) raised to at least
// -126, and b, the lowest bit of the words of columns 0..7, spelling the
// 8-bit field e + 126 (255: the tile holds a non-finite value).  Each value
// is held to within 2^-13 of the tile's largest magnitude, at half the bytes
// of fp32, and every line is written once and read once, so no cache ever
// holds a stale copy of it.  The words fill the first P*H*2 bytes of the pair
// buffer.
constexpr int kPairNonFinite = 255;

__device__ __forceinline__ int16_t* pair_codes(const GemmParams& p) { return reinterpret_cast<int16_t*>(p.pair_out); }
// Running largest magnitude of a tile that also records non-finite values:
// a NaN or an infinity makes it +Inf for good (fmaxf alone would drop a NaN),
// so the tile's field below becomes kPairNonFinite and its sum NaN.
__device__ __forceinline__ float tile_amax(float amax, float v) {
  const float m = fabsf(v);
  return m <= 3.4028234664e38f ? fmaxf(amax, m) : __builtin_inff();
}
// The tile's 8-bit exponent field from its largest magnitude.
__device__ __forceinline__ int pair_tile_field(float amax) {
  if (!(amax <= 3.4028234664e38f)) return kPairNonFinite;  // Inf or NaN
  int ex;
  (void)__builtin_frexpf(amax, &ex);  // amax = m * 2^ex, m in [0.5, 1); 0 for amax = 0
  return (ex < -126 ? -126 : ex) + 126;
}
// Words of two values of columns col, col + 1 of the tile (low half first).
__device__ __forceinline__ uint32_t pair_code2(float a, float b, int field, int col) {
  const int sh = 14 - ((field == kPairNonFinite ? 0 : field) - 126);
  int qa = (int)__builtin_rintf(__builtin_ldexpf(a, sh));
  int qb = (int)__builtin_rintf(__builtin_ldexpf(b, sh));
  qa = qa > 16383 ? 16383 : (qa < -16383 ? -16383 : qa);
  qb = qb > 16383 ? 16383 : (qb < -16383 ? -16383 : qb);
  const int ba = col < 8 ? (field >> col) & 1 : 0;
  const int bb = col + 1 < 8 ? (field >> (col + 1)) & 1 : 0;
  return ((uint32_t)(2 * qa + ba) & 0xFFFFu) | ((uint32_t)(2 * qb + bb) << 16);
}

// Stage-2 pair rows of the waves' last arrivals: the addend plus the token's
// k_total pair rows in slot order (each q times its tile's power of two, an
// exact product, added in fp32), one rounding.  Eight lanes share a token
// (lane part c sums columns cbase + 8c .. + 7), so each load of a row reads
// its 128-byte line whole; part 0 holds the exponent bits and passes the
// field to the other seven.  Read with ordinary loads: every pair row of the
// tile was written through this XCD's L2.
__device__ __forceinline__ void last_arrival_sum8_xcd(const GemmParams& p, int tok, int cbase, int c, int lane) {
  const int col = cbase + 8 * c;
  float v[8];
  if (p.acc) {
    const float4 a0 = *reinterpret_cast<const float4*>(p.acc + (size_t)tok * p.H + col);
    const float4 a1 = *reinterpret_cast<const float4*>(p.acc + (size_t)tok * p.H + col + 4);
    v[0] = a0.x, v[1] = a0.y, v[2] = a0.z, v[3] = a0.w;
    v[4] = a1.x, v[5] = a1.y, v[6] = a1.z, v[7] = a1.w;
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = 0.f;
  }
  const int16_t* rows = pair_codes(p) + (size_t)tok * p.k_total * p.H + col;
  const int src = lane & ~7;  // part 0 of this token
  auto add_row = [&](const uint4& t) {
    const uint32_t w[4] = {t.x, t.y, t.z, t.w};
    int field = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) field |= (int)((w[q] & 1u) << (2 * q)) | (int)(((w[q] >> 16) & 1u) << (2 * q + 1));
    field = __shfl(field, src, kWave);
    const float s = field == kPairNonFinite ? __builtin_nanf("") : __builtin_ldexpf(1.0f, field - 126 - 14);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] += (float)((int)(int16_t)(w[q] & 0xFFFFu) >> 1) * s;
      v[2 * q + 1] += (float)((int)(int16_t)(w[q] >> 16) >> 1) * s;
    }
  };
  int jj = 0;
  for (; jj + 4 <= p.k_total; jj += 4) {
    uint4 t[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) t[r] = *reinterpret_cast<const uint4*>(rows + (size_t)(jj + r) * p.H);
#pragma unroll
    for (int r = 0; r < 4; ++r) add_row(t[r]);
  }
  for (; jj < p.k_total; ++jj) add_row(*reinterpret_cast<const uint4*>(rows + (size_t)jj * p.H));
  if (p.out_bf16) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = f32_to_bf16(v[2 * q]) | (f32_to_bf16(v[2 * q + 1]) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + (size_t)tok * p.H + col) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    float4* o = reinterpret_cast<float4*>(static_cast<float*>(p.out) + (size_t)tok * p.H + col);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

}  // namespace moe
