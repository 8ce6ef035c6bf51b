// Grouped GEMM for 256-row sorted blocks with both operands staged in LDS by
// direct-to-LDS buffer loads (gfx950), both stages.
//
// What it computes is what gemm_tile.hip computes (stage 1: x_gathered .
// W13[e]^T, the per-token / per-expert scales on the fp32 accumulator, MX-32
// block scales inside the block-scaled MFMA, bias, act(gate) * up rounded or
// quantised to the stage-2 format -- AITER PR 6106, "Technical Details";
// stage 2: h . W2[e]^T, the weighted pair rows and the last-arrival reduction
// onto the shared-expert addend -- vLLM PR 65207, "Purpose", commit 2); the
// difference is how the operands reach the matrix cores.
//
// Macro tile.  A workgroup of eight waves (two per SIMD) multiplies 256
// weight rows by the 256 token rows of a sorted block, 128 bytes of K at a
// time.  Both operands of a K tile (32 KiB each) are copied HBM/L2 -> LDS by
// buffer loads that write LDS directly (no VGPR staging, no ds_write), and
// every wave reads its fragments from LDS: each weight byte and each token
// byte crosses the CU's load path once per workgroup, i.e. 32 bytes per
// MFMA cycle of the CU at full rate (128-row blocks with weights in
// registers need 48), and the LDS serves the fragment reads (about 94 bytes
// per cycle at full rate; it delivers about 200 with eight waves per CU).
//
// Waves.  Wave w (w = 0..7) owns weight-row slots 8 (w & 1) .. + 7 (128
// rows) and token rows 64 (w >> 1) .. + 63.  Waves w and w + 4 share a SIMD
// and own token quarters q and q + 2, so a block with at most 128 live rows
// still keeps every SIMD busy, and quarters holding only padding skip their
// multiplies.  Stage 1: the wave's 128 weight rows are the gate and up rows of
// 64 h columns, so SiLU-mul happens in registers.  Stage 2: they are two
// 64-column reduction tiles.
//
// LDS per K tile (two buffers in ping-pong): the 16 weight row blocks in the
// tiled operand order the weights are stored in (16 rows x 128 bytes = 2 KiB,
// two 1 KiB halves, so a direct load of 1 KiB lands in operand order and a
// fragment read is 1 KiB contiguous); the 256 token rows row-major, 128 bytes
// each, with 16-byte chunk c of row r at slot c ^ ((r >> 1) & 7).  A direct
// load gives lane l row 8 i + l / 8 and slot l % 8, so eight lanes read one
// row's whole 128-byte line, and the fragment reads (lane (g, r): chunks g
// and 4 + g of row r; 32x32: chunk 2 s + l / 32 of row l % 32) hit sixteen
// different 16-byte bank groups per 16 lanes.
//
// Pipeline: the loads of K tile kt + 1 are issued before tile kt is
// multiplied; one vmcnt wait and one barrier per K tile.
//
// Stage 2 (ACCUMULATE) runs persistent workgroups on the per-XCD queues of
// gemm_tile.hip: item = (256-row block, group of four reduction tiles
// t = x + 8 (4 j + u), u = 0..3); every writer and the last-arrival reader of
// a (token, tile) run on XCD x.
#include "tile_common.hpp"

namespace moe {

constexpr int kLdsThreads = 512;
constexpr int kLdsBM = 256;

struct LdsStage {
  uint8_t w[16 * 2048];  // weight row blocks, tiled operand order
  uint8_t x[256 * 128];  // token rows, row-major, chunks XOR-swizzled
  uint8_t ws[16 * 64];   // MX: the weight row blocks' 64-byte scale tiles
  uint8_t xs[256 * 4];   // MX: the token rows' four e8m0 scales
};

struct LdsSmem {
  LdsStage st[2];
  int tok[kLdsBM];
  int pair[kLdsBM];
  float rw[kLdsBM];  // stage 2: pair weight
  float rs[kLdsBM];  // row scale (A8W8: stage 1 x scale, stage 2 h row scale)
  int item;
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ lds_ptr_t to_lds(void* p) { return (lds_ptr_t)p; }

// LDS byte offset of 16-byte chunk c of token row r
__device__ __forceinline__ int xrow_off(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

template <int FMT>
__device__ __forceinline__ void mfma_frag(f32x4& acc, const uint4& a0, const uint4& a1, const uint4& b0,
                                          const uint4& b1, int sa, int sb) {
  i32x8 A = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  i32x8 B = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 0, 0, 0, sa, 0, sb);
}

// One sorted block b (256 rows) against 256 weight rows.  Stage 1: h columns
// c0 .. c0 + 127 of expert view ev; stage 2: reduction tiles tiles[0..3]
// (tile < 0: none).  Fills the row tables first; the caller synchronises
// before the shared memory is reused.
template <int FMT, int STAGE, bool EPI>
__device__ __forceinline__ void lds_block(const GemmParams& p, LdsSmem& sm, int b, const ExpertView& ev, int c0,
                                          const int (&tiles)[4]) {
  constexpr int esz = FmtInfo<FMT>::esz;
  constexpr bool k32 = (FMT == FMT_BF16);
  constexpr bool mx = (FMT == FMT_MX);
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wv & 1, wn = wv >> 1;
  const int g = lane / 16, l16 = lane % 16;
  const int P = p.T * p.k_total;

  // ---- row tables ----
  float rw_row = 0.f, rs_row = 1.0f;
  bool real = false;
  if (tid < kLdsBM) {
    const int slot = b * kLdsBM + tid;
    const int pair = p.sorted[slot];
    int tok = -1, pr = -1;
    if (pair < P) {
      pr = pair;
      tok = pair / p.k_total;
      if (STAGE == 2) rw_row = p.pair_w[pair];
      real = true;
    }
    if (FMT == FMT_A8W8) {
      if (STAGE == 1) {
        rs_row = tok >= 0 ? static_cast<const float*>(p.x_s)[tok] : 0.f;
      } else {
        const float amax = static_cast<const float*>(p.h_s)[slot];
        if (amax > 0.f) rs_row = __fdiv_rn(amax, 448.0f);
      }
    }
    sm.tok[tid] = tok;
    sm.pair[tid] = pr;
    sm.rw[tid] = rw_row;
    sm.rs[tid] = rs_row;
  }
  const int live = __syncthreads_count(real);  // real rows come first, padding last
  if (live == 0) return;

  // ---- weight slots: slot s = 8 m + j of 16-row block (global) wrb[s] ----
  // stage 1: j < 4 gate rows c0 + 64 m + 16 j, j >= 4 the matching up rows;
  // stage 2: rows 64 t + 16 (j % 4) of tile t = tiles[2 m + j / 4].  Slots
  // whose rows lie past the view's width (a narrow pseudo chunk, a missing
  // tile) read row block 0 and their results are not stored.
  const int kbytes = (STAGE == 1) ? p.H * esz : ev.width * esz;
  const int nk = kbytes / 128;
  auto slot_rb = [&](int s, bool& up, bool& ok) {
    const int m = s / 8, j = s % 8;
    if (STAGE == 1) {
      up = j >= 4;
      const int col = c0 + 64 * m + 16 * (j % 4);
      ok = col < ev.width;
      return ok ? col / 16 : 0;
    }
    up = false;
    const int t = tiles[2 * m + j / 4];
    ok = t >= 0;
    return ok ? 4 * t + (j % 4) : 0;
  };
  // this wave loads slots 2 wv and 2 wv + 1 (both halves each)
  __amdgpu_buffer_rsrc_t wrs[2];
  uint32_t wtile[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    bool up, ok;
    const int rb = slot_rb(2 * wv + i, up, ok);
    wrs[i] = tile_rsrc(up ? ev.wb : ev.wa, 0x7FFFFFFF);
    wtile[i] = (uint32_t)tile_off(ev, rb, 0);
  }
  // MX weight scales (wave 0): lane l -> slot l / 4, 16-byte piece l % 4 of
  // the slot's 64-byte scale tile; offsets relative to ev.sa
  const __amdgpu_buffer_rsrc_t wsrs = tile_rsrc(mx ? ev.sa : ev.wa, 0x7FFFFFFF);
  uint32_t wsoff = 0;
  if constexpr (mx) {
    bool up, ok;
    const int rb = slot_rb(lane / 4, up, ok);
    wsoff = (uint32_t)((up ? (size_t)(ev.sb - ev.sa) : 0) + scale_tile_off(ev, rb, 0)) + 16 * (lane % 4);
  }

  // ---- token rows: instruction i (0..3) of wave wv covers rows 8 (4 wv + i)
  // .. + 7; lane l -> row 8 (4 wv + i) + l / 8, slot l % 8 ----
  const size_t hrb = h_row_bytes<FMT>(p);
  const size_t srows = (size_t)p.max_blocks * kLdsBM;
  const __amdgpu_buffer_rsrc_t xrs = (STAGE == 1) ? tile_rsrc(p.x, (uint32_t)((size_t)p.T * p.H * esz))
                                                  : tile_rsrc(p.h, (uint32_t)(srows * hrb));
  // (MX only) the token rows' e8m0 scales
  const __amdgpu_buffer_rsrc_t xsrs = (STAGE == 1) ? tile_rsrc(p.x_s, (uint32_t)((size_t)p.T * (p.H / 32)))
                                                   : tile_rsrc(p.h_s, (uint32_t)(srows * (p.ld_h / 32)));
  uint32_t xoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * (4 * wv + i) + lane / 8;
    const int c = (lane % 8) ^ ((r >> 1) & 7);  // the chunk that lands in slot lane % 8
    const int tok = sm.tok[r];
    if (tok < 0) xoff[i] = kTileOutOfRange;
    else if (STAGE == 1) xoff[i] = (uint32_t)((size_t)tok * p.H * esz) + 16 * c;
    else xoff[i] = (uint32_t)(((size_t)b * kLdsBM + r) * hrb) + 16 * c;
  }
  // MX token scales (waves 4..7, one dword per row): row 64 (wv - 4) + lane
  uint32_t xsoff = kTileOutOfRange;
  if (mx && wv >= 4) {
    const int r = 64 * (wv - 4) + lane;
    const int tok = sm.tok[r];
    if (tok >= 0)
      xsoff = (STAGE == 1) ? (uint32_t)(tok * (p.H / 32)) : (uint32_t)((b * kLdsBM + r) * (p.ld_h / 32));
  }

  auto issue = [&](int buf, int kt) {
    LdsStage& S = sm.st[buf];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs[i / 2], to_lds(S.w + (2 * wv + i / 2) * 2048 + (i % 2) * 1024),
                                               16, (int)(lane * 16 + (i % 2) * 1024),
                                               (int)(wtile[i / 2] + (uint32_t)kt * 2048), 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (8 * (4 * wv + i) < live)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, to_lds(S.x + (4 * wv + i) * 1024), 16, (int)xoff[i],
                                                 kt * 128, 0, 0);
    if constexpr (mx) {
      if (wv == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wsrs, to_lds(S.ws), 16, (int)wsoff, kt * 64, 0, 0);
      if (wv >= 4 && 64 * (wv - 4) < live)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xsrs, to_lds(S.xs + (wv - 4) * 256), 4, (int)xsoff, kt * 4, 0,
                                                 0);
    }
  };

  // ---- accumulators: one of the two sets is used ----
  f32x4 acc[8][4];    // 16x16x128: [slot j][token block q]
  f32x16 acc32[4][2];  // 32x32x16: [32-row weight block][32-row token block]
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[j][q] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc32[i][n][v] = 0.f;

  const int rq0 = 64 * wn;  // the wave's first token row
  const bool wave_live = rq0 < live;

  auto compute = [&](int buf) {
    const LdsStage& S = sm.st[buf];
    if (!wave_live) return;
    __builtin_amdgcn_s_setprio(1);
    if constexpr (k32) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        uint4 bf[2];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const int r = rq0 + 32 * n + lane % 32;
          bf[n] = *reinterpret_cast<const uint4*>(&S.x[xrow_off(r, 2 * st + lane / 32)]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = 8 * wm + 2 * i + (lane % 32) / 16;
          const uint4 af = *reinterpret_cast<const uint4*>(&S.w[s * 2048 + 512 * st + 16 * (16 * (lane / 32) + l16)]);
#pragma unroll
          for (int n = 0; n < 2; ++n) {
            if (rq0 + 32 * n >= live) continue;  // wave-uniform: padding rows only
            acc32[i][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af),
                                                                 __builtin_bit_cast(bf16x8, bf[n]), acc32[i][n], 0, 0,
                                                                 0);
          }
        }
      }
    } else {
      uint4 b0[4], b1[4];
      int sbv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = rq0 + 16 * q + l16;
        b0[q] = *reinterpret_cast<const uint4*>(&S.x[xrow_off(r, g)]);
        b1[q] = *reinterpret_cast<const uint4*>(&S.x[xrow_off(r, 4 + g)]);
        sbv[q] = mx ? (int)S.xs[r * 4 + g] : 127;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int s = 8 * wm + j;
        const uint4 a0 = *reinterpret_cast<const uint4*>(&S.w[s * 2048 + lane * 16]);
        const uint4 a1 = *reinterpret_cast<const uint4*>(&S.w[s * 2048 + 1024 + lane * 16]);
        const int sa = mx ? (int)S.ws[s * 64 + lane] : 127;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (rq0 + 16 * q >= live) continue;  // wave-uniform: padding rows only
          mfma_frag<FMT>(acc[j][q], a0, a1, b0[q], b1[q], sa, sbv[q]);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- K loop: loads of tile kt + 1 in flight while tile kt multiplies ----
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) issue((kt + 1) & 1, kt + 1);
    compute(kt & 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- epilogues ----
  if (!wave_live) {
    if (STAGE == 1 || p.mode == 0) return;
  }
  if constexpr (STAGE == 1) {
    const int hc0 = c0 + 64 * wm;  // the wave's 64 h columns
    if (hc0 >= ev.width) return;
    if constexpr (k32) {
      // acc32[i][n][4 jj + v] = weight row 8 jj + 4 (l / 32) + v of 32-row block i
      // x token row rq0 + 32 n + l % 32; blocks 0, 1 gate, 2, 3 up
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int r = rq0 + 32 * n + lane % 32;
        if (r >= live) continue;
        const size_t slot = (size_t)b * kLdsBM + r;
        const float sc = sm.rs[r] * ev.wscale;
        uint16_t* dst = reinterpret_cast<uint16_t*>(p.h) + slot * p.ld_h + hc0 + 4 * (lane / 32);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (hc0 + 32 * i >= ev.width) continue;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            uint32_t bits[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int col = hc0 + 4 * (lane / 32) + 32 * i + 8 * jj + v;
              bits[v] = f32_to_bf16(epi_act<EPI>(acc32[i][n][4 * jj + v] * sc + epi_bias<EPI>(ev.bg, col, ev.width),
                                            acc32[i + 2][n][4 * jj + v] * sc + epi_bias<EPI>(ev.bu, col, ev.width),
                                            p.act));
            }
            *reinterpret_cast<uint2*>(dst + 32 * i + 8 * jj) =
                make_uint2(bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16));
          }
        }
      }
    } else {
      // acc[j][q][v] = weight row 4 g + v of slot j x token row rq0 + 16 q + l16;
      // h column hc0 + 16 j + 4 g + v (j < 4 gate, j + 4 up)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (rq0 + 16 * q >= live) continue;  // wave-uniform
        const int r = rq0 + 16 * q + l16;
        const bool rok = r < live;
        const size_t slot = (size_t)b * kLdsBM + r;
        const float sc = sm.rs[r] * ev.wscale;
        float hv[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int col = hc0 + 16 * j + 4 * g + v;
            hv[j][v] = epi_act<EPI>(acc[j][q][v] * sc + epi_bias<EPI>(ev.bg, col, ev.width),
                               acc[j + 4][q][v] * sc + epi_bias<EPI>(ev.bu, col, ev.width), p.act);
          }
        if constexpr (mx) {
          // columns hc0 + 32 k .. + 31 (j = 2 k, 2 k + 1) are one MX-32 block
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            float amax = 0.f;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                hv[2 * k + jj][v] = bf16_to_f32(f32_to_bf16(hv[2 * k + jj][v]));
                amax = fmaxf(amax, fabsf(hv[2 * k + jj][v]));
              }
            amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
            amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
            const int eb = (int)((__float_as_uint(amax) >> 23) & 0xFF);
            int X = (eb == 0) ? -127 : (eb - 127 - 8);
            X = X < -127 ? -127 : (X > 127 ? 127 : X);
            const float mul = __builtin_ldexpf(1.0f, -X);
            const int col = hc0 + 32 * k;
            if (rok && col < ev.width) {
              uint8_t* dst = p.h + slot * p.ld_h + col + 4 * g;
#pragma unroll
              for (int jj = 0; jj < 2; ++jj)
                *reinterpret_cast<uint32_t*>(dst + 16 * jj) =
                    pack4_e4m3(hv[2 * k + jj][0] * mul, hv[2 * k + jj][1] * mul, hv[2 * k + jj][2] * mul,
                               hv[2 * k + jj][3] * mul);
              if (g == 0) static_cast<uint8_t*>(p.h_s)[slot * (p.ld_h / 32) + col / 32] = (uint8_t)(X + 127);
            }
          }
        } else {
          float amax = 0.f;
          uint16_t* dst = reinterpret_cast<uint16_t*>(p.h) + slot * p.ld_h + hc0 + 4 * g;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t bits[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              bits[v] = f32_to_bf16(hv[j][v]);
              if (hc0 + 16 * j < ev.width) amax = fmaxf(amax, fabsf(bf16_to_f32(bits[v])));
            }
            if (rok && hc0 + 16 * j < ev.width)
              *reinterpret_cast<uint2*>(dst + 16 * j) = make_uint2(bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16));
          }
          if constexpr (FMT == FMT_A8W8) {
            amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
            amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
            if (g == 0 && rok) atomicMax(reinterpret_cast<unsigned int*>(p.h_s) + slot, __float_as_uint(amax));
          }
        }
      }
    }
    return;
  }

  // ---- stage 2, ACCUMULATE: the weighted pair rows of the wave's two tiles
  // in the 16-bit block-scaled form, staged through this wave's 4 KiB of the
  // idle token buffer (16-byte chunk c of row rr at rr * 128 + 16 (c ^ (rr & 7)))
  // so that eight lanes store each (pair, tile) line whole ----
  const int ta = tiles[2 * wm], tb = tiles[2 * wm + 1];
  uint8_t* wl = &sm.st[0].x[0] + wv * 4096;
  auto store_rows = [&](int r0, int nrows, int t) {
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rr = lane / 8 + 8 * k;
      const int c = lane % 8;
      if (rr < nrows) {
        const uint4 v = *reinterpret_cast<const uint4*>(wl + rr * 128 + 16 * (c ^ (rr & 7)));
        const int pr = sm.pair[r0 + rr];
        if (pr >= 0) *reinterpret_cast<uint4*>(pair_codes(p) + (size_t)pr * p.H + 64 * t + 8 * c) = v;
      }
    }
    wave_lds_sync();  // the next group rewrites the region
  };
  if (wave_live) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = u ? tb : ta;
      if (t < 0) continue;
      if constexpr (k32) {
        // lanes l and l + 32 hold the tile's 64 columns of token row
        // rq0 + 32 n + l % 32 (columns 32 ii + 8 jj + 4 (l / 32) + 0..3, block 2 u + ii)
        const int rl = lane % 32, hh = lane / 32;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          if (rq0 + 32 * n >= live) continue;
          const int r = rq0 + 32 * n + rl;
          const float sc = sm.rs[r] * ev.wscale;
          const float wgt = sm.rw[r];
          float amax = 0.f;
#pragma unroll
          for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              acc32[2 * u + ii][n][v] =
                  wgt * (acc32[2 * u + ii][n][v] * sc + epi_bias<EPI>(ev.b2, 64 * t + 32 * ii + 8 * (v / 4) + 4 * hh + v % 4));
              amax = tile_amax(amax, acc32[2 * u + ii][n][v]);
            }
          amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
          const int field = pair_tile_field(amax);
#pragma unroll
          for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const int col = 32 * ii + 8 * jj + 4 * hh;
              *reinterpret_cast<uint2*>(wl + rl * 128 + 16 * ((4 * ii + jj) ^ (rl & 7)) + 8 * hh) =
                  make_uint2(pair_code2(acc32[2 * u + ii][n][4 * jj], acc32[2 * u + ii][n][4 * jj + 1], field, col),
                             pair_code2(acc32[2 * u + ii][n][4 * jj + 2], acc32[2 * u + ii][n][4 * jj + 3], field,
                                        col + 2));
            }
          store_rows(rq0 + 32 * n, 32, t);
        }
      } else {
        // lanes (g, l16) hold the tile's 64 columns of token row rq0 + 16 q +
        // l16 (columns 16 jj + 4 g + 0..3, slot 4 u + jj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (rq0 + 16 * q >= live) continue;
          const int r = rq0 + 16 * q + l16;
          const float sc = sm.rs[r] * ev.wscale;
          const float wgt = sm.rw[r];
          float amax = 0.f;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              acc[4 * u + jj][q][v] = wgt * (acc[4 * u + jj][q][v] * sc + epi_bias<EPI>(ev.b2, 64 * t + 16 * jj + 4 * g + v));
              amax = tile_amax(amax, acc[4 * u + jj][q][v]);
            }
          amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
          amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
          const int field = pair_tile_field(amax);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int col = 16 * jj + 4 * g;
            *reinterpret_cast<uint2*>(wl + l16 * 128 + 16 * ((2 * jj + g / 2) ^ (l16 & 7)) + 8 * (g % 2)) =
                make_uint2(pair_code2(acc[4 * u + jj][q][0], acc[4 * u + jj][q][1], field, col),
                           pair_code2(acc[4 * u + jj][q][2], acc[4 * u + jj][q][3], field, col + 2));
          }
          store_rows(rq0 + 16 * q, 16, t);
        }
      }
    }
  }
  // count arrivals once the wave's stores have reached the L2 (their
  // acknowledgement): lane l counts token row rq0 + l for both tiles
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  const int n64 = p.H / 64;
  uint64_t done[2] = {0, 0};
  if (wave_live) {
    const int r = rq0 + lane;
    const int pr = sm.pair[r];
    const int tok = sm.tok[r];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = u ? tb : ta;
      int old = -1;
      if (t >= 0 && pr >= 0) old = atomicAdd(p.counters + (size_t)tok * n64 + t, 1);
      done[u] = __ballot(old == p.expected - 1);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  // the wave's last arrivals, eight lanes per (token, tile)
  const int total = __popcll(done[0]) + __popcll(done[1]);
  for (int base = 0; base < total; base += 8) {
    const int i = base + lane / 8;
    if (i < total) {
      int rem = i, u = 0;
      uint64_t msk = done[0];
      if (rem >= __popcll(done[0])) {
        rem -= __popcll(done[0]);
        u = 1;
        msk = done[1];
      }
      for (int k = 0; k < rem; ++k) msk &= msk - 1;  // drop the lowest rem set bits
      const int r = rq0 + (__ffsll((unsigned long long)msk) - 1);
      last_arrival_sum8_xcd(p, sm.tok[r], 64 * (u ? tb : ta), lane % 8, lane);
    }
  }
}

// Stage 1: one workgroup per (256-row block, 128 h columns), expert-major
// and XCD-contiguous like the tiled kernels.
template <int FMT, bool EPI>
__global__ __launch_bounds__(kLdsThreads) void gemm_lds_stage1_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) LdsSmem sm;
  const int n_col = p.I / 128;
  const int nblk = *p.num_blocks;
  const int active = nblk * n_col;
  if ((int)blockIdx.x >= active) return;
  const int lt = xcd_remap((int)blockIdx.x, active);
  int b = lt / n_col, nc = lt % n_col;
  const int e = p.offsets ? expert_major(p, kLdsBM, n_col, lt, b, nc) : p.block_expert[b];
  const ExpertView ev = resolve_expert<FMT, 1>(p, e);
  const int c0 = nc * 128;
  if (c0 >= ev.width) return;  // past a narrow pseudo-expert chunk (uniform)
  const int none[4] = {-1, -1, -1, -1};
  lds_block<FMT, 1, EPI>(p, sm, b, ev, c0, none);
}

// Stage 2 ACCUMULATE: persistent workgroups draining the per-XCD queues
// (queue x: items (block, group j), tiles t = x + 8 (4 j + u), u = 0..3).
template <int FMT, bool EPI>
__global__ __launch_bounds__(kLdsThreads) void gemm_lds_accum_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) LdsSmem sm;
  const int tid = threadIdx.x;
  const int n64 = p.H / 64;
  const int nblk = *p.num_blocks;
  int* q_next = p.counters + (size_t)p.T * n64;
  int* q_owner = q_next + kNumXcd;
  const int me = xcc_id();
  for (int step = 0; step < kNumXcd; ++step) {
    const int q = (me + step) % kNumXcd;
    const int tiles_q = (n64 - q + kNumXcd - 1) / kNumXcd;  // t = q (mod 8), t < n64
    const int groups_q = (tiles_q + 3) / 4;
    const int items_q = nblk * groups_q;
    if (items_q <= 0) continue;
    if (tid == 0) {
      const int o = atomicCAS(q_owner + q, 0, me + 1);
      sm.item = (o == 0 || o == me + 1) ? 1 : 0;
    }
    __syncthreads();
    const bool ours = sm.item != 0;
    __syncthreads();
    if (!ours) continue;
    for (;;) {
      if (tid == 0) sm.item = atomicAdd(q_next + q, 1);
      __syncthreads();
      const int it = sm.item;
      __syncthreads();
      if (it >= items_q) break;
      int b = it / groups_q, j = it % groups_q;
      const int e = p.offsets ? expert_major(p, kLdsBM, groups_q, it, b, j) : p.block_expert[b];
      int tiles[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = q + kNumXcd * (4 * j + u);
        tiles[u] = t < n64 ? t : -1;
      }
      const ExpertView ev = resolve_expert<FMT, 2>(p, e);
      lds_block<FMT, 2, EPI>(p, sm, b, ev, 0, tiles);
      __syncthreads();  // the next item rewrites the row tables and buffers
    }
  }
}

// 256-row blocks, sorted problem: stage 1 needs whole 128-column workgroups
// (and 32-column-aligned pseudo chunks), stage 2 ACCUMULATE 64-column tiles;
// 32-bit buffer offsets for the token rows.
bool lds_kernel_fits(const GemmParams& p, int stage, int fmt) {
  if (fmt == FMT_F32 || fmt == FMT_MX4 || p.dense || p.block_m != kLdsBM || p.bsplit > 1) return false;
  const size_t esz = fmt == FMT_BF16 ? 2 : 1;
  const size_t hsz = fmt == FMT_A8W8 ? 2 : esz;
  if (stage == 1) {
    if (p.I % 128) return false;
    if (p.n_pseudo > 0 && p.I_s % 32) return false;
    return (size_t)p.T * p.H * esz < 0x7FFFFFFFu;
  }
  if (p.mode == 0 || p.H % 64) return false;
  return (size_t)p.max_blocks * kLdsBM * p.ld_h * hsz < 0x7FFFFFFFu;
}

template <int FMT, bool EPI>
static hipError_t launch_lds_fe(const GemmParams& p, int stage, hipStream_t s) {
  if (stage == 1) {
    const dim3 grid((unsigned)(p.max_blocks * (p.I / 128)));
    return launch_gemm_kernel(gemm_lds_stage1_kernel<FMT, EPI>, grid, dim3(kLdsThreads), s, p);
  }
  // persistent: one workgroup per CU (an XCD has 32), no more than the
  // largest queue has items
  const int n64 = p.H / 64;
  const int groups = ((n64 + kNumXcd - 1) / kNumXcd + 3) / 4;
  long long per_xcd = (long long)p.max_blocks * groups;
  if (per_xcd > 32) per_xcd = 32;
  return launch_gemm_kernel(gemm_lds_accum_kernel<FMT, EPI>, dim3((unsigned)(kNumXcd * per_xcd)), dim3(kLdsThreads),
                            s, p);
}

template <int FMT>
static hipError_t launch_lds_fmt(const GemmParams& p, int stage, hipStream_t s) {
  return epi_general(p, stage) ? launch_lds_fe<FMT, true>(p, stage, s) : launch_lds_fe<FMT, false>(p, stage, s);
}

hipError_t launch_gemm_lds(const GemmParams& p, int stage, int fmt, hipStream_t s) {
  switch (fmt) {
    case FMT_BF16: return launch_lds_fmt<FMT_BF16>(p, stage, s);
    case FMT_MX: return launch_lds_fmt<FMT_MX>(p, stage, s);
    case FMT_A8W8: return launch_lds_fmt<FMT_A8W8>(p, stage, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
