// Two-stage routed grouped GEMM for gfx950 (MFMA, LDS-staged tiles).
//
// Stage 1 (vLLM PR 65207, "Purpose", commit 2 names the AITER stages): for
// each sorted block of rows owned by expert e, a = x_gathered . W13[e]^T with
// fp32 accumulation; the per-token and per-expert scales multiply the fp32
// accumulator before the activation (AITER PR 6106, "Technical Details"),
// MX-32 block scales are applied by the block-scaled MFMA inside the K loop;
// the epilogue computes h = act(a_gate) * a_up (bias added first) and rounds / quantises it to
// the stage-2 input format (bf16, MX-32 e4m3, or bf16 plus a per-row amax
// from which stage 2 derives the per-row e4m3 scale).
//
// Stage 2: o = h . W2[e]^T, times the scales; the epilogue stores pair_w * o
// as the pair's fp32 row, and the last of the expected contributions to a
// (token, column tile) sums the addend (the shared expert's output when it ran
// on the aux stream) and the token's pair rows in slot order and rounds the
// fp32 sum once into the output (vLLM PR 65207, commit 2: the shared output is
// accumulated in the stage-2 epilogue instead of by a separate add).  In
// STORE mode (dense shared expert) it writes gamma_t * o into the addend.
//
// Tiles: 256 threads = 4 waves; BM sorted rows x BN output columns; the K tile
// is 128 bytes of the operand format (32 fp32, 64 bf16 or 128 fp8 elements).
// Operands live in LDS as 128-byte rows of eight 16-byte chunks, XOR-swizzled
// by row.  In every 128-byte K tile, lane group g = lane/16 feeds chunks g and
// 4+g to the MFMA; this matches the gfx950 16x16x128 f8f6f4 operand order
// (bytes 0-15 = K 16g.., bytes 16-31 = K 64+16g..) and the 32-element MX
// blocks, and for the other formats it is a consistent permutation of K on
// both operands.
#include "gemm_common.hpp"

namespace moe {

template <int FMT, int STAGE, int BM, int BN>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams p) {
  constexpr int esz = FmtInfo<FMT>::esz;
  constexpr bool kFp8 = FmtInfo<FMT>::fp8;
  constexpr int WM = (BM >= 32) ? 2 : 1;
  constexpr int WN = 4 / WM;
  constexpr int RW = BM / WM, CW = BN / WN;
  constexpr int TI = RW / 16, TJ = CW / 16;
  constexpr int BROWS = (STAGE == 1) ? 2 * BN : BN;
  constexpr int A_CH = BM * 8, B_CH = BROWS * 8;
  constexpr int A_PER = (A_CH + 255) / 256, B_PER = (B_CH + 255) / 256;
  constexpr int TILE_BYTES = 2 * (BM + BROWS) * 128;
  constexpr int EPI_BYTES = BM * (BN + 4) * 4;
  constexpr int SMEM = TILE_BYTES > EPI_BYTES ? TILE_BYTES : EPI_BYTES;

  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  __shared__ uint32_t s_asc[2][BM];
  __shared__ uint32_t s_bsc[2][BROWS];
  __shared__ int s_tok[BM];
  __shared__ int s_pair[BM];
  __shared__ float s_rs[BM];   // row scale (stage 1 A8W8: x scale; stage 2 A8W8: h row scale)
  __shared__ float s_rw[BM];   // stage 2: pair weight / gate
  __shared__ int s_done[BM];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wv = tid / kWave;
  const int wm = wv / WN, wn = wv % WN;

  const int width_max = (STAGE == 1) ? (p.dense ? p.I_s : p.I) : p.H;
  const int n_tiles = (width_max + BN - 1) / BN;
  const int b = blockIdx.x / n_tiles;
  const int nt = blockIdx.x % n_tiles;
  const int n0 = nt * BN;

  int e;
  if (p.dense) {
    if (b * BM >= p.T) return;
    e = -1;
  } else {
    if (b >= *p.num_blocks) return;
    e = p.block_expert[b];
  }
  const ExpertView ev = resolve_expert<FMT, STAGE>(p, e);
  if (STAGE == 1 && n0 >= ev.width) return;  // tile past a narrow pseudo-expert chunk

  setup_rows<FMT, STAGE, BM>(p, b, tid, s_tok, s_pair, s_rw, s_rs);
  __syncthreads();

  // ---- per-thread load descriptors ----
  const int kbytes = (STAGE == 1) ? p.H * esz : ev.width * esz;  // valid K bytes (LDS format)
  const int nk = (kbytes + 127) / 128;
  const uint8_t* a_ptr[A_PER];
  bool a_ok[A_PER];
#pragma unroll
  for (int q = 0; q < A_PER; ++q) {
    const int cid = tid + q * 256;
    const int r = cid / 8, c = cid % 8;
    a_ok[q] = false;
    a_ptr[q] = nullptr;
    if (cid < A_CH) {
      if (STAGE == 1) {
        const int tok = s_tok[r];
        a_ok[q] = tok >= 0;
        a_ptr[q] = p.x + ((size_t)(tok < 0 ? 0 : tok) * p.H * esz + c * 16);
      } else {
        const int slot = b * BM + r;
        a_ok[q] = s_tok[r] >= 0;
        a_ptr[q] = p.h + (size_t)slot * h_row_bytes<FMT>(p) + c * 16;
      }
    }
  }
  const uint8_t* b_ptr[B_PER];
  bool b_ok[B_PER];
#pragma unroll
  for (int q = 0; q < B_PER; ++q) {
    const int cid = tid + q * 256;
    const int r = cid / 8, c = cid % 8;
    b_ok[q] = false;
    b_ptr[q] = nullptr;
    if (cid < B_CH) {
      // chunk c of weight row col in K tile 0 of the tiled layout; a K tile
      // further on is 2048 bytes later
      if (STAGE == 1) {
        const int col = n0 + (r % BN);
        b_ok[q] = col < ev.width;
        const int cr = b_ok[q] ? col : 0;
        const uint8_t* base = (r < BN) ? ev.wa : ev.wb;
        b_ptr[q] = base + tile_off(ev, cr / 16, 0) + (c / 4) * 1024 + ((c % 4) * 16 + cr % 16) * 16;
      } else {
        const int col = n0 + r;  // output feature (row of W2)
        b_ok[q] = true;
        b_ptr[q] = ev.wa + tile_off(ev, col / 16, 0) + (c / 4) * 1024 + ((c % 4) * 16 + col % 16) * 16;
      }
    }
  }

  uint4 ra[A_PER];
  uint4 rb[B_PER];
  uint32_t rasc = 0x7F7F7F7Fu, rbsc = 0x7F7F7F7Fu;

  auto load_tile = [&](int kt) {
    const int kb = kt * 128;
#pragma unroll
    for (int q = 0; q < A_PER; ++q) {
      const int c = (tid + q * 256) % 8;
      const bool kin = (kb + c * 16) < kbytes;
      ra[q] = (a_ok[q] && kin) ? ld16(a_ptr[q] + (size_t)kb) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < B_PER; ++q) {
      const int c = (tid + q * 256) % 8;
      const bool kin = (kb + c * 16) < kbytes;
      rb[q] = (b_ok[q] && kin) ? ld16(b_ptr[q] + (size_t)kt * 2048) : make_uint4(0, 0, 0, 0);
    }
    if constexpr (FMT == FMT_MX) {
      // 4 e8m0 bytes per row per K tile; blocks past the valid K read as 2^0
      const int kblk0 = kt * 4;
      const int kblk_valid = kbytes / 32;
      if (tid < BM) {
        uint32_t v = 0x7F7F7F7Fu;
        if (s_tok[tid] >= 0) {
          const uint8_t* sp;
          if (STAGE == 1)
            sp = static_cast<const uint8_t*>(p.x_s) + (size_t)s_tok[tid] * (p.H / 32) + kblk0;
          else
            sp = static_cast<uint8_t*>(p.h_s) + (size_t)(b * BM + tid) * (p.ld_h / 32) + kblk0;
          v = *reinterpret_cast<const uint32_t*>(sp);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (kblk0 + q >= kblk_valid) v = (v & ~(0xFFu << (8 * q))) | (0x7Fu << (8 * q));
        rasc = v;
      }
      if (tid < BROWS) {
        uint32_t v = 0x7F7F7F7Fu;
        // the 4 scale bytes of (row, K tile) sit 16 bytes apart in the tile
        const uint8_t* sp = nullptr;
        if (STAGE == 1) {
          const int col = n0 + (tid % BN);
          if (col < ev.width) sp = ((tid < BN) ? ev.sa : ev.sb) + scale_tile_off(ev, col / 16, kt) + col % 16;
        } else {
          const int col = n0 + tid;
          sp = ev.sa + scale_tile_off(ev, col / 16, kt) + col % 16;
        }
        if (sp) v = (uint32_t)sp[0] | ((uint32_t)sp[16] << 8) | ((uint32_t)sp[32] << 16) | ((uint32_t)sp[48] << 24);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (kblk0 + q >= kblk_valid) v = (v & ~(0xFFu << (8 * q))) | (0x7Fu << (8 * q));
        rbsc = v;
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint8_t* sA = smem + buf * (BM + BROWS) * 128;
    uint8_t* sB = sA + BM * 128;
#pragma unroll
    for (int q = 0; q < A_PER; ++q) {
      const int cid = tid + q * 256;
      if (cid < A_CH) {
        const int r = cid / 8, c = cid % 8;
        *reinterpret_cast<uint4*>(sA + swz(r, c)) = ra[q];
      }
    }
#pragma unroll
    for (int q = 0; q < B_PER; ++q) {
      const int cid = tid + q * 256;
      if (cid < B_CH) {
        const int r = cid / 8, c = cid % 8;
        *reinterpret_cast<uint4*>(sB + swz(r, c)) = rb[q];
      }
    }
    if constexpr (FMT == FMT_MX) {
      if (tid < BM) s_asc[buf][tid] = rasc;
      if (tid < BROWS) s_bsc[buf][tid] = rbsc;
    }
  };

  f32x4 acc[TI][TJ];
  f32x4 acc2[STAGE == 1 ? TI : 1][STAGE == 1 ? TJ : 1];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
  if constexpr (STAGE == 1) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc2[i][j] = f32x4{0, 0, 0, 0};
  }

  const int g = lane / 16, l16 = lane % 16;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tile(kt + 1);
    const uint8_t* sA = smem + buf * (BM + BROWS) * 128;
    const uint8_t* sB = sA + BM * 128;
    uint4 a0[TI], a1[TI];
    int sa[TI];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int r = wm * RW + i * 16 + l16;
      a0[i] = *reinterpret_cast<const uint4*>(sA + swz(r, g));
      a1[i] = *reinterpret_cast<const uint4*>(sA + swz(r, 4 + g));
      sa[i] = kFp8 ? ((FMT == FMT_MX) ? (int)((s_asc[buf][r] >> (8 * g)) & 0xFFu) : 127) : 0;
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int r = wn * CW + j * 16 + l16;
      const uint4 b0 = *reinterpret_cast<const uint4*>(sB + swz(r, g));
      const uint4 b1 = *reinterpret_cast<const uint4*>(sB + swz(r, 4 + g));
      const int sb = kFp8 ? ((FMT == FMT_MX) ? (int)((s_bsc[buf][r] >> (8 * g)) & 0xFFu) : 127) : 0;
#pragma unroll
      for (int i = 0; i < TI; ++i) mfma_tile<FMT>(acc[i][j], a0[i], a1[i], b0, b1, sa[i], sb);
      if constexpr (STAGE == 1) {
        const int ru = BN + r;
        const uint4 u0 = *reinterpret_cast<const uint4*>(sB + swz(ru, g));
        const uint4 u1 = *reinterpret_cast<const uint4*>(sB + swz(ru, 4 + g));
        const int su = kFp8 ? ((FMT == FMT_MX) ? (int)((s_bsc[buf][ru] >> (8 * g)) & 0xFFu) : 127) : 0;
#pragma unroll
        for (int i = 0; i < TI; ++i) mfma_tile<FMT>(acc2[i][j], a0[i], a1[i], u0, u1, sa[i], su);
      }
    }
    if (kt + 1 < nk) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: fp32 tile into LDS ----
  float* sT = reinterpret_cast<float*>(smem);
  constexpr int LDT = BN + 4;
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = wm * RW + i * 16 + 4 * g + v;
        const int c = wn * CW + j * 16 + l16;
        float val;
        if constexpr (STAGE == 1) {
          const float sc = s_rs[r] * ev.wscale;
          val = act_mul(acc[i][j][v] * sc + bias_at(ev.bg, n0 + c, ev.width),
                        acc2[i][j][v] * sc + bias_at(ev.bu, n0 + c, ev.width), p.act);
        } else {
          val = acc[i][j][v] * (s_rs[r] * ev.wscale) + bias_at(ev.b2, n0 + c);
        }
        sT[r * LDT + c] = val;
      }
  __syncthreads();

  if constexpr (STAGE == 1) {
    epilogue_stage1<FMT, BM, BN>(p, sT, LDT, b, n0, ev.width - n0, s_tok, tid);
  } else {
    epilogue_stage2<BM, BN>(p, sT, LDT, n0, nt, n_tiles, s_tok, s_pair, s_rw, s_done, tid);
  }
}

template <int FMT, int STAGE, int BM>
static hipError_t launch_bm(const GemmParams& p, int bn, hipStream_t s) {
  constexpr int BN = 64;
  (void)bn;
  const int width_max = (STAGE == 1) ? (p.dense ? p.I_s : p.I) : p.H;
  const int n_tiles = (width_max + BN - 1) / BN;
  dim3 grid((unsigned)(p.max_blocks * n_tiles));
  return launch_gemm_kernel(gemm_kernel<FMT, STAGE, BM, BN>, grid, dim3(256), s, p);
}

template <int FMT, int STAGE>
static hipError_t launch_fs(const GemmParams& p, int bn, hipStream_t s) {
  switch (p.block_m) {
    case 16: return launch_bm<FMT, STAGE, 16>(p, bn, s);
    case 32: return launch_bm<FMT, STAGE, 32>(p, bn, s);
    case 64: return launch_bm<FMT, STAGE, 64>(p, bn, s);
    case 128: return launch_bm<FMT, STAGE, 128>(p, bn, s);
    default: return hipErrorInvalidValue;
  }
}

template <int STAGE>
static hipError_t launch_stage(const GemmParams& p, int fmt, int bn, hipStream_t s) {
  switch (fmt) {
    case FMT_F32: return launch_fs<FMT_F32, STAGE>(p, bn, s);
    case FMT_BF16: return launch_fs<FMT_BF16, STAGE>(p, bn, s);
    case FMT_MX: return launch_fs<FMT_MX, STAGE>(p, bn, s);
    case FMT_A8W8: return launch_fs<FMT_A8W8, STAGE>(p, bn, s);
    default: return hipErrorInvalidValue;
  }
}

// A8W8 stage-2 input (per-row rule: q = e4m3_rne_sat(v * 448 / amax) over the
// bf16 values v of the row, amax their largest magnitude from stage 1): each
// row of h is quantised once, in place -- its codes go to the first ld_h bytes
// of the row's 2 ld_h-byte bf16 storage.  One wave per row, lane chunks of 8
// values in increasing order, so the codes of chunk c (bytes 8c..8c+7) only
// overwrite values of chunk c / 2, which the wave has already loaded.  Rows
// with amax = 0 (padding, empty blocks, all-zero rows) are left as they are:
// their bytes are zero or never read.
__global__ __launch_bounds__(256) void quant_rows_kernel(uint8_t* h, const float* amax, int rows, int ld_h,
                                                         const int32_t* num_blocks, int block_m) {
  constexpr int U = 4;  // chunks of 8 values per lane per round
  const int lane = threadIdx.x % kWave;
  const int nrows = num_blocks ? min(rows, *num_blocks * block_m) : rows;
  const int nchunk = ld_h / 8;
  for (int r = blockIdx.x * 4 + (int)threadIdx.x / kWave; r < nrows; r += gridDim.x * 4) {
    const float a = amax[r];
    if (!(a > 0.f)) continue;
    const float inv = __fdiv_rn(448.0f, a);
    uint8_t* row = h + (size_t)r * ld_h * 2;
    for (int base = 0; base < nchunk; base += U * kWave) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = base + u * kWave + lane;
        v[u] = c < nchunk ? *reinterpret_cast<const uint4*>(row + (size_t)c * 16) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = base + u * kWave + lane;
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        uint32_t o[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
          o[t] = pack4_e4m3(bf16_to_f32(w[2 * t] & 0xFFFFu) * inv, bf16_to_f32(w[2 * t] >> 16) * inv,
                            bf16_to_f32(w[2 * t + 1] & 0xFFFFu) * inv, bf16_to_f32(w[2 * t + 1] >> 16) * inv);
        if (c < nchunk) *reinterpret_cast<uint2*>(row + (size_t)c * 8) = make_uint2(o[0], o[1]);
      }
    }
  }
}

hipError_t launch_quant_rows(const GemmParams& p, hipStream_t s) {
  const int rows = p.max_blocks * p.block_m;
  const int32_t* nblk = (p.dense || p.self_sort) ? nullptr : p.num_blocks;
  int grid = (rows + 3) / 4;
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(quant_rows_kernel, dim3(grid), dim3(256), 0, s, p.h, static_cast<const float*>(p.h_s), rows,
                     p.ld_h, nblk, p.block_m);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmParams& p, int stage, int fmt, int bn, hipStream_t s) {
  if (stage == 2 && fmt == FMT_A8W8) {
    const hipError_t e = launch_quant_rows(p, s);
    if (e != hipSuccess) return e;
  }
  // 16-row blocks: weights and activations streamed straight into registers,
  // one wave per 32 (stage 1) or 64 (stage 2) columns of a block
  if (p.block_m == 16 && wave_kernel_fits(p, stage, fmt)) return launch_gemm_wave(p, stage, fmt, s);
  if (p.self_sort) return hipErrorInvalidValue;  // only the one-wave kernels scan the ids
  // 256-row sorted blocks: both operands through LDS, eight waves
  if (p.block_m == 256) return lds_kernel_fits(p, stage, fmt) ? launch_gemm_lds(p, stage, fmt, s) : hipErrorInvalidValue;
  // 32-128-row blocks: weights streamed into registers, token rows through LDS.
  // The stage-2 reduction runs 128-row sorted blocks as two 64-row halves
  // (more workgroups per CU; measured faster on MI355X).
  if (tile_kernel_fits(p, stage, fmt)) {
    if (stage == 2 && p.mode != 0 && !p.dense && p.block_m == 128) {
      GemmParams q = p;
      q.block_m = 64;
      q.max_blocks = p.max_blocks * 2;
      q.bsplit = 2;
      return launch_gemm_tile(q, stage, fmt, s);
    }
    return launch_gemm_tile(p, stage, fmt, s);
  }
  if (fmt == FMT_MX4) return hipErrorInvalidValue;  // e2m1 weights: one-wave and tiled kernels only
  return stage == 1 ? launch_stage<1>(p, fmt, bn, s) : launch_stage<2>(p, fmt, bn, s);
}

}  // namespace moe
