// Two-stage routed grouped GEMM for gfx950 (MFMA, LDS-staged tiles).
//
// Stage 1 (vLLM PR 65207, "Purpose", commit 2 names the AITER stages): for
// each sorted block of rows owned by expert e, a = x_gathered . W13[e]^T with
// fp32 accumulation; the per-token and per-expert scales multiply the fp32
// accumulator before the activation (AITER PR 6106, "Technical Details"),
// MX-32 block scales are applied by the block-scaled MFMA inside the K loop;
// the epilogue computes h = SiLU(a_gate) * a_up and rounds / quantises it to
// the stage-2 input format (bf16, MX-32 e4m3, or bf16 plus a per-row amax
// from which stage 2 derives the per-row e4m3 scale).
//
// Stage 2: o = h . W2[e]^T, times the scales; the epilogue adds pair_w * o
// into the fp32 accumulator, which already holds the shared-expert addend
// when the shared expert ran on the aux stream (vLLM PR 65207, commit 2: the
// shared output is accumulated in the stage-2 epilogue instead of by a
// separate add), and the last of the expected contributions to a
// (token, column tile) rounds the fp32 sum once into the output.  In STORE
// mode (dense shared expert) it writes gamma_t * o into the accumulator.
//
// Tiles: 256 threads = 4 waves; BM sorted rows x BN output columns; the K tile
// is 128 bytes of the operand format (32 fp32, 64 bf16 or 128 fp8 elements).
// Operands live in LDS as 128-byte rows of eight 16-byte chunks, XOR-swizzled
// by row.  In every 128-byte K tile, lane group g = lane/16 feeds chunks g and
// 4+g to the MFMA; this matches the gfx950 16x16x128 f8f6f4 operand order
// (bytes 0-15 = K 16g.., bytes 16-31 = K 64+16g..) and the 32-element MX
// blocks, and for the other formats it is a consistent permutation of K on
// both operands.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

template <int FMT>
struct FmtInfo;
template <>
struct FmtInfo<FMT_F32> { static constexpr int esz = 4; static constexpr bool fp8 = false; };
template <>
struct FmtInfo<FMT_BF16> { static constexpr int esz = 2; static constexpr bool fp8 = false; };
template <>
struct FmtInfo<FMT_MX> { static constexpr int esz = 1; static constexpr bool fp8 = true; };
template <>
struct FmtInfo<FMT_A8W8> { static constexpr int esz = 1; static constexpr bool fp8 = true; };

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

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
  } else {
    i32x8 A = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    i32x8 B = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 0, 0, 0, sa, 0, sb);
  }
}

// Per-block problem description resolved from the expert index.
struct ExpertView {
  const uint8_t* wa;   // stage 1: gate rows; stage 2: W2 rows
  const uint8_t* wb;   // stage 1: up rows
  const uint8_t* sa;   // MX scales of wa rows
  const uint8_t* sb;   // MX scales of wb rows
  int ldw;             // weight row stride (elements)
  int ldsc;            // MX scale row stride (bytes)
  int width;           // stage 1: valid h columns; stage 2: valid K (h columns)
  float wscale;        // A8W8 per-expert scale
};

template <int FMT, int STAGE>
__device__ __forceinline__ ExpertView resolve_expert(const GemmParams& p, int e) {
  constexpr int esz = FmtInfo<FMT>::esz;
  ExpertView v{};
  v.wscale = 1.0f;
  const int H = p.H, I = p.I, Is = p.I_s;
  if (e >= 0 && e < p.E) {
    if (STAGE == 1) {
      v.wa = p.w13 + (size_t)e * 2 * I * H * esz;
      v.wb = v.wa + (size_t)I * H * esz;
      v.ldw = H;
      v.width = I;
      if (FMT == FMT_MX) {
        v.sa = static_cast<const uint8_t*>(p.w13_s) + (size_t)e * 2 * I * (H / 32);
        v.sb = v.sa + (size_t)I * (H / 32);
        v.ldsc = H / 32;
      }
      if (FMT == FMT_A8W8) v.wscale = static_cast<const float*>(p.w13_s)[e];
    } else {
      v.wa = p.w2 + (size_t)e * H * I * esz;
      v.ldw = I;
      v.width = I;
      if (FMT == FMT_MX) {
        v.sa = static_cast<const uint8_t*>(p.w2_s) + (size_t)e * H * (I / 32);
        v.ldsc = I / 32;
      }
      if (FMT == FMT_A8W8) v.wscale = static_cast<const float*>(p.w2_s)[e];
    }
  } else {
    // shared expert: whole (e < 0, dense) or pseudo-expert chunk c = e - E
    const int c = (e < 0) ? 0 : e - p.E;
    const int col0 = (e < 0) ? 0 : c * I;
    const int w = (e < 0) ? Is : min(I, Is - col0);
    if (STAGE == 1) {
      v.wa = p.ws13 + (size_t)col0 * H * esz;
      v.wb = p.ws13 + (size_t)(Is + col0) * H * esz;
      v.ldw = H;
      v.width = w;
      if (FMT == FMT_MX) {
        v.sa = static_cast<const uint8_t*>(p.ws13_s) + (size_t)col0 * (H / 32);
        v.sb = static_cast<const uint8_t*>(p.ws13_s) + (size_t)(Is + col0) * (H / 32);
        v.ldsc = H / 32;
      }
      if (FMT == FMT_A8W8) v.wscale = static_cast<const float*>(p.ws13_s)[0];
    } else {
      v.wa = p.ws2 + (size_t)col0 * esz;
      v.ldw = Is;
      v.width = w;
      if (FMT == FMT_MX) {
        v.sa = static_cast<const uint8_t*>(p.ws2_s) + col0 / 32;
        v.ldsc = Is / 32;
      }
      if (FMT == FMT_A8W8) v.wscale = static_cast<const float*>(p.ws2_s)[0];
    }
  }
  return v;
}

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
  // stage-2 A8W8 reads bf16 h and quantises it while staging into LDS
  constexpr bool kQuantA = (STAGE == 2 && FMT == FMT_A8W8);
  constexpr int A_GMUL = kQuantA ? 2 : 1;
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
  __shared__ float s_inv[BM];  // stage 2 A8W8: 448 / amax
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
    float rs = 1.0f, inv = 0.f;
    if (FMT == FMT_A8W8) {
      if (STAGE == 1) {
        rs = tok >= 0 ? static_cast<const float*>(p.x_s)[tok] : 0.f;
      } else {
        const float amax = static_cast<const float*>(p.h_s)[slot];
        if (amax > 0.f) {
          inv = __fdiv_rn(448.0f, amax);
          rs = __fdiv_rn(amax, 448.0f);
        }
      }
    }
    s_rs[tid] = rs;
    s_inv[tid] = inv;
  }
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
        a_ptr[q] = p.h + ((size_t)slot * p.ld_h * esz + c * 16) * A_GMUL;
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
      if (STAGE == 1) {
        const int col = n0 + (r % BN);
        b_ok[q] = col < ev.width;
        const uint8_t* base = (r < BN) ? ev.wa : ev.wb;
        b_ptr[q] = base + ((size_t)(b_ok[q] ? col : 0) * ev.ldw * esz + c * 16);
      } else {
        const int col = n0 + r;  // output feature (row of W2)
        b_ok[q] = true;
        b_ptr[q] = ev.wa + ((size_t)col * ev.ldw * esz + c * 16);
      }
    }
  }

  uint4 ra[A_PER][A_GMUL];
  uint4 rb[B_PER];
  uint32_t rasc = 0x7F7F7F7Fu, rbsc = 0x7F7F7F7Fu;

  auto load_tile = [&](int kt) {
    const int kb = kt * 128;
#pragma unroll
    for (int q = 0; q < A_PER; ++q) {
      const int c = (tid + q * 256) % 8;
      const bool kin = (kb + c * 16) < kbytes;
#pragma unroll
      for (int u = 0; u < A_GMUL; ++u) {
        ra[q][u] = (a_ok[q] && kin) ? ld16(a_ptr[q] + (size_t)kb * A_GMUL + u * 16) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int q = 0; q < B_PER; ++q) {
      const int c = (tid + q * 256) % 8;
      const bool kin = (kb + c * 16) < kbytes;
      rb[q] = (b_ok[q] && kin) ? ld16(b_ptr[q] + kb) : make_uint4(0, 0, 0, 0);
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
        if (STAGE == 1) {
          const int col = n0 + (tid % BN);
          if (col < ev.width) {
            const uint8_t* base = (tid < BN) ? ev.sa : ev.sb;
            v = *reinterpret_cast<const uint32_t*>(base + (size_t)col * ev.ldsc + kblk0);
          }
        } else {
          v = *reinterpret_cast<const uint32_t*>(ev.sa + (size_t)(n0 + tid) * ev.ldsc + kblk0);
        }
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
        uint4 v;
        if constexpr (kQuantA) {
          const float inv = s_inv[r];
          const uint32_t w[8] = {ra[q][0].x, ra[q][0].y, ra[q][0].z, ra[q][0].w,
                                 ra[q][1].x, ra[q][1].y, ra[q][1].z, ra[q][1].w};
          uint32_t o[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            o[u] = pack4_e4m3(bf16_to_f32(w[2 * u] & 0xFFFFu) * inv, bf16_to_f32(w[2 * u] >> 16) * inv,
                              bf16_to_f32(w[2 * u + 1] & 0xFFFFu) * inv, bf16_to_f32(w[2 * u + 1] >> 16) * inv);
          v = make_uint4(o[0], o[1], o[2], o[3]);
        } else {
          v = ra[q][0];
        }
        *reinterpret_cast<uint4*>(sA + swz(r, c)) = v;
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
          val = silu_mul(acc[i][j][v] * sc, acc2[i][j][v] * sc);
        } else {
          val = acc[i][j][v] * (s_rs[r] * ev.wscale);
        }
        sT[r * LDT + c] = val;
      }
  __syncthreads();

  if constexpr (STAGE == 1) {
    const int ncol_valid = ev.width - n0;  // > 0
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
  } else {
    // ---- stage 2: STORE (dense addend) or per-pair rows + last-arrival sum ----
    if (p.mode == 0) {
      for (int r = wv; r < BM; r += 4) {
        const int tok = s_tok[r];
        if (tok < 0) continue;
        const float wgt = s_rw[r];
        float* dst = p.acc + (size_t)tok * p.H + n0;
        for (int c = lane; c < BN; c += kWave) dst[c] = wgt * sT[r * LDT + c];
      }
    } else {
      // Each (token, slot) pair owns one row of the pair buffer; rows are
      // written with device-coherent stores so that whichever workgroup
      // completes a (token, column tile) last can read them from any XCD.
      for (int r = wv; r < BM; r += 4) {
        const int pair = s_pair[r];
        if (pair < 0) continue;
        const float wgt = s_rw[r];
        float* dst = p.pair_out + (size_t)pair * p.H + n0;
        for (int c = lane; c < BN; c += kWave)
          __hip_atomic_store(dst + c, wgt * sT[r * LDT + c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      // The counter increment only has to wait until this workgroup's row
      // stores are acknowledged (they are coherent by themselves); an
      // agent-scope fence would also write back and invalidate the XCD's L2.
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
  }
}

template <int FMT, int STAGE, int BM>
static hipError_t launch_bm(const GemmParams& p, int bn, hipStream_t s) {
  constexpr int BN = 64;
  (void)bn;
  const int width_max = (STAGE == 1) ? (p.dense ? p.I_s : p.I) : p.H;
  const int n_tiles = (width_max + BN - 1) / BN;
  dim3 grid((unsigned)(p.max_blocks * n_tiles));
  hipLaunchKernelGGL((gemm_kernel<FMT, STAGE, BM, BN>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
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

hipError_t launch_gemm(const GemmParams& p, int stage, int fmt, int bn, hipStream_t s) {
  return stage == 1 ? launch_stage<1>(p, fmt, bn, s) : launch_stage<2>(p, fmt, bn, s);
}

}  // namespace moe
