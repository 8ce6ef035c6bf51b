// Grouped GEMM for sorted blocks of 32-128 rows (gfx950), both stages.
//
// Stage 1 computes a = x_gathered . W13[e]^T, applies the per-token and
// per-expert scales to the fp32 accumulator (MX-32 block scales inside the
// block-scaled MFMA), adds the expert's bias, then h = act(a_gate) * a_up
// (SiLU or GELU), rounded or quantised to
// the stage-2 input format (AITER PR 6106, "Technical Details"; vLLM PR 65207,
// "Purpose", commit 2 for the two-stage structure).  Stage 2 computes
// o = h . W2[e]^T with the same scale rules and hands the weighted pair rows to
// the deterministic last-arrival reduction onto the shared-expert addend
// (vLLM PR 65207, commit 2: the shared output is accumulated in stage 2), or in
// STORE mode writes gamma_t * o as the dense addend.
//
// Mapping.  The expert weights are the MFMA "A" operand (M = weight rows) and
// the block's tokens the "B" operand (N = tokens).  The tiled weight layout
// (16-row x 128-byte tiles, two 1 KiB halves in operand order) means one wave
// loads a 16-row fragment of a K tile as two contiguous 1 KiB reads straight
// into MFMA operand registers: weights never pass through LDS, and no two
// waves load the same weight bytes.  The gathered token rows are shared by the
// four waves, so they are staged through LDS, double buffered.  Each lane
// loads one 16-byte chunk and eight consecutive lanes one row's whole
// 128-byte K tile (a wave touches eight full cache lines; reading 64 bytes
// of sixteen rows instead costs measurably more L1/L2 traffic).  In LDS a
// 16-row x 128-byte fragment is 2 KiB in operand order (chunk c of row r at
// (c / 4) * 1024 + (c % 4) * 256 + 16 * slot) with the row slot XOR-swizzled,
// slot = r ^ c ^ 8 (r & 1), so that the row-wise writes and the
// operand-order ds_read_b128 fragment reads are both free of bank conflicts.
//
// Workgroup = 4 waves x 64 weight rows: in stage 1 a wave owns 32 h columns
// (32 gate rows + the matching 32 up rows, so SiLU-mul happens in registers),
// in stage 2 one 64-column reduction tile.  Per wave and K tile (128 bytes of
// K): 8 x 16 B weight loads per lane issued one tile ahead, 2 x NB fragment
// reads from LDS, and 4 x NB MFMA tiles.
//
// Placement.  Workgroups are dealt round-robin to the eight XCDs.  Stage 1
// remaps launch order so that consecutive logical tiles share one XCD's L2;
// with the experts' row offsets at hand the logical order is expert-major
// (the blocks of one weight column tile side by side), else block-major.  The
// stage-2 queues below take the same expert-major order.
// Stage 2 (ACCUMULATE) runs persistent workgroups that take work from one
// queue per XCD: queue x holds the 64-column reduction tiles t = x (mod 8) of
// every block, and a workgroup reads the XCD it actually runs on from the
// XCC_ID hardware register, so every writer and the last-arrival reader of a
// (token, tile) run on the same XCD.  Their pair rows then meet in that XCD's
// L2 with ordinary stores and loads; cross-XCD coherence is needed only for
// the counters (device-scope atomics).  A queue is claimed by the first XCD
// that touches it; an XCD whose own workgroups never arrive has its queue
// claimed and drained by another, which keeps the property.
#include "tile_common.hpp"

namespace moe {

constexpr int kTileThreads = 256;

// Row tables of block b: the token and pair of each row go to LDS; the
// row's epilogue factors (stage-2 pair weight, A8W8 row scale) stay in the
// loading thread's registers (tid < BM) until the epilogue, so no load of
// the K loop waits behind them.
template <int FMT, int STAGE, int BM>
__device__ __forceinline__ bool tile_rows(const GemmParams& p, int b, int tid, int* s_tok, int* s_pair, float& rw,
                                          float& rs) {
  const int P = p.T * p.k_total;
  rw = 0.f;
  rs = 1.0f;
  bool live = false;
  if (tid < BM) {
    const int slot = b * BM + tid;
    int tok = -1, pair = -1;
    if (p.dense) {
      tok = slot < p.T ? slot : -1;
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
    live = tok >= 0;
    if (FMT == FMT_A8W8) {
      if (STAGE == 1) {
        rs = tok >= 0 ? static_cast<const float*>(p.x_s)[tok] : 0.f;
      } else {
        const float amax = static_cast<const float*>(p.h_s)[slot];
        if (amax > 0.f) rs = __fdiv_rn(amax, 448.0f);
      }
    }
  }
  return live;
}

template <int BM>
struct TileSmem {
  // staged token rows, swizzled operand order; after the K loop each wave's
  // 4 KiB of it stages the stage-2 pair-row codes of 32 rows
  uint8_t x[2][(BM < 64 ? 64 : BM) * 128];
  uint32_t xsc[2][BM + 1];  // MX: the rows' e8m0 scales of the staged K tile, + a spare slot
  int tok[BM];
  int pair[BM];
  float rw[BM];   // stage 2: pair weight / gate
  float rs[BM];   // row scale (stage 1 A8W8: x scale; stage 2 A8W8: h row scale)
  int item;       // persistent stage 2: the claimed work item / queue
  uint64_t done[(BM + 63) / 64];  // stage 2, counted per group: rows whose count completed
};

// LDS offset of 16-byte chunk c (0..7) of row r (0..15) in a staged 16-row
// fragment: operand order, row slot XOR-swizzled.  For a fixed row the eight
// chunks land in eight different 16-byte bank groups (and rows r, r + 1 in
// the other eight), and for a fixed chunk the sixteen rows in sixteen.
__device__ __forceinline__ int lds_chunk_off(int r, int c) {
  return (c / 4) * 1024 + (c % 4) * 256 + ((r ^ c ^ ((r & 1) << 3)) & 15) * 16;
}

// One block b of expert view ev: this wave's columns start at c0 (stage 1: h
// columns c0..c0+31; stage 2: output columns c0..c0+63); waves with
// wave_ok = false take part in the staging and barriers but store nothing.
// Starts by filling the row tables (the caller synchronises before reusing
// the shared memory).
template <int FMT, int STAGE, int NB, bool EPI>
__device__ __forceinline__ void tile_block(const GemmParams& p, TileSmem<16 * NB>& sm, int b, const ExpertView& ev,
                                           int c0, bool wave_ok, int cslot, bool group_count) {
  constexpr int esz = FmtInfo<FMT>::esz;
  constexpr int BM = 16 * NB;                                // sorted rows of a block
  constexpr int CPT = NB / 2;                                // staged 16-byte chunks per thread per K tile
  // bf16 runs on 32x32x16 MFMA tiles (the 16x16x32 form issues at half the
  // rate on gfx950); the fp8 formats on the block-scaled 16x16x128 form
  constexpr bool k32 = (FMT == FMT_BF16);
  constexpr int NN = NB / 2;  // 32-row token groups of a block (k32)

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int g = lane / 16, l16 = lane % 16;

  // K extent in bytes of the staged (MFMA) format; a multiple of 128
  const int kbytes = (STAGE == 1) ? p.H * esz : ev.width * esz;
  const int nk = kbytes / 128;

  // ---- this wave's weight fragments: 4 row blocks of 16, addressed as
  // (uniform tile offset, lane * 16) in a buffer over the matrix ----
  __amdgpu_buffer_rsrc_t wrs[2], srs[2];
  uint32_t wtile[4], stile[4];
  wrs[0] = tile_rsrc(ev.wa, 0x7FFFFFFF);
  wrs[1] = tile_rsrc((STAGE == 1) ? ev.wb : ev.wa, 0x7FFFFFFF);
  if constexpr (fmt_mx(FMT)) {
    srs[0] = tile_rsrc(ev.sa, 0x7FFFFFFF);
    srs[1] = tile_rsrc((STAGE == 1) ? ev.sb : ev.sa, 0x7FFFFFFF);
  }
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    // 16-row blocks (stage 1: gate rows c0.., c0+16.. then the same up rows);
    // k32: 32-row blocks, stage 1 gate rows c0.. and up rows c0.., stage 2
    // rows c0.. and c0+32..
    int rb = (STAGE == 1) ? c0 / 16 + (mb & 1) : c0 / 16 + mb;
    if (k32) rb = (STAGE == 1) ? c0 / 16 : c0 / 16 + 2 * (mb & 1);
    wtile[mb] = (uint32_t)tile_off(ev, rb, 0);
    stile[mb] = (uint32_t)scale_tile_off(ev, rb, 0);
  }
  // 16x16 operands: lane (g, r) reads chunk position lane of each 1 KiB half.
  // k32: lane l takes row l % 32 (tile row block (l % 32) / 16, row l % 16)
  // and, at K step s of 16 elements, the 16-byte chunk 2s + l / 32 of the
  // 128-byte K tile, which sits at 512 s + 16 (16 (l / 32) + l % 16) in the
  // tile: two contiguous 512-byte runs per row block and step.
  const uint32_t kfrag32 = (uint32_t)(((lane / 32) * 16 + l16) * 16);
  const uint32_t wlane = k32 ? (uint32_t)(((lane % 32) / 16) * ev.nkt * 2048) + kfrag32 : (uint32_t)lane * 16;

  int live = 0;  // real rows of the block (set once its row tables are read)

  // ---- staged token rows: chunk q = tid + 256 u is chunk q % 8 of row q / 8;
  // padding rows read past the buffer ----
  __amdgpu_buffer_rsrc_t xrs, xsrs;
  if (STAGE == 1) {
    xrs = tile_rsrc(p.x, (uint32_t)((size_t)p.T * p.H * esz));
    if constexpr (fmt_mx(FMT)) xsrs = tile_rsrc(p.x_s, (uint32_t)((size_t)p.T * (p.H / 32)));
  } else {
    const size_t rows = (size_t)p.max_blocks * BM;
    xrs = tile_rsrc(p.h, (uint32_t)(rows * h_row_bytes<FMT>(p)));
    if constexpr (fmt_mx(FMT)) xsrs = tile_rsrc(p.h_s, (uint32_t)(rows * (p.ld_h / 32)));
  }
  // LDS offset of chunk u: row tid / 8 + 32 u sits two 16-row fragments
  // (4 KiB) further on per u, with the same swizzle
  const uint32_t soff = (uint32_t)(lds_chunk_off((tid / 8) % 16, tid % 8) + (tid / 128) * 2048);
  // buffer offsets of the thread's chunks (set once the row tables are in LDS)
  uint32_t xoff[CPT];
  uint32_t xsoff = kTileOutOfRange;  // the row's e8m0 scales (MX), for threads tid < BM
  auto row_offsets = [&]() {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int q = tid + kTileThreads * u;
      const int r = q / 8;
      const int c = q % 8;  // 16-byte chunk of the 128-byte K tile
      const int tok = sm.tok[r];
      if (tok < 0) {
        xoff[u] = kTileOutOfRange;
      } else if (STAGE == 1) {
        xoff[u] = (uint32_t)((size_t)tok * p.H * esz) + c * 16;
      } else {
        xoff[u] = (uint32_t)(((size_t)b * BM + r) * h_row_bytes<FMT>(p)) + c * 16;
      }
    }
    if (fmt_mx(FMT) && tid < BM && sm.tok[tid] >= 0)
      xsoff = (STAGE == 1) ? (uint32_t)(sm.tok[tid] * (p.H / 32)) : (uint32_t)((b * BM + tid) * (p.ld_h / 32));
  };

  auto load_w = [&](uint4 (&w)[4][2], int (&sc)[4], int kt) {
    kt = kt < nk ? kt : nk - 1;  // past the end: a harmless reload of the last tile
    if constexpr (k32) {
      // w[2 mm + s / 2][s % 2]: M block mm, K step s
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const __amdgpu_buffer_rsrc_t r = wrs[(STAGE == 1) ? mm : 0];
        const uint32_t so = wtile[mm] + (uint32_t)(kt * ev.tb);
#pragma unroll
        for (int st = 0; st < 4; ++st) w[2 * mm + st / 2][st % 2] = tile_load16(r, wlane + 512 * st, so);
        sc[2 * mm] = sc[2 * mm + 1] = 127;
      }
      return;
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const __amdgpu_buffer_rsrc_t r = wrs[mb >> 1];
      const uint32_t so = wtile[mb] + (uint32_t)(kt * ev.tb);
      w[mb][0] = tile_load16(r, wlane, so);
      // MXFP4: one 1 KiB half per tile (lane (g, r): 32 e2m1 values)
      w[mb][1] = FMT == FMT_MX4 ? make_uint4(0, 0, 0, 0) : tile_load16(r, wlane + 1024, so);
      if constexpr (fmt_mx(FMT))
        sc[mb] = (int)__builtin_amdgcn_raw_buffer_load_b8(srs[mb >> 1], (int)lane, (int)(stile[mb] + kt * 64), 0);
      else
        sc[mb] = 127;
    }
  };

  // token-row register sets in flight: XD = 2 keeps the rows of K tiles
  // kt + 1 and kt + 2 loading while tile kt is multiplied
  constexpr int XD =
      (((FMT == FMT_A8W8 || FMT == FMT_BF16) && STAGE == 1 && NB == 8) || (FMT == FMT_A8W8 && STAGE == 2 && NB == 4))
          ? 1
          : 2;
  uint4 xr[XD][CPT];
  uint32_t xsr[XD] = {};
  auto load_x = [&](int set, int kt) {
    kt = kt < nk ? kt : nk - 1;
#pragma unroll
    for (int u = 0; u < CPT; ++u)
      xr[set][u] = tile_load16(xrs, xoff[u], (uint32_t)kt * 128);
    if constexpr (fmt_mx(FMT)) {
      xsr[set] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(xsrs, (int)xsoff, kt * 4, 0);  // tid >= BM: reads 0
    }
  };
  auto store_x = [&](int buf, int set) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      *reinterpret_cast<uint4*>(&sm.x[buf][soff + 4096 * u]) = xr[set][u];
    }
    if constexpr (fmt_mx(FMT)) {
      sm.xsc[buf][tid < BM ? tid : BM] = xsr[set];  // no branch: the other threads write the spare slot
    }
  };

  // one of the two accumulator sets is used (the other is dead code)
  f32x4 acc[4][NB];
  f32x16 acc32[2][NN];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int mm = 0; mm < 2; ++mm)
#pragma unroll
    for (int nn = 0; nn < NN; ++nn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc32[mm][nn][v] = 0.f;
  // k32 token fragment of lane l at K step st: row l % 16 of row block
  // (l % 32) / 16 of a 32-row group, chunk 2 st + l / 32; the swizzle of step
  // st is that of step 0 with slot bits 1-2 flipped (XOR 32 st on the offset)
  const uint32_t xfrag32 = (uint32_t)(((lane % 32) / 16) * 2048 + lds_chunk_off(l16, lane / 32));
  auto xf32 = [&](int st) { return (xfrag32 ^ (uint32_t)(32 * st)) + (uint32_t)(512 * st); };
  // 16x16 operands: lane (g, r) takes chunks g and 4 + g of row r
  const uint32_t xo0 = (uint32_t)lds_chunk_off(l16, g), xo1 = (uint32_t)lds_chunk_off(l16, 4 + g);

  // The multiply of a K tile runs at raised wave priority, so a wave with its
  // operands ready keeps the matrix core busy ahead of the SIMD's other wave
  // issuing loads (measured: a8w8 stage 1 -5 %, bf16 and MX unchanged).
  // k32: four K steps of 16; consecutive MFMAs update different accumulators
  auto compute_k32 = [&](int buf, const uint4 (&w)[4][2]) {
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int nn = 0; nn < NN; ++nn) {
        const uint4 bf = *reinterpret_cast<const uint4*>(&sm.x[buf][nn * 4096 + xf32(st)]);
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
          acc32[mm][nn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, w[2 * mm + st / 2][st % 2]), __builtin_bit_cast(bf16x8, bf), acc32[mm][nn],
              0, 0, 0);
      }
  };
  auto compute = [&](int buf, const uint4 (&w)[4][2], const int (&sc)[4]) {
    __builtin_amdgcn_s_setprio(1);
    if constexpr (k32 && STAGE == 1) {
      {
        // four K steps of 16; the token fragments of step st + 1 are read
        // while step st multiplies (LDS latency behind eight MFMAs); the
        // scheduling groups pin that order (the default schedule reads each
        // fragment just before its two MFMAs and exposes the LDS latency)
        __builtin_amdgcn_sched_barrier(0);
        uint4 bf[2][NN];
#pragma unroll
        for (int nn = 0; nn < NN; ++nn)
          bf[0][nn] = *reinterpret_cast<const uint4*>(&sm.x[buf][nn * 4096 + xf32(0)]);
        __builtin_amdgcn_sched_group_barrier(0x100, NN, 0);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          if (st < 3) {
#pragma unroll
            for (int nn = 0; nn < NN; ++nn)
              bf[(st + 1) & 1][nn] = *reinterpret_cast<const uint4*>(&sm.x[buf][nn * 4096 + xf32(st + 1)]);
            __builtin_amdgcn_sched_group_barrier(0x100, NN, 0);
          }
#pragma unroll
          for (int nn = 0; nn < NN; ++nn)
#pragma unroll
            for (int mm = 0; mm < 2; ++mm)
              acc32[mm][nn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, w[2 * mm + st / 2][st % 2]), __builtin_bit_cast(bf16x8, bf[st & 1][nn]),
                  acc32[mm][nn], 0, 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * NN, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (k32) {
      compute_k32(buf, w);
    } else {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint4 b0 = *reinterpret_cast<const uint4*>(&sm.x[buf][nb * 2048 + xo0]);
        const uint4 b1 = *reinterpret_cast<const uint4*>(&sm.x[buf][nb * 2048 + xo1]);
        const int sb = (fmt_mx(FMT)) ? (int)((sm.xsc[buf][nb * 16 + l16] >> (8 * g)) & 0xFFu) : 127;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) mfma_tile<FMT>(acc[mb][nb], w[mb][0], w[mb][1], b0, b1, sc[mb], sb);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Two weight register sets and two LDS buffers in ping-pong: while K tile
  // kt is multiplied, the weights of kt + 1 are in flight (issued one step
  // earlier) and the token rows of kt + 1 (XD = 1) or of kt + 1 and kt + 2
  // (XD = 2, register set = tile parity) are loading; after the multiply the
  // rows of kt + 1 are staged into the other LDS buffer.  Every step is
  // unconditional; loads past the end reload the last tile.
  // The weights of the first two K tiles depend only on the expert and the
  // columns, so they are in flight before the row tables are read; the
  // token rows follow once the tables are in LDS.
  uint4 wA[4][2], wB[4][2];
  int sA[4], sB[4];
  load_w(wA, sA, 0);
  load_w(wB, sB, 1);
  float rw_row, rs_row;
  // a block's real rows come first and its padding last
  live = __syncthreads_count(tile_rows<FMT, STAGE, BM>(p, b, tid, sm.tok, sm.pair, rw_row, rs_row));
  if (live == 0) return;  // a block part holding only padding rows
  row_offsets();
  if constexpr (XD == 2) {
    load_x(0, 0);
    load_x(1, 1);
    store_x(0, 0);
    load_x(0, 2);
  } else {
    load_x(0, 0);
    store_x(0, 0);
  }
  __syncthreads();
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {
    if constexpr (XD == 1) load_x(0, kt + 1);
    compute(0, wA, sA);
    load_w(wA, sA, kt + 2);
    store_x(1, XD - 1);
    if constexpr (XD == 2) load_x(1, kt + 3);
    __syncthreads();
    if constexpr (XD == 1) load_x(0, kt + 2);
    compute(1, wB, sB);
    load_w(wB, sB, kt + 3);
    store_x(0, 0);
    if constexpr (XD == 2) load_x(0, kt + 4);
    __syncthreads();
  }
  if (kt < nk) compute(0, wA, sA);  // odd tile count: the last tile sits in buffer 0 / set A
  if (tid < BM) {
    sm.rw[tid] = rw_row;
    sm.rs[tid] = rs_row;
  }
  __syncthreads();

  // ---- epilogues (per wave, from registers) ----
  // acc[mb][nb][v] = row (mb, 4g + v) of the wave's weight rows x token row nb*16 + l16
  // (counted per group: every wave takes part in the count)
  if (!wave_ok && !(k32 && STAGE == 2 && p.mode != 0 && group_count)) return;
  // k32: acc32[mm][nn][4 j + v] = weight row 8 j + 4 (l / 32) + v of M block
  // mm x token row nn * 32 + l % 32
  if constexpr (STAGE == 1 && k32) {
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) {
      const int r = nn * 32 + lane % 32;
      if (sm.tok[r] < 0) continue;
      const size_t slot = (size_t)b * BM + r;
      const float sc = sm.rs[r] * ev.wscale;
      uint16_t* dst = reinterpret_cast<uint16_t*>(p.h) + slot * p.ld_h + c0 + 4 * (lane / 32);
      const int cb = c0 + 4 * (lane / 32);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t bits[4];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          bits[v] = f32_to_bf16(epi_act<EPI>(acc32[0][nn][4 * j + v] * sc + epi_bias<EPI>(ev.bg, cb + 8 * j + v, ev.width),
                                        acc32[1][nn][4 * j + v] * sc + epi_bias<EPI>(ev.bu, cb + 8 * j + v, ev.width),
                                        p.act));
        *reinterpret_cast<uint2*>(dst + 8 * j) = make_uint2(bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16));
      }
    }
  } else if constexpr (STAGE == 1) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int r = nb * 16 + l16;
      const int tok = sm.tok[r];
      const size_t slot = (size_t)b * BM + r;
      const float sc = sm.rs[r] * ev.wscale;
      float hv[2][4];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int col = c0 + 4 * g + 16 * m + v;
          hv[m][v] = epi_act<EPI>(acc[m][nb][v] * sc + epi_bias<EPI>(ev.bg, col, ev.width),
                             acc[m + 2][nb][v] * sc + epi_bias<EPI>(ev.bu, col, ev.width), p.act);
        }
      if constexpr (fmt_mx(FMT)) {
        // the wave's 32 columns are one MX-32 block of the token's h row
        float amax = 0.f;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            hv[m][v] = bf16_to_f32(f32_to_bf16(hv[m][v]));
            amax = fmaxf(amax, fabsf(hv[m][v]));
          }
        amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
        amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
        const int eb = (int)((__float_as_uint(amax) >> 23) & 0xFF);
        int X = (eb == 0) ? -127 : (eb - 127 - 8);
        X = X < -127 ? -127 : (X > 127 ? 127 : X);
        const float mul = __builtin_ldexpf(1.0f, -X);
        if (tok >= 0) {
          uint8_t* dst = p.h + slot * p.ld_h + c0 + 4 * g;
#pragma unroll
          for (int m = 0; m < 2; ++m)
            *reinterpret_cast<uint32_t*>(dst + 16 * m) =
                pack4_e4m3(hv[m][0] * mul, hv[m][1] * mul, hv[m][2] * mul, hv[m][3] * mul);
          if (g == 0) static_cast<uint8_t*>(p.h_s)[slot * (p.ld_h / 32) + c0 / 32] = (uint8_t)(X + 127);
        }
      } else {
        float amax = 0.f;
        uint32_t bits[2][4];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            bits[m][v] = f32_to_bf16(hv[m][v]);
            amax = fmaxf(amax, fabsf(bf16_to_f32(bits[m][v])));
          }
        if (tok >= 0) {
          uint16_t* dst = reinterpret_cast<uint16_t*>(p.h) + slot * p.ld_h + c0 + 4 * g;
#pragma unroll
          for (int m = 0; m < 2; ++m)
            *reinterpret_cast<uint2*>(dst + 16 * m) =
                make_uint2(bits[m][0] | (bits[m][1] << 16), bits[m][2] | (bits[m][3] << 16));
        }
        if constexpr (FMT == FMT_A8W8) {
          // row amax of the bf16-rounded values over the wave's 32 columns
          amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
          amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
          if (g == 0 && tok >= 0) atomicMax(reinterpret_cast<unsigned int*>(p.h_s) + slot, __float_as_uint(amax));
        }
      }
    }
  } else {
    if (p.mode == 0 && k32) {  // STORE: gamma * S(x), the dense shared expert's addend
#pragma unroll
      for (int nn = 0; nn < NN; ++nn) {
        const int r = nn * 32 + lane % 32;
        const int tok = sm.tok[r];
        if (tok < 0) continue;
        const float sc = sm.rs[r] * ev.wscale;
        const float gm = p.gamma ? p.gamma[tok] : 1.0f;
        const int cb = c0 + 4 * (lane / 32);
        float* dst = p.acc + (size_t)tok * p.H + cb;
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int col = cb + 32 * mm + 8 * j;
            *reinterpret_cast<float4*>(dst + 32 * mm + 8 * j) =
                make_float4(gm * (acc32[mm][nn][4 * j] * sc + epi_bias<EPI>(ev.b2, col)),
                            gm * (acc32[mm][nn][4 * j + 1] * sc + epi_bias<EPI>(ev.b2, col + 1)),
                            gm * (acc32[mm][nn][4 * j + 2] * sc + epi_bias<EPI>(ev.b2, col + 2)),
                            gm * (acc32[mm][nn][4 * j + 3] * sc + epi_bias<EPI>(ev.b2, col + 3)));
          }
      }
      return;
    }
    if (p.mode == 0) {  // STORE: gamma * S(x), the dense shared expert's addend
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int r = nb * 16 + l16;
        const int tok = sm.tok[r];
        if (tok < 0) continue;
        const float sc = sm.rs[r] * ev.wscale;
        const float gm = p.gamma ? p.gamma[tok] : 1.0f;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int col = c0 + mb * 16 + 4 * g;
          *reinterpret_cast<float4*>(p.acc + (size_t)tok * p.H + col) =
              make_float4(gm * (acc[mb][nb][0] * sc + epi_bias<EPI>(ev.b2, col)),
                          gm * (acc[mb][nb][1] * sc + epi_bias<EPI>(ev.b2, col + 1)),
                          gm * (acc[mb][nb][2] * sc + epi_bias<EPI>(ev.b2, col + 2)),
                          gm * (acc[mb][nb][3] * sc + epi_bias<EPI>(ev.b2, col + 3)));
        }
      }
      return;
    }
    // ACCUMULATE: the weighted pair rows (64 columns each) in the 16-bit
    // block-scaled form; the tile's reduction is XCD-local, so ordinary stores
    // Each (pair, tile) is one 128-byte line of codes.  The codes pass through
    // this wave's 4 KiB of the idle staging buffer (16-byte chunk c of row r
    // at r * 128 + 16 (c ^ (r & 7))) so that eight lanes store a row's line
    // whole, eight rows per instruction.
    uint8_t* wl = &sm.x[0][0] + (tid / kWave) * 4096;
    auto store_rows = [&](int r0, int nrows) {  // rows r0 .. r0 + nrows - 1 of the block, staged at wl
      wave_lds_sync();
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int rr = lane / 8 + 8 * k;
        const int c = lane % 8;
        if (rr < nrows) {
          const uint4 v = *reinterpret_cast<const uint4*>(wl + rr * 128 + 16 * (c ^ (rr & 7)));
          const int pr = sm.pair[r0 + rr];
          if (pr >= 0) *reinterpret_cast<uint4*>(pair_codes(p) + (size_t)pr * p.H + c0 + 8 * c) = v;
        }
      }
      wave_lds_sync();  // the next group rewrites the region
    };
    if (!wave_ok) {
      // no columns: this wave only takes part in the count below
    } else if constexpr (k32) {
      // lanes l and l + 32 hold the tile's 64 columns of token row l % 32 of
      // each 32-row group (columns 32 mm + 8 j + 4 (l / 32) + 0..3)
      const int rl = lane % 32, h = lane / 32;
#pragma unroll
      for (int nn = 0; nn < NN; ++nn) {
        const int r = nn * 32 + rl;
        const float sc = sm.rs[r] * ev.wscale;
        const float wgt = sm.rw[r];
        float amax = 0.f;
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            acc32[mm][nn][v] = wgt * (acc32[mm][nn][v] * sc + epi_bias<EPI>(ev.b2, c0 + 32 * mm + 8 * (v / 4) + 4 * h + v % 4));
            amax = tile_amax(amax, acc32[mm][nn][v]);
          }
        amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
        const int field = pair_tile_field(amax);
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int col = 32 * mm + 8 * j + 4 * h;
            *reinterpret_cast<uint2*>(wl + rl * 128 + 16 * ((4 * mm + j) ^ (rl & 7)) + 8 * h) =
                make_uint2(pair_code2(acc32[mm][nn][4 * j], acc32[mm][nn][4 * j + 1], field, col),
                           pair_code2(acc32[mm][nn][4 * j + 2], acc32[mm][nn][4 * j + 3], field, col + 2));
          }
        store_rows(nn * 32, 32);
      }
    } else {
      // lanes (g, l16), g = 0..3, hold the tile's 64 columns of token row l16
      // of each 16-row group (columns 16 mb + 4 g + 0..3)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int r = nb * 16 + l16;
        const float sc = sm.rs[r] * ev.wscale;
        const float wgt = sm.rw[r];
        float amax = 0.f;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            acc[mb][nb][v] = wgt * (acc[mb][nb][v] * sc + epi_bias<EPI>(ev.b2, c0 + 16 * mb + 4 * g + v));
            amax = tile_amax(amax, acc[mb][nb][v]);
          }
        amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
        amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
        const int field = pair_tile_field(amax);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int col = 16 * mb + 4 * g;
          *reinterpret_cast<uint2*>(wl + l16 * 128 + 16 * ((2 * mb + g / 2) ^ (l16 & 7)) + 8 * (g % 2)) =
              make_uint2(pair_code2(acc[mb][nb][0], acc[mb][nb][1], field, col),
                         pair_code2(acc[mb][nb][2], acc[mb][nb][3], field, col + 2));
        }
        store_rows(nb * 16, 16);
      }
    }
    if constexpr (k32) {
      if (group_count) {
        // One group per queue (H <= 2048): a row counts once for the group,
        // on the counter (token, cslot), once every wave's stores have
        // reached the L2 (each wave waits for its acknowledgements, then the
        // barrier); the first wave counts all rows.  A quarter of the atomics
        // (measured faster for bf16 there; slower for the fp8 formats).
        constexpr int ND = (BM + kWave - 1) / kWave;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid < kWave) {
#pragma unroll
          for (int d = 0; d < ND; ++d) {
            const int r = d * kWave + lane;
            int old = -1;
            if (r < BM && sm.pair[r] >= 0) old = atomicAdd(p.counters + (size_t)sm.tok[r] * (p.H / 64) + cslot, 1);
            const uint64_t m = __ballot(old == p.expected - 1);
            if (lane == 0) sm.done[d] = m;
          }
        }
        __syncthreads();
        if (!wave_ok) return;
        uint64_t done[ND];
        int total = 0;
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          done[d] = sm.done[d];
          total += __popcll(done[d]);
        }
        // completed rows, compacted 8 at a time: entry i -> lanes 8 (i % 8) .. + 7
        for (int base = 0; base < total; base += 8) {
          const int i = base + lane / 8;
          if (i < total) {
            int rem = i, r = -1;
#pragma unroll
            for (int d = 0; d < ND; ++d) {
              const int c = __popcll(done[d]);
              if (r < 0 && rem < c) {
                uint64_t m = done[d];
                for (int k = 0; k < rem; ++k) m &= m - 1;  // drop the lowest rem set bits
                r = d * kWave + (__ffsll((unsigned long long)m) - 1);
              }
              if (r < 0) rem -= c;
            }
            last_arrival_sum8_xcd(p, sm.tok[r], c0, lane % 8, lane);
          }
        }
        return;
      }
    }
    // count arrivals once the stores have reached the L2 (their acknowledgement);
    // all of the block's counter atomics are issued before any result is used
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    const int n_tiles = p.H / 64;
    const int tile = c0 / 64;
    // cnt[nb]: 16-bit mask of the done (last-arrival) tokens of row block nb
    uint32_t cnt[NB];
    int total = 0;
    if constexpr (k32) {
      // lanes 0..31 hold the 32 tokens of each group
      int old[NN];
#pragma unroll
      for (int nn = 0; nn < NN; ++nn) {
        const int r = nn * 32 + lane % 32;
        old[nn] = -1;
        if (lane < 32 && sm.pair[r] >= 0) old[nn] = atomicAdd(p.counters + (size_t)sm.tok[r] * n_tiles + tile, 1);
      }
#pragma unroll
      for (int nn = 0; nn < NN; ++nn) {
        const uint64_t m = __ballot(old[nn] == p.expected - 1);  // only lanes < 32 can match
        cnt[2 * nn] = (uint32_t)m & 0xFFFFu;
        cnt[2 * nn + 1] = (uint32_t)(m >> 16) & 0xFFFFu;
      }
    } else {
      int old[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int r = nb * 16 + l16;
        old[nb] = -1;
        if (g == 0 && sm.pair[r] >= 0) old[nb] = atomicAdd(p.counters + (size_t)sm.tok[r] * n_tiles + tile, 1);
      }
      // lanes 0..15 hold the tokens of each row block
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) cnt[nb] = (uint32_t)__ballot(old[nb] == p.expected - 1 && g == 0) & 0xFFFFu;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) total += __popc(cnt[nb]);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // the wave's last arrivals, compacted 8 at a time: entry i -> lanes
    // 8 (i % 8) .. + 7, each summing 8 of the tile's 64 columns
    if (total > 0) {
      for (int base = 0; base < total; base += 8) {
        const int i = base + lane / 8;
        if (i < total) {
          // the i-th done slot in (row block, token) order
          int rem = i, r = -1;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int c = __popc(cnt[nb]);
            if (r < 0 && rem < c) {
              uint32_t m = cnt[nb];
              for (int k = 0; k < rem; ++k) m &= m - 1;  // drop the lowest rem set bits
              r = nb * 16 + (__ffs(m) - 1);
            }
            if (r < 0) rem -= c;
          }
          last_arrival_sum8_xcd(p, sm.tok[r], c0, lane % 8, lane);
        }
      }
    }
  }
}

// Waves per SIMD the register allocation targets: two or three workgroups per
// CU keep more loads in flight, where the operand registers allow it without
// spilling much (bf16; 32- and 64-row blocks; 128-row a8w8 stage 1; three
// for the 64-row a8w8 stage-2 items).
template <int FMT, int STAGE, int NB>
constexpr int tile_waves_per_eu() {
  if (FMT == FMT_A8W8 && STAGE == 2 && NB == 4) return 3;  // with one token-row set in flight (a8w8 stage 2 -2 %)
  return (FMT == FMT_BF16 || NB <= 4 || (FMT == FMT_A8W8 && STAGE == 1)) ? 2 : 1;
}

// Stage 1 (and the dense STORE stage 2): one workgroup per (block, column
// tile) of 128 h columns / 256 output columns.
template <int FMT, int STAGE, int NB, bool EPI>
__global__ __launch_bounds__(kTileThreads)
__attribute__((amdgpu_waves_per_eu(tile_waves_per_eu<FMT, STAGE, NB>(), tile_waves_per_eu<FMT, STAGE, NB>())))
void gemm_tile_kernel(GemmParams p) {
  constexpr int BM = 16 * NB;
  constexpr int WCOLS = (STAGE == 1) ? 128 : 256;
  __shared__ __attribute__((aligned(16))) TileSmem<BM> sm;

  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);  // uniform: weight offsets stay scalar
  const int width_max = (STAGE == 1) ? (p.dense ? p.I_s : p.I) : p.H;
  const int n_col = width_max / WCOLS;
  const int nblk = p.dense ? (p.T + BM - 1) / BM : *p.num_blocks;
  const int active = nblk * n_col;
  if ((int)blockIdx.x >= active) return;
  const int lt = (STAGE == 1) ? xcd_remap((int)blockIdx.x, active) : (int)blockIdx.x;
  int b = lt / n_col, nc = lt % n_col;
  int e = -1;
  if (STAGE == 1 && !p.dense && p.offsets) e = expert_major(p, BM, n_col, lt, b, nc);
  else if (!p.dense) e = p.block_expert[b];
  const int n0 = nc * WCOLS;

  const ExpertView ev = resolve_expert<FMT, STAGE>(p, e);
  if (STAGE == 1 && n0 >= ev.width) return;  // past a narrow pseudo-expert chunk (uniform)
  int c0 = n0 + wv * ((STAGE == 1) ? 32 : 64);
  const bool wave_ok = (STAGE == 1) ? (c0 < ev.width) : true;
  if (!wave_ok) c0 = 0;  // rows past a narrow chunk: read block 0, store nothing
  tile_block<FMT, STAGE, NB, EPI>(p, sm, b, ev, c0, wave_ok, 0, false);
}

// Stage 2 ACCUMULATE: persistent workgroups draining the per-XCD queues.
// Queue x's items are (block b, group j): its waves own the reduction tiles
// t = x + 8 (4 j + w), w = 0..3 (t < H/64).  A row's arrival is counted on
// the counter (token, t) of its tile, or (bf16, every queue with one group)
// once for the group on the counter (token, x) (x * groups + j < H/64 for
// every non-empty group), among the T * (H/64) counter words.  Queue state
// (next item, owner) follows the counters and is zero on entry.
template <int FMT, int NB, bool EPI>
__global__ __launch_bounds__(kTileThreads)
__attribute__((amdgpu_waves_per_eu(tile_waves_per_eu<FMT, 2, NB>(), tile_waves_per_eu<FMT, 2, NB>())))
void gemm_tile_accum_kernel(GemmParams p) {
  constexpr int BM = 16 * NB;
  __shared__ __attribute__((aligned(16))) TileSmem<BM> sm;

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n64 = p.H / 64;
  const int nblk = *p.num_blocks * split_of(p);
  int* q_next = p.counters + (size_t)p.T * n64;
  int* q_owner = q_next + kNumXcd;
  const int me = xcc_id();
  const bool group_count = (n64 + kNumXcd - 1) / kNumXcd <= 4;  // one group per queue

  for (int step = 0; step < kNumXcd; ++step) {
    const int q = (me + step) % kNumXcd;
    const int tiles_q = (n64 - q + kNumXcd - 1) / kNumXcd;  // t = q (mod 8), t < n64
    const int groups_q = (tiles_q + 3) / 4;
    const int items_q = nblk * groups_q;
    if (items_q <= 0) continue;
    // claim the queue for this XCD (or find it already ours)
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
      const int e = p.offsets ? expert_major(p, BM, groups_q, it, b, j) : p.block_expert[b / split_of(p)];
      const int t = q + kNumXcd * (4 * j + wv);
      const bool wave_ok = t < n64;
      const ExpertView ev = resolve_expert<FMT, 2>(p, e);
      tile_block<FMT, 2, NB, EPI>(p, sm, b, ev, wave_ok ? 64 * t : 0, wave_ok, q * groups_q + j, group_count);
      __syncthreads();  // the next item rewrites the row tables
    }
  }
}

// Stage 1 needs whole 128-column workgroups (and 32-column waves for a
// narrow last pseudo-expert chunk); stage 2 whole 256-column workgroups in
// STORE mode and 64-column tiles in ACCUMULATE mode.  The token rows are
// addressed with 32-bit buffer offsets.
bool tile_kernel_fits(const GemmParams& p, int stage, int fmt) {
  if (fmt == FMT_F32) return false;
  if (p.block_m != 32 && p.block_m != 64 && p.block_m != 128) return false;
  const size_t esz = fmt == FMT_BF16 ? 2 : 1;
  const size_t hsz = fmt == FMT_A8W8 ? 2 : esz;
  if (stage == 1) {
    const int w = p.dense ? p.I_s : p.I;
    if (w % 128) return false;
    if (!p.dense && p.n_pseudo > 0 && p.I_s % 32) return false;
    return (size_t)p.T * p.H * esz < 0x7FFFFFFFu;
  }
  if (p.mode == 0 ? p.H % 256 : p.H % 64) return false;
  return (size_t)p.max_blocks * p.block_m * p.ld_h * hsz < 0x7FFFFFFFu;
}

template <int FMT, int STAGE, int NB, bool EPI>
static hipError_t launch_tile_nbe(const GemmParams& p, hipStream_t s) {
  if (STAGE == 2 && p.mode != 0) {
    // persistent: as many workgroups per CU of each XCD as the register
    // allocation allows (an XCD has 32 CUs), no more than the largest queue
    // has items
    const int n64 = p.H / 64;
    const int groups = ((n64 + kNumXcd - 1) / kNumXcd + 3) / 4;
    long long per_xcd = (long long)p.max_blocks * groups;
    if (per_xcd > 32 * tile_waves_per_eu<FMT, 2, NB>()) per_xcd = 32 * tile_waves_per_eu<FMT, 2, NB>();
    return launch_gemm_kernel(gemm_tile_accum_kernel<FMT, NB, EPI>, dim3((unsigned)(kNumXcd * per_xcd)),
                              dim3(kTileThreads), s, p);
  }
  constexpr int WCOLS = (STAGE == 1) ? 128 : 256;
  const int width_max = (STAGE == 1) ? (p.dense ? p.I_s : p.I) : p.H;
  const dim3 grid((unsigned)(p.max_blocks * (width_max / WCOLS)));
  return launch_gemm_kernel(gemm_tile_kernel<FMT, STAGE, NB, EPI>, grid, dim3(kTileThreads), s, p);
}

template <int FMT, int STAGE, int NB>
static hipError_t launch_tile_nb(const GemmParams& p, hipStream_t s) {
  return epi_general(p, STAGE) ? launch_tile_nbe<FMT, STAGE, NB, true>(p, s) : launch_tile_nbe<FMT, STAGE, NB, false>(p, s);
}

template <int FMT, int STAGE>
static hipError_t launch_tile_fs(const GemmParams& p, hipStream_t s) {
  switch (p.block_m) {
    case 32: return launch_tile_nb<FMT, STAGE, 2>(p, s);
    case 64: return launch_tile_nb<FMT, STAGE, 4>(p, s);
    case 128: return launch_tile_nb<FMT, STAGE, 8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_tile(const GemmParams& p, int stage, int fmt, hipStream_t s) {
  switch (fmt) {
    case FMT_BF16: return stage == 1 ? launch_tile_fs<FMT_BF16, 1>(p, s) : launch_tile_fs<FMT_BF16, 2>(p, s);
    case FMT_MX: return stage == 1 ? launch_tile_fs<FMT_MX, 1>(p, s) : launch_tile_fs<FMT_MX, 2>(p, s);
    case FMT_MX4: return stage == 1 ? launch_tile_fs<FMT_MX4, 1>(p, s) : launch_tile_fs<FMT_MX4, 2>(p, s);
    case FMT_A8W8: return stage == 1 ? launch_tile_fs<FMT_A8W8, 1>(p, s) : launch_tile_fs<FMT_A8W8, 2>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
