// Internal launch interface between the host dispatcher (api.cpp) and the
// gfx950 kernels.  Not part of the public C ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// FMT_MX4: MXFP4 weights (e2m1, e8m0 per 32) with the MX-fp8 activations and
// intermediate of FMT_MX
enum Fmt : int { FMT_F32 = 0, FMT_BF16 = 1, FMT_MX = 2, FMT_A8W8 = 3, FMT_MX4 = 4 };
// formats whose activations, intermediate and weights carry MX-32 scales
constexpr bool fmt_mx(int f) { return f == FMT_MX || f == FMT_MX4; }

struct RouteParams {
  const float* logits;
  const float* bias;
  int T, E, topk, n_group, topk_group, gtopk, score, renorm;
  float scale;
  int n_pseudo;
  const float* gamma_in;  // pseudo-slot weights when the gate is not fused (or NULL)
  int32_t* ids;
  float* w;
  // fused gate dot (gate_w != NULL)
  const void* x;
  int x_f32;  // 1: x/gate are fp32, 0: bf16
  const void* gate_w;
  int H;
  float* gamma_out;
  // fused MX quantisation of bf16 x (xq != NULL)
  uint8_t* xq;
  uint8_t* xs;
  int do_route;
  // region cleared by the workgroups after the routing ones (or NULL)
  uint4* zero_ptr;
  long long zero_vec;
};

// Router-logit GEMM: logits [T][E] = x . w^T (fp32 accumulation); x_fmt 0:
// fp32 x and w; 1: bf16 x and w; 2: e4m3 x with an fp32 scale per token,
// bf16 w.  w is row-major [E][H].
struct RouterParams {
  const void* x;
  int x_fmt;
  const float* x_scale;
  const void* w;
  int T, H, E;
  float* logits;
};

struct SortParams {
  const int32_t* ids;
  int P, n_experts, block_m, capacity;
  int32_t* sorted;
  int32_t* block_expert;
  int32_t* counts;
  int32_t* offsets;
  int32_t* num_blocks;
  int32_t* chunk_base;  // [ceil(P/1024)][n_experts] scratch, or NULL (single-workgroup sort)
  uint4* zero_ptr;
  long long zero_vec;  // number of 16-byte vectors to clear
};

struct GemmParams {
  int T, H, E, I, I_s, n_pseudo, k_total;
  const uint8_t* w13;
  const uint8_t* w2;
  const void* w13_s;
  const void* w2_s;
  const uint8_t* ws13;
  const uint8_t* ws2;
  const void* ws13_s;
  const void* ws2_s;
  // per-expert fp32 biases (or NULL): b13 [E][2I], b2 [E][H]; shared bs13
  // [2 I_s], bs2 [H]
  const float* b13;
  const float* b2;
  const float* bs13;
  const float* bs2;
  int act;  // stage-1 activation: 0 SiLU, 1 GELU (tanh form)
  const uint8_t* x;
  const void* x_s;
  int dense, block_m, max_blocks;
  // self_sort (16-row blocks of the one-wave kernel): block b = sb * (E + n_pseudo)
  // + e holds expert e's pairs of rank 16 sb.. in pair order, found by scanning
  // ids [T][k_total]; sorted / block_expert / num_blocks are then unused
  int self_sort;
  const int32_t* ids;
  const int32_t* sorted;
  const int32_t* block_expert;
  const int32_t* num_blocks;
  const int32_t* offsets;  // [E' + 1] padded row offsets of the experts (sort output), or NULL
  // bsplit > 1: the launch runs each sorted block of block_m * bsplit rows as
  // bsplit blocks of block_m rows (block_expert and num_blocks count the
  // sorted blocks); 0 or 1: no split
  int bsplit;
  uint8_t* h;
  void* h_s;
  int ld_h;
  const float* pair_w;
  const float* gamma;
  float* acc;       // STORE: destination of gamma * S(x); ACCUMULATE: addend (or NULL)
  float* pair_out;  // ACCUMULATE: [T * k_total][H] per-pair weighted outputs
  void* out;
  int out_bf16;
  int mode;  // 0 store, 1 accumulate
  int32_t* counters;
  int expected;
  // route_fused (self_sort stage 1, softmax scores without groups): the
  // routing runs inside the stage-1 launch.  Each GEMM wave finds its
  // expert's tokens from the router logits with the selection rule of the
  // routing itself, and route.T workgroups after the GEMM grid route the
  // tokens (ids, weights and gamma for stage 2), the ones after those clear
  // route.zero_ptr
  int route_fused;
  RouteParams route;
  // host side only: events stamped with the GEMM kernel's own start and end
  // (instrumentation; both NULL for an ordinary launch)
  hipEvent_t ev_start, ev_stop;
};

// Whether a stage needs the general epilogue (a bias, or an activation other
// than SiLU).
inline bool epi_general(const GemmParams& p, int stage) {
  return stage == 1 ? (p.b13 || p.bs13 || p.act != 0) : (p.b2 || p.bs2);
}

// Launch of a GEMM kernel taking GemmParams; with instrumentation events the
// dispatch itself records the kernel's start and end times on them.
template <typename K>
inline hipError_t launch_gemm_kernel(K kernel, dim3 grid, dim3 block, hipStream_t s, const GemmParams& p) {
  if (p.ev_start || p.ev_stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, p.ev_start, p.ev_stop, 0, p);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_route(const RouteParams& p, hipStream_t s);
// the router GEMM, then (rp.do_route) the routing of RouteParams from the
// computed logits in the same launch (rp.logits is not read)
hipError_t launch_router(const RouterParams& g, const RouteParams& rp, hipStream_t s);
hipError_t launch_gate_dot(const void* x, int x_f32, const void* g, int T, int H, int apply_sigmoid,
                           float* out, hipStream_t s);
hipError_t launch_sort(const SortParams& p, hipStream_t s);
size_t sort_scratch_bytes(int P, int n_experts);
hipError_t launch_gemm(const GemmParams& p, int stage, int fmt, int bn, hipStream_t s);
hipError_t launch_gemm_wave(const GemmParams& p, int stage, int fmt, hipStream_t s);
bool wave_kernel_fits(const GemmParams& p, int stage, int fmt);
hipError_t launch_gemm_tile(const GemmParams& p, int stage, int fmt, hipStream_t s);
bool tile_kernel_fits(const GemmParams& p, int stage, int fmt);
hipError_t launch_gemm_lds(const GemmParams& p, int stage, int fmt, hipStream_t s);
bool lds_kernel_fits(const GemmParams& p, int stage, int fmt);
hipError_t launch_pack_weights(const void* src, void* dst, int64_t rows, int32_t row_bytes, hipStream_t s);
hipError_t launch_pack_scales(const void* src, void* dst, int64_t rows, int32_t scale_bytes, hipStream_t s);

}  // namespace moe
