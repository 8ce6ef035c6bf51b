// Host side of the C ABI: argument validation (pure host, before any launch),
// workspace carving, and the launch sequence of the fused layer forward on one
// or two HIP streams.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "../../include/moe.h"
#include "kernels.hpp"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxSortExperts = 576;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Layer format from a weight family; -1 when the combination is not provided.
int weights_fmt(const moe_weights& w) {
  if (w.dtype == MOE_F32 && w.scale == MOE_SCALE_NONE) return FMT_F32;
  if (w.dtype == MOE_BF16 && w.scale == MOE_SCALE_NONE) return FMT_BF16;
  if (w.dtype == MOE_FP8_E4M3 && w.scale == MOE_SCALE_MX32) return FMT_MX;
  if (w.dtype == MOE_FP8_E4M3 && w.scale == MOE_SCALE_PER_EXPERT) return FMT_A8W8;
  if (w.dtype == MOE_FP4_E2M1 && w.scale == MOE_SCALE_MX32) return FMT_MX4;
  return -1;
}

int ktile_elems(int fmt) { return fmt == FMT_F32 ? 32 : (fmt == FMT_BF16 ? 64 : 128); }

// MXFP4 weight rows pack whole 128-byte tiles (256 e2m1 elements)
bool mx4_shapes_ok(long long H, long long I, long long Is) { return H % 256 == 0 && I % 256 == 0 && Is % 256 == 0; }
int h_elem_bytes(int fmt) { return fmt == FMT_F32 ? 4 : (fmt_mx(fmt) ? 1 : 2); }

bool weights_ok(const moe_weights& w, int fmt) {
  if (!w.w13 || !w.w2 || !aligned16(w.w13) || !aligned16(w.w2)) return false;
  if (fmt_mx(fmt) || fmt == FMT_A8W8) {
    if (!w.w13_scale || !w.w2_scale) return false;
    if (fmt_mx(fmt) && (((uintptr_t)w.w13_scale & 3u) || ((uintptr_t)w.w2_scale & 3u))) return false;
    if (fmt == FMT_A8W8 && (((uintptr_t)w.w13_scale & 3u) || ((uintptr_t)w.w2_scale & 3u))) return false;
  }
  if (((uintptr_t)w.b13 & 3u) || ((uintptr_t)w.b2 & 3u)) return false;  // fp32 biases
  return true;
}

bool activation_ok(int32_t act) { return act == MOE_ACT_SILU || act == MOE_ACT_GELU_TANH; }

// MOE_OK, or the error for a weight family in a layout the kernels do not read
moe_status layout_status(const moe_weights& w) {
  if (w.layout == MOE_LAYOUT_TILED) return MOE_OK;
  return w.layout == MOE_LAYOUT_ROW_MAJOR ? MOE_ERR_UNSUPPORTED : MOE_ERR_INVALID_ARG;
}

bool overlaps(const void* a, const void* b, size_t n) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + n && y < x + n;
}

// batches up to this many tokens use the self-sorting one-wave kernels when
// their blocks have 16 rows
constexpr int kSelfSortMaxTokens = 64;

// The smallest block that holds about 1.5x the mean rows of an expert, so
// that a typical expert is one block and streams its weights once (measured
// on MI355X: MXFP8 with ~36 rows per expert runs faster in 64-row blocks than
// in 32-row ones, where most experts spill into a second block).
int auto_block_m(double rows_per_expert) {
  const double need = 1.5 * rows_per_expert;
  if (need <= 16) return 16;
  if (need <= 32) return 32;
  if (need <= 64) return 64;
  return 128;
}

struct Plan {
  int fmt;
  int mode;  // resolved shared mode: NONE, PSEUDO or AUX
  int m;     // pseudo experts
  int k_total, E_total, block_m, capacity, max_blocks;
  // self_sort: the one-wave GEMM kernels find each 16-row block's pairs in the
  // routing ids themselves (block b = sb * E_total + e), so no sort launch runs
  int self_sort, ss_blocks, h_rows;
  int dense_bm, dense_blocks;
  size_t off_logits;  // router logits [T][E] fp32 when the layer computes them
  size_t off_ids, off_w, off_gamma, off_xq, off_xs, off_counts, off_offsets, off_nblk, off_sorted, off_sortws,
      off_bexp, off_h, off_hs, off_hsh, off_hshs, off_amax_sh, off_acc, off_pair, off_cnt, off_amax, off_end;
  size_t zero_begin, zero_end;  // region the sort launch clears
  size_t amax_sh_bytes;
};

int resolve_mode(const moe_forward_args* a, int fmt);

// 256-row sorted blocks run on the LDS-staged kernels only: both routed
// stages must fit them (whole 128-column stage-1 workgroups, 32-column pseudo
// chunks, 32-bit buffer offsets).
bool big_blocks_fit(const moe_forward_args* a, int fmt) {
  if (fmt == FMT_MX4) return false;
  const int m = resolve_mode(a, fmt) == MOE_SHARED_PSEUDO ? (a->I_s + a->I - 1) / a->I : 0;
  const size_t esz = fmt == FMT_BF16 ? 2 : 1, hsz = fmt == FMT_A8W8 ? 2 : esz;
  if (a->I % 128 || (m > 0 && a->I_s % 32)) return false;
  if ((size_t)a->T * a->H * esz >= 0x7FFFFFFFu) return false;
  const size_t cap = (size_t)moe_sort_capacity(a->T, a->topk + m, a->E + m, 256);
  return cap * a->I * hsz < 0x7FFFFFFFu;
}

moe_status validate_impl(const moe_forward_args* a, int* fmt_out) {
  if (!a) return MOE_ERR_INVALID_ARG;
  // T = 0 is an empty batch: valid, and then logits, x, out and the row
  // scales may be NULL
  if (a->T < 0 || a->H <= 0 || a->E <= 0 || a->I <= 0 || a->I_s < 0 || a->topk <= 0)
    return MOE_ERR_INVALID_ARG;
  if (a->E > 512 || a->topk > a->E) return MOE_ERR_INVALID_ARG;
  if (a->H % 16 || a->I % 16 || a->I_s % 16) return MOE_ERR_INVALID_ARG;
  if (a->score != MOE_SCORE_SOFTMAX && a->score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (a->n_group < 1 || a->n_group > 64 || a->E % a->n_group) return MOE_ERR_INVALID_ARG;
  if (a->topk_group < 1 || a->topk_group > a->n_group) return MOE_ERR_INVALID_ARG;
  if (a->group_score_topk != 1 && a->group_score_topk != 2) return MOE_ERR_INVALID_ARG;
  if (a->n_group > 1 && a->group_score_topk == 2 && a->E / a->n_group < 2) return MOE_ERR_INVALID_ARG;
  if ((long long)a->topk > (long long)a->topk_group * (a->E / a->n_group)) return MOE_ERR_INVALID_ARG;
  if (a->T > 0 && ((!a->logits && !a->router_w) || !a->x || !a->out)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(a->logits) || !aligned16(a->x) || !aligned16(a->out) || !aligned16(a->router_w))
    return MOE_ERR_INVALID_ARG;
  if (a->bias && ((uintptr_t)a->bias & 3u)) return MOE_ERR_INVALID_ARG;
  if (a->bias && a->score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (a->out_dtype != MOE_F32 && a->out_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (!activation_ok(a->activation)) return MOE_ERR_INVALID_ARG;
  if (a->shared_mode < MOE_SHARED_NONE || a->shared_mode > MOE_SHARED_AUTO) return MOE_ERR_INVALID_ARG;
  if (a->block_m != 0 && a->block_m != 16 && a->block_m != 32 && a->block_m != 64 && a->block_m != 128 &&
      a->block_m != 256)
    return MOE_ERR_INVALID_ARG;
  const int fmt = weights_fmt(a->routed);
  if (fmt < 0) return MOE_ERR_UNSUPPORTED;
  if (!weights_ok(a->routed, fmt)) return MOE_ERR_INVALID_ARG;
  if (const moe_status st = layout_status(a->routed)) return st;
  // activation format must match the weight format
  if (fmt == FMT_F32 && a->x_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  if ((fmt == FMT_BF16 || fmt_mx(fmt)) && a->x_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (fmt == FMT_A8W8) {
    if (a->x_dtype != MOE_FP8_E4M3) return MOE_ERR_UNSUPPORTED;
    if ((a->T > 0 && !a->x_row_scale) || ((uintptr_t)a->x_row_scale & 3u)) return MOE_ERR_INVALID_ARG;
  }
  if (fmt == FMT_F32 && a->out_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (fmt == FMT_F32 && a->block_m == 256) return MOE_ERR_UNSUPPORTED;  // 256-row blocks: tiled kernels only
  const int kt = ktile_elems(fmt);
  if (a->H % kt || a->I % kt || (a->I_s % kt)) return MOE_ERR_INVALID_ARG;
  if (a->H % 64) return MOE_ERR_INVALID_ARG;  // stage-2 column tile
  if (fmt == FMT_MX4 && !mx4_shapes_ok(a->H, a->I, a->I_s)) return MOE_ERR_INVALID_ARG;
  if (a->router_w && a->H % (a->x_dtype == MOE_F32 ? 32 : 64)) return MOE_ERR_INVALID_ARG;
  if (a->gate_w) {
    if (!aligned16(a->gate_w)) return MOE_ERR_INVALID_ARG;
    if (fmt != FMT_F32 && fmt != FMT_BF16) return MOE_ERR_UNSUPPORTED;
  }
  if (a->I_s > 0) {
    if (a->shared_mode == MOE_SHARED_NONE) return MOE_ERR_INVALID_ARG;
    const int sfmt = weights_fmt(a->shared);
    if (sfmt < 0) return MOE_ERR_UNSUPPORTED;
    if (!weights_ok(a->shared, sfmt)) return MOE_ERR_INVALID_ARG;
    if (const moe_status st = layout_status(a->shared)) return st;
    if (a->shared_mode == MOE_SHARED_PSEUDO) {
      // fusion only when the shared weights use the routed experts' format
      if (sfmt != fmt) return MOE_ERR_UNSUPPORTED;
      if (fmt == FMT_A8W8 && a->I_s > a->I) return MOE_ERR_UNSUPPORTED;
      const int m = (a->I_s + a->I - 1) / a->I;
      if (a->topk + m > 64 || a->E + m > kMaxSortExperts) return MOE_ERR_UNSUPPORTED;
    }
    if (a->shared_mode == MOE_SHARED_AUX && sfmt != fmt) return MOE_ERR_UNSUPPORTED;
  } else if (a->shared_mode == MOE_SHARED_PSEUDO || a->shared_mode == MOE_SHARED_AUX) {
    return MOE_ERR_INVALID_ARG;
  }
  if ((long long)a->T * (a->topk + 64) >= (1LL << 31) / 2) return MOE_ERR_UNSUPPORTED;
  if (a->block_m == 256 && !big_blocks_fit(a, fmt)) return MOE_ERR_UNSUPPORTED;
  if (fmt_out) *fmt_out = fmt;
  return MOE_OK;
}

int resolve_mode(const moe_forward_args* a, int fmt) {
  if (a->I_s == 0) return MOE_SHARED_NONE;
  if (a->shared_mode != MOE_SHARED_AUTO) return a->shared_mode;
  const int sfmt = weights_fmt(a->shared);
  const int m = (a->I_s + a->I - 1) / a->I;
  const bool pseudo_ok = sfmt == fmt && !(fmt == FMT_A8W8 && a->I_s > a->I) && a->topk + m <= 64 &&
                         a->E + m <= kMaxSortExperts;
  return pseudo_ok ? MOE_SHARED_PSEUDO : MOE_SHARED_AUX;
}

Plan make_plan(const moe_forward_args* a, int fmt) {
  Plan pl{};
  pl.fmt = fmt;
  pl.mode = resolve_mode(a, fmt);
  pl.m = pl.mode == MOE_SHARED_PSEUDO ? (a->I_s + a->I - 1) / a->I : 0;
  pl.k_total = a->topk + pl.m;
  pl.E_total = a->E + pl.m;
  const long long P = (long long)a->T * pl.k_total;
  pl.block_m = a->block_m ? a->block_m : auto_block_m((double)P / pl.E_total);
  pl.capacity = moe_sort_capacity(a->T, pl.k_total, pl.E_total, pl.block_m);
  pl.max_blocks = pl.capacity / pl.block_m;
  {
    // the one-wave kernels must take both stages (32-bit buffer offsets)
    const size_t ss_rows = (size_t)pl.E_total * ((a->T + 15) / 16) * 16;
    const size_t hsz = fmt == FMT_A8W8 ? 2 : (size_t)h_elem_bytes(fmt);
    pl.self_sort = pl.block_m == 16 && a->T <= kSelfSortMaxTokens && a->I % 32 == 0 && a->I_s % 32 == 0 &&
                   ss_rows * a->I * hsz < 0x7FFFFFFFu;
  }
  pl.ss_blocks = pl.self_sort ? pl.E_total * ((a->T + 15) / 16) : 0;
  pl.h_rows = pl.capacity > pl.ss_blocks * 16 ? pl.capacity : pl.ss_blocks * 16;
  // dense (aux-stream) blocks: at most 128 rows, which every kernel provides
  pl.dense_bm = a->block_m ? (a->block_m < 128 ? a->block_m : 128) : auto_block_m((double)a->T);
  if (pl.dense_bm > 128) pl.dense_bm = 128;
  pl.dense_blocks = (a->T + pl.dense_bm - 1) / pl.dense_bm;
  const int esz_h = h_elem_bytes(fmt);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, kAlign); return at; };
  pl.off_logits = take(a->router_w ? (size_t)a->T * a->E * 4 : 0);
  pl.off_ids = take((size_t)P * 4);
  pl.off_w = take((size_t)P * 4);
  pl.off_gamma = take((size_t)a->T * 4);
  pl.off_xq = take(fmt_mx(fmt) ? (size_t)a->T * a->H : 0);
  pl.off_xs = take(fmt_mx(fmt) ? (size_t)a->T * (a->H / 32) : 0);
  pl.off_counts = take((size_t)pl.E_total * 4);
  pl.off_offsets = take((size_t)(pl.E_total + 1) * 4);
  pl.off_nblk = take(16);
  pl.off_sorted = take((size_t)pl.capacity * 4);
  pl.off_sortws = take(sort_scratch_bytes((int)P, pl.E_total));
  pl.off_bexp = take((size_t)pl.max_blocks * 4);
  pl.off_h = take((size_t)pl.h_rows * a->I * esz_h);
  pl.off_hs = take(fmt_mx(fmt) ? (size_t)pl.h_rows * (a->I / 32) : 0);
  const size_t dense_rows = (size_t)pl.dense_blocks * pl.dense_bm;
  const bool aux = pl.mode == MOE_SHARED_AUX;
  pl.off_hsh = take(aux ? dense_rows * a->I_s * esz_h : 0);
  pl.off_hshs = take(aux && fmt_mx(fmt) ? dense_rows * (a->I_s / 32) : 0);
  pl.amax_sh_bytes = aux && fmt == FMT_A8W8 ? align_up(dense_rows * 4, kAlign) : 0;
  pl.off_amax_sh = take(pl.amax_sh_bytes);
  // the addend (AUX mode only) and the per-pair stage-2 rows
  pl.off_acc = take(aux ? (size_t)a->T * a->H * 4 : 0);
  pl.off_pair = take((size_t)P * a->H * 4);
  // cleared by the sort launch: arrival counters, then the routed row amax (A8W8)
  pl.off_cnt = take(moe_stage2_counters(a->T, a->H) * 4);
  pl.off_amax = take(fmt == FMT_A8W8 ? (size_t)pl.h_rows * 4 : 0);
  pl.off_end = o;
  pl.zero_begin = pl.off_cnt;
  pl.zero_end = o;
  return pl;
}

__global__ void fill_zero_kernel(uint4* p, long long n) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t zero_async(void* p, size_t bytes, hipStream_t s) {
  const long long n = (long long)(bytes / 16);
  if (n == 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint4*>(p), n);
  return hipGetLastError();
}

void fill_weights(GemmParams& g, const moe_weights& r, const moe_weights& s) {
  g.w13 = static_cast<const uint8_t*>(r.w13);
  g.w2 = static_cast<const uint8_t*>(r.w2);
  g.w13_s = r.w13_scale;
  g.w2_s = r.w2_scale;
  g.ws13 = static_cast<const uint8_t*>(s.w13);
  g.ws2 = static_cast<const uint8_t*>(s.w2);
  g.ws13_s = s.w13_scale;
  g.ws2_s = s.w2_scale;
  g.b13 = r.b13;
  g.b2 = r.b2;
  g.bs13 = s.b13;
  g.bs2 = s.b2;
}

thread_local hipError_t g_last_hip = hipSuccess;  // last HIP failure reported as MOE_ERR_HIP

#define HIP_TRY(x)                     \
  do {                                 \
    const hipError_t e_ = (x);         \
    if (e_ != hipSuccess) {            \
      g_last_hip = e_;                 \
      return MOE_ERR_HIP;              \
    }                                  \
  } while (0)

// Drops an error that earlier runtime calls of the caller left pending, so
// that the hipGetLastError() after each launch here reports that launch.
// (Errors from a faulted kernel are sticky and still surface.)
inline void clear_pending_error() { (void)hipGetLastError(); }

}  // namespace

// ---- the allocation-free forward ------------------------------------------
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc): the workspace lives in a
// file-scope device array, one copy per GPU for the life of the process.  In
// host code the array's name is only a stand-in; its device address on the
// current GPU is looked up once per device and used from then on.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxScratchDevices];  // device address of `scratch`, per device

moe_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip = e;
    return MOE_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      g_last_hip = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return MOE_ERR_HIP;
    }
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_last_hip_error(void) {
  if (g_last_hip == hipSuccess) return "";
  return hipGetErrorString(g_last_hip);
}

const char* moe_status_str(int32_t status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_UNKNOWN_STATUS";
  }
}

int32_t moe_query_feature(int32_t feature) {
  switch (feature) {
    case MOE_FEATURE_ACCUMULATE_OUTPUT:
    case MOE_FEATURE_PSEUDO_SHARED:
    case MOE_FEATURE_AUX_STREAM:
    case MOE_FEATURE_MXFP8:
    case MOE_FEATURE_MXFP4:
    case MOE_FEATURE_A8W8:
    case MOE_FEATURE_F32:
    case MOE_FEATURE_BF16:
    case MOE_FEATURE_EXPERT_BIAS:
    case MOE_FEATURE_GELU_TANH:
    case MOE_FEATURE_ROUTER_GEMM: return 1;
    default: return 0;
  }
}

int32_t moe_sort_capacity(int32_t T, int32_t k_total, int32_t n_experts, int32_t block_m) {
  if (T < 0 || k_total <= 0 || n_experts <= 0 || block_m <= 0) return 0;
  const long long P = (long long)T * k_total;
  long long cap = P + (long long)(n_experts < P ? n_experts : P) * (block_m - 1);
  cap = (cap + block_m - 1) / block_m * block_m;
  if (cap == 0) cap = block_m;
  return (int32_t)cap;
}

moe_status moe_validate(const moe_forward_args* a) { return validate_impl(a, nullptr); }

size_t moe_sort_scratch_bytes(int32_t T, int32_t k_total, int32_t n_experts) {
  if (T <= 0 || k_total <= 0 || n_experts <= 0) return 0;
  return sort_scratch_bytes(T * k_total, n_experts);
}

size_t moe_workspace_bytes(const moe_forward_args* a) {
  int fmt = -1;
  if (validate_impl(a, &fmt) != MOE_OK) return 0;
  return make_plan(a, fmt).off_end;
}

moe_status moe_route(const float* logits, const float* bias, int32_t T, int32_t E, int32_t topk,
                     int32_t n_group, int32_t topk_group, int32_t group_score_topk, int32_t score,
                     int32_t renormalize, float routed_scaling_factor, int32_t n_pseudo,
                     const float* gamma, int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  if (!logits || !topk_ids || !topk_w || T <= 0 || E <= 0 || E > 512 || topk <= 0 || topk > E)
    return MOE_ERR_INVALID_ARG;
  if (n_pseudo < 0 || topk + n_pseudo > 64) return MOE_ERR_INVALID_ARG;
  if (n_group < 1 || n_group > 64 || E % n_group || topk_group < 1 || topk_group > n_group)
    return MOE_ERR_INVALID_ARG;
  if (group_score_topk != 1 && group_score_topk != 2) return MOE_ERR_INVALID_ARG;
  if (n_group > 1 && group_score_topk == 2 && E / n_group < 2) return MOE_ERR_INVALID_ARG;
  if ((long long)topk > (long long)topk_group * (E / n_group)) return MOE_ERR_INVALID_ARG;
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  RouteParams p{};
  p.logits = logits;
  p.bias = bias;
  p.T = T;
  p.E = E;
  p.topk = topk;
  p.n_group = n_group;
  p.topk_group = topk_group;
  p.gtopk = group_score_topk;
  p.score = score;
  p.renorm = renormalize != 0;
  p.scale = routed_scaling_factor;
  p.n_pseudo = n_pseudo;
  p.gamma_in = gamma;
  p.ids = topk_ids;
  p.w = topk_w;
  p.do_route = 1;
  clear_pending_error();
  HIP_TRY(launch_route(p, stream));
  return MOE_OK;
}

moe_status moe_router_logits(const void* x, int32_t x_dtype, const float* x_row_scale, const void* router_w,
                             int32_t T, int32_t H, int32_t E, float* logits, hipStream_t stream) {
  if (T < 0 || H <= 0 || E <= 0 || E > 512) return MOE_ERR_INVALID_ARG;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16 && x_dtype != MOE_FP8_E4M3) return MOE_ERR_UNSUPPORTED;
  if (H % (x_dtype == MOE_F32 ? 32 : 64)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !router_w || !logits || !aligned16(x) || !aligned16(router_w) || !aligned16(logits))
    return MOE_ERR_INVALID_ARG;
  if (x_dtype == MOE_FP8_E4M3 && (!x_row_scale || ((uintptr_t)x_row_scale & 3u))) return MOE_ERR_INVALID_ARG;
  RouterParams rg{};
  rg.x = x;
  rg.x_fmt = x_dtype == MOE_F32 ? 0 : (x_dtype == MOE_BF16 ? 1 : 2);
  rg.x_scale = x_row_scale;
  rg.w = router_w;
  rg.T = T;
  rg.H = H;
  rg.E = E;
  rg.logits = logits;
  RouteParams rp{};  // do_route = 0: logits only
  clear_pending_error();
  HIP_TRY(launch_router(rg, rp, stream));
  return MOE_OK;
}

moe_status shared_gate_dot(const void* x, int32_t x_dtype, const void* g, int32_t T, int32_t H,
                           int32_t apply_sigmoid, float* gate_out, hipStream_t stream) {
  if (!x || !g || !gate_out || T <= 0 || H <= 0 || !aligned16(x) || !aligned16(g)) return MOE_ERR_INVALID_ARG;
  if (x_dtype == MOE_F32) {
    if (H % 4) return MOE_ERR_INVALID_ARG;
  } else if (x_dtype == MOE_BF16) {
    if (H % 8) return MOE_ERR_INVALID_ARG;
  } else {
    return MOE_ERR_UNSUPPORTED;
  }
  clear_pending_error();
  HIP_TRY(launch_gate_dot(x, x_dtype == MOE_F32, g, T, H, apply_sigmoid, gate_out, stream));
  return MOE_OK;
}

moe_status moe_pack_weights(const void* src, void* dst, int64_t rows, int32_t row_bytes, hipStream_t stream) {
  if (!src || !dst || rows < 0 || row_bytes <= 0 || rows % 16 || row_bytes % 128) return MOE_ERR_INVALID_ARG;
  if (!aligned16(src) || !aligned16(dst)) return MOE_ERR_INVALID_ARG;
  if (overlaps(src, dst, (size_t)rows * row_bytes)) return MOE_ERR_INVALID_ARG;
  clear_pending_error();
  HIP_TRY(launch_pack_weights(src, dst, rows, row_bytes, stream));
  return MOE_OK;
}

moe_status moe_pack_mx_scales(const void* src, void* dst, int64_t rows, int32_t scale_bytes, hipStream_t stream) {
  if (!src || !dst || rows < 0 || scale_bytes <= 0 || rows % 16 || scale_bytes % 4) return MOE_ERR_INVALID_ARG;
  if (((uintptr_t)src & 3u) || ((uintptr_t)dst & 3u)) return MOE_ERR_INVALID_ARG;
  if (overlaps(src, dst, (size_t)rows * scale_bytes)) return MOE_ERR_INVALID_ARG;
  clear_pending_error();
  HIP_TRY(launch_pack_scales(src, dst, rows, scale_bytes, stream));
  return MOE_OK;
}

moe_status moe_quant_mx(const void* x, int32_t T, int32_t H, uint8_t* codes, uint8_t* scales,
                        hipStream_t stream) {
  if (!x || !codes || !scales || T <= 0 || H <= 0 || H % 32 || !aligned16(x) || ((uintptr_t)codes & 7u))
    return MOE_ERR_INVALID_ARG;
  RouteParams p{};
  p.T = T;
  p.H = H;
  p.x = x;
  p.xq = codes;
  p.xs = scales;
  p.do_route = 0;
  clear_pending_error();
  HIP_TRY(launch_route(p, stream));
  return MOE_OK;
}

moe_status moe_sort_tokens(const int32_t* topk_ids, int32_t T, int32_t k_total, int32_t n_experts,
                           int32_t block_m, int32_t capacity, int32_t* sorted_pair_ids,
                           int32_t* block_expert, int32_t* counts, int32_t* offsets,
                           int32_t* num_blocks, void* scratch, size_t scratch_bytes, void* zero_ptr,
                           size_t zero_bytes, hipStream_t stream) {
  if (!topk_ids || !sorted_pair_ids || !block_expert || !counts || !offsets || !num_blocks)
    return MOE_ERR_INVALID_ARG;
  if (T <= 0 || k_total <= 0 || n_experts <= 0 || n_experts > kMaxSortExperts || block_m <= 0)
    return MOE_ERR_INVALID_ARG;
  if ((long long)T * k_total >= (1LL << 31) - 1) return MOE_ERR_INVALID_ARG;
  if (capacity < moe_sort_capacity(T, k_total, n_experts, block_m) || capacity % block_m)
    return MOE_ERR_INVALID_ARG;
  if (zero_bytes % 16 || (zero_bytes && (!zero_ptr || !aligned16(zero_ptr)))) return MOE_ERR_INVALID_ARG;
  const size_t need = sort_scratch_bytes(T * k_total, n_experts);
  if (scratch && scratch_bytes < need) return MOE_ERR_WORKSPACE;
  if (scratch && ((uintptr_t)scratch & 3u)) return MOE_ERR_INVALID_ARG;
  SortParams p{};
  p.chunk_base = (scratch && need) ? static_cast<int32_t*>(scratch) : nullptr;
  p.ids = topk_ids;
  p.P = T * k_total;
  p.n_experts = n_experts;
  p.block_m = block_m;
  p.capacity = capacity;
  p.sorted = sorted_pair_ids;
  p.block_expert = block_expert;
  p.counts = counts;
  p.offsets = offsets;
  p.num_blocks = num_blocks;
  p.zero_ptr = static_cast<uint4*>(zero_ptr);
  p.zero_vec = (long long)(zero_bytes / 16);
  clear_pending_error();
  HIP_TRY(launch_sort(p, stream));
  return MOE_OK;
}

static moe_status stage_params(const moe_stage_args* a, GemmParams& g, int& fmt) {
  if (!a) return MOE_ERR_INVALID_ARG;
  if (a->T <= 0 || a->H <= 0 || a->E <= 0 || a->I <= 0 || a->I_s < 0 || a->n_pseudo < 0 || a->k_total <= 0)
    return MOE_ERR_INVALID_ARG;
  if (a->block_m != 16 && a->block_m != 32 && a->block_m != 64 && a->block_m != 128 && a->block_m != 256)
    return MOE_ERR_INVALID_ARG;
  if (a->max_blocks <= 0) return MOE_ERR_INVALID_ARG;
  if (!activation_ok(a->activation)) return MOE_ERR_INVALID_ARG;
  const moe_weights& wf = a->dense ? a->shared : a->routed;
  fmt = weights_fmt(wf);
  if (fmt < 0) return MOE_ERR_UNSUPPORTED;
  if (fmt == FMT_F32 && a->block_m == 256) return MOE_ERR_UNSUPPORTED;
  if (!weights_ok(wf, fmt)) return MOE_ERR_INVALID_ARG;
  if ((a->n_pseudo > 0 || a->dense) && (a->I_s <= 0 || weights_fmt(a->shared) != fmt || !weights_ok(a->shared, fmt)))
    return MOE_ERR_INVALID_ARG;
  if (const moe_status st = layout_status(wf)) return st;
  if (a->n_pseudo > 0 || a->dense) {
    if (const moe_status st = layout_status(a->shared)) return st;
  }
  if (!a->dense && (!a->sorted_pair_ids || !a->block_expert || !a->num_blocks)) return MOE_ERR_INVALID_ARG;
  if (a->dense && a->max_blocks * a->block_m < a->T) return MOE_ERR_INVALID_ARG;
  const int kt = ktile_elems(fmt);
  if (a->H % kt || a->H % 64 || a->I % kt || a->I_s % kt) return MOE_ERR_INVALID_ARG;
  if (fmt == FMT_MX4 && (a->block_m == 256 || !mx4_shapes_ok(a->H, a->I, a->I_s))) return MOE_ERR_INVALID_ARG;
  if (!a->x || !a->h || !aligned16(a->x) || !aligned16(a->h)) return MOE_ERR_INVALID_ARG;
  if ((fmt_mx(fmt) || fmt == FMT_A8W8) && (!a->x_scale || !a->h_scale)) return MOE_ERR_INVALID_ARG;
  g = GemmParams{};
  g.T = a->T;
  g.H = a->H;
  g.E = a->E;
  g.I = a->I;
  g.I_s = a->I_s;
  g.n_pseudo = a->n_pseudo;
  g.k_total = a->k_total;
  fill_weights(g, a->routed, a->shared);
  g.act = a->activation;
  g.x = static_cast<const uint8_t*>(a->x);
  g.x_s = a->x_scale;
  g.dense = a->dense != 0;
  g.block_m = a->block_m;
  g.max_blocks = a->max_blocks;
  g.sorted = a->sorted_pair_ids;
  g.block_expert = a->block_expert;
  g.num_blocks = a->num_blocks;
  g.h = static_cast<uint8_t*>(a->h);
  g.h_s = a->h_scale;
  g.ld_h = a->dense ? a->I_s : a->I;
  g.pair_w = a->pair_w;
  g.gamma = a->gamma;
  g.acc = a->acc;
  g.pair_out = a->pair_out;
  g.out = a->out;
  g.out_bf16 = a->out_dtype == MOE_BF16;
  g.mode = a->mode;
  g.counters = a->counters;
  g.expected = a->expected_arrivals;
  // 256-row blocks run on the LDS-staged kernels only (sorted problem, the
  // ACCUMULATE stage 2)
  if (a->block_m == 256) {
    GemmParams g2 = g;
    g2.mode = MOE_STAGE2_ACCUMULATE;
    if (!lds_kernel_fits(g, 1, fmt) || !lds_kernel_fits(g2, 2, fmt)) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

moe_status moe_stage1(const moe_stage_args* a, hipStream_t stream) {
  GemmParams g;
  int fmt;
  moe_status st = stage_params(a, g, fmt);
  if (st != MOE_OK) return st;
  clear_pending_error();
  HIP_TRY(launch_gemm(g, 1, fmt, 64, stream));
  return MOE_OK;
}

moe_status moe_stage2_accum(const moe_stage_args* a, hipStream_t stream) {
  GemmParams g;
  int fmt;
  moe_status st = stage_params(a, g, fmt);
  if (st != MOE_OK) return st;
  if (a->acc && !aligned16(a->acc)) return MOE_ERR_INVALID_ARG;
  if (a->mode == MOE_STAGE2_STORE) {
    if (!a->dense) return MOE_ERR_UNSUPPORTED;
    if (!a->acc) return MOE_ERR_INVALID_ARG;
  } else if (a->mode == MOE_STAGE2_ACCUMULATE) {
    if (a->dense) return MOE_ERR_UNSUPPORTED;
    if (!a->out || !a->counters || !a->pair_out || !a->pair_w || a->expected_arrivals != a->k_total)
      return MOE_ERR_INVALID_ARG;
    if (a->out_dtype != MOE_F32 && a->out_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  } else {
    return MOE_ERR_INVALID_ARG;
  }
  clear_pending_error();
  if (a->addend_ready) HIP_TRY(hipStreamWaitEvent(stream, a->addend_ready, 0));
  HIP_TRY(launch_gemm(g, 2, fmt, 64, stream));
  return MOE_OK;
}

moe_status moe_forward(const moe_forward_args* a, void* workspace, size_t workspace_bytes, hipStream_t main_s,
                       hipStream_t aux_s, hipEvent_t ev_fork, hipEvent_t ev_ready) {
  int fmt = -1;
  moe_status st = validate_impl(a, &fmt);
  if (st != MOE_OK) return st;
  if (a->T == 0) return MOE_OK;  // empty batch: nothing to launch, workspace and streams untouched
  const Plan pl = make_plan(a, fmt);
  if (!workspace || ((uintptr_t)workspace & (kAlign - 1))) return MOE_ERR_WORKSPACE;
  if (workspace_bytes < pl.off_end) return MOE_ERR_WORKSPACE;
  const bool aux = pl.mode == MOE_SHARED_AUX;
  if (aux && (!aux_s || aux_s == main_s || !ev_fork || !ev_ready)) return MOE_ERR_INVALID_ARG;

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* ids = reinterpret_cast<int32_t*>(ws + pl.off_ids);
  float* pw = reinterpret_cast<float*>(ws + pl.off_w);
  float* gamma = reinterpret_cast<float*>(ws + pl.off_gamma);
  uint8_t* xq = ws + pl.off_xq;
  uint8_t* xs = ws + pl.off_xs;
  int32_t* counts = reinterpret_cast<int32_t*>(ws + pl.off_counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + pl.off_offsets);
  int32_t* nblk = reinterpret_cast<int32_t*>(ws + pl.off_nblk);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + pl.off_sorted);
  int32_t* bexp = reinterpret_cast<int32_t*>(ws + pl.off_bexp);
  float* acc = aux ? reinterpret_cast<float*>(ws + pl.off_acc) : nullptr;
  float* pair = reinterpret_cast<float*>(ws + pl.off_pair);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + pl.off_cnt);

  hipEvent_t* tev = a->timing_events;
  clear_pending_error();
  if (tev) HIP_TRY(hipEventRecord(tev[0], main_s));
  // 1. prologue: routing (+ gate dot + MX quantisation of x)
  RouteParams rp{};
  rp.logits = a->logits;
  rp.bias = a->bias;
  rp.T = a->T;
  rp.E = a->E;
  rp.topk = a->topk;
  rp.n_group = a->n_group;
  rp.topk_group = a->topk_group;
  rp.gtopk = a->group_score_topk;
  rp.score = a->score;
  rp.renorm = a->renormalize != 0;
  rp.scale = a->routed_scaling_factor;
  rp.n_pseudo = pl.m;
  rp.ids = ids;
  rp.w = pw;
  rp.x = a->x;
  rp.x_f32 = a->x_dtype == MOE_F32;
  rp.H = a->H;
  const bool gated = a->gate_w != nullptr && a->I_s > 0;
  rp.gate_w = gated ? a->gate_w : nullptr;
  rp.gamma_out = gated ? gamma : nullptr;
  rp.xq = fmt_mx(fmt) ? xq : nullptr;
  rp.xs = fmt_mx(fmt) ? xs : nullptr;
  rp.do_route = 1;

  // sort (+ clearing of the accumulator unless the addend fills it)
  SortParams sp{};
  sp.ids = ids;
  sp.P = a->T * pl.k_total;
  sp.n_experts = pl.E_total;
  sp.block_m = pl.block_m;
  sp.capacity = pl.capacity;
  sp.sorted = sorted;
  sp.block_expert = bexp;
  sp.counts = counts;
  sp.offsets = offsets;
  sp.num_blocks = nblk;
  sp.chunk_base = sort_scratch_bytes(sp.P, pl.E_total) ? reinterpret_cast<int32_t*>(ws + pl.off_sortws) : nullptr;
  sp.zero_ptr = reinterpret_cast<uint4*>(ws + pl.zero_begin);
  sp.zero_vec = (long long)((pl.zero_end - pl.zero_begin) / 16);
  if (pl.self_sort) {  // no sort launch: the routing launch clears the region
    rp.zero_ptr = sp.zero_ptr;
    rp.zero_vec = sp.zero_vec;
  }
  // Self-sorted stage 1 with softmax scores over at most 64 experts (no
  // groups) and nothing else in the prologue that stage 1 reads (no MX
  // quantisation of x, no a8w8 row maxima to clear) runs the routing inside
  // its own launch; the aux stream needs gamma before stage 1, so not with it.
  // With router weights the logits come from the router GEMM, which routes
  // its tokens in the same launch.
  const bool fuse_route = !a->router_w && pl.self_sort && !aux && a->score == MOE_SCORE_SOFTMAX &&
                          a->n_group <= 1 && (fmt == FMT_BF16 || fmt == FMT_F32) && a->E <= 64 && a->E % 4 == 0 &&
                          aligned16(a->logits);
  if (a->router_w) {
    RouterParams rg{};
    rg.x = a->x;
    rg.x_fmt = a->x_dtype == MOE_F32 ? 0 : (a->x_dtype == MOE_BF16 ? 1 : 2);
    rg.x_scale = a->x_row_scale;
    rg.w = a->router_w;
    rg.T = a->T;
    rg.H = a->H;
    rg.E = a->E;
    rg.logits = reinterpret_cast<float*>(ws + pl.off_logits);
    rp.logits = rg.logits;
    HIP_TRY(launch_router(rg, rp, main_s));
  } else if (!fuse_route) {
    HIP_TRY(launch_route(rp, main_s));
  }
  if (tev) HIP_TRY(hipEventRecord(tev[1], main_s));

  GemmParams g{};
  g.T = a->T;
  g.H = a->H;
  g.E = a->E;
  g.I = a->I;
  g.I_s = a->I_s;
  g.n_pseudo = pl.m;
  g.k_total = pl.k_total;
  fill_weights(g, a->routed, a->shared);
  g.act = a->activation;
  const void* x_stage = fmt_mx(fmt) ? static_cast<const void*>(xq) : a->x;
  const void* xs_stage = fmt_mx(fmt) ? static_cast<const void*>(xs)
                                       : (fmt == FMT_A8W8 ? static_cast<const void*>(a->x_row_scale) : nullptr);
  g.x = static_cast<const uint8_t*>(x_stage);
  g.x_s = xs_stage;
  g.acc = acc;
  g.pair_out = pair;
  g.out = a->out;
  g.out_bf16 = a->out_dtype == MOE_BF16;

  // 2. shared expert on the aux stream (dense), storing gamma * S(x) into acc
  if (aux) {
    HIP_TRY(hipEventRecord(ev_fork, main_s));
    HIP_TRY(hipStreamWaitEvent(aux_s, ev_fork, 0));
    GemmParams gs = g;
    gs.dense = 1;
    gs.block_m = pl.dense_bm;
    gs.max_blocks = pl.dense_blocks;
    gs.h = ws + pl.off_hsh;
    gs.ld_h = a->I_s;
    if (fmt_mx(fmt)) gs.h_s = ws + pl.off_hshs;
    if (fmt == FMT_A8W8) {
      gs.h_s = ws + pl.off_amax_sh;
      HIP_TRY(zero_async(gs.h_s, pl.amax_sh_bytes, aux_s));
    }
    gs.gamma = gated ? gamma : nullptr;
    gs.mode = MOE_STAGE2_STORE;
    HIP_TRY(launch_gemm(gs, 1, fmt, 64, aux_s));
    HIP_TRY(launch_gemm(gs, 2, fmt, 64, aux_s));
    HIP_TRY(hipEventRecord(ev_ready, aux_s));
  }

  // 3. sort (self-sorted blocks need none)
  if (!pl.self_sort) HIP_TRY(launch_sort(sp, main_s));
  if (tev) HIP_TRY(hipEventRecord(tev[2], main_s));

  // 4. routed stage 1
  g.dense = 0;
  g.block_m = pl.block_m;
  g.max_blocks = pl.self_sort ? pl.ss_blocks : pl.max_blocks;
  g.self_sort = pl.self_sort;
  g.route_fused = fuse_route;
  if (fuse_route) g.route = rp;
  g.ids = ids;
  g.sorted = sorted;
  g.block_expert = bexp;
  g.num_blocks = nblk;
  g.offsets = pl.self_sort ? nullptr : offsets;
  g.h = ws + pl.off_h;
  g.ld_h = a->I;
  g.h_s = fmt_mx(fmt) ? static_cast<void*>(ws + pl.off_hs)
                        : (fmt == FMT_A8W8 ? static_cast<void*>(ws + pl.off_amax) : nullptr);
  if (tev) {
    g.ev_start = tev[3];
    g.ev_stop = tev[4];
  }
  HIP_TRY(launch_gemm(g, 1, fmt, 64, main_s));

  // 5. routed stage 2: weighted scatter-add onto the addend, last arrival writes out
  if (aux) HIP_TRY(hipStreamWaitEvent(main_s, ev_ready, 0));
  g.pair_w = pw;
  g.mode = MOE_STAGE2_ACCUMULATE;
  g.counters = cnt;
  g.expected = pl.k_total;
  if (tev) {
    g.ev_start = tev[5];
    g.ev_stop = tev[6];
  }
  HIP_TRY(launch_gemm(g, 2, fmt, 64, main_s));
  return MOE_OK;
}

moe_status moe_forward_noalloc(const moe_forward_args* a, hipStream_t main_s, hipStream_t aux_s,
                               hipEvent_t ev_fork, hipEvent_t ev_ready) {
  int fmt = -1;
  const moe_status st = validate_impl(a, &fmt);
  if (st != MOE_OK) return st;
  if (a->T == 0) return MOE_OK;
  if (make_plan(a, fmt).off_end > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  const moe_status sst = scratch_of_current_device(&ws);
  if (sst != MOE_OK) return sst;
  return moe_forward(a, ws, MOE_NOALLOC_SCRATCH_BYTES, main_s, aux_s, ev_fork, ev_ready);
}

}  // extern "C"
