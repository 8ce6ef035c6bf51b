// Token-by-expert sort with per-expert padding (vLLM PR 65207, "Purpose",
// commit 2, and the review's "moe_sorting without zeroing" experiment: the
// sort also clears the output accumulator unless an addend is present).
//
// Workgroup 0 (1024 threads) does the whole sort in LDS (sort_wg in
// prologue.hpp: histogram, padded scan and block map, stable ballot-ranked
// scatter); workgroups 1.. clear the requested region with 16-byte stores.
// Larger pair counts use the three-launch variant further below.
#include "prologue.hpp"

namespace moe {

constexpr int kSmallSort = 8192;  // pair counts up to this use the single-workgroup sort

__global__ __launch_bounds__(kSortThreads) void sort_kernel(SortParams p) {
  if (blockIdx.x > 0) {
    clear_region(p.zero_ptr, p.zero_vec, 1);
    return;
  }
  __shared__ SortSmem sm;
  sort_wg(p, p.ids, sm);
}

// ---- three-launch sort for large pair counts --------------------------------
// A: per-chunk expert histograms (order-independent LDS atomics);
// B: one workgroup scans the histograms over chunks per expert and over the
//    padded expert counts, and writes counts, offsets, block map, sentinels and
//    each chunk's base position per expert;
// C: per chunk, the same ballot-match ranking as the single-workgroup sort
//    places every pair at base[chunk][e] + (rank within the chunk).
constexpr int kChunk = kSortThreads;  // pairs per chunk (one per thread)

__global__ __launch_bounds__(kSortThreads) void sort_count_kernel(SortParams p) {
  const int nchunk = (p.P + kChunk - 1) / kChunk;
  if ((int)blockIdx.x >= nchunk) {
    clear_region(p.zero_ptr, p.zero_vec, nchunk);
    return;
  }
  __shared__ int s_count[kMaxSortExperts];
  for (int e = threadIdx.x; e < p.n_experts; e += kSortThreads) s_count[e] = 0;
  __syncthreads();
  const int pi = blockIdx.x * kChunk + threadIdx.x;
  if (pi < p.P) atomicAdd(&s_count[p.ids[pi]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < p.n_experts; e += kSortThreads)
    p.chunk_base[(size_t)blockIdx.x * p.n_experts + e] = s_count[e];
}

__global__ __launch_bounds__(kSortThreads) void sort_scan_kernel(SortParams p) {
  __shared__ int s_count[kMaxSortExperts];
  __shared__ int s_off[kMaxSortExperts + 1];
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int nE = p.n_experts, BM = p.block_m;
  const int nchunk = (p.P + kChunk - 1) / kChunk;
  // per-expert totals: every (chunk, expert) count once, all loads in flight
  // together (coalesced over experts), summed with LDS atomics
  for (int e = tid; e < nE; e += kSortThreads) s_count[e] = 0;
  __syncthreads();
  const int ncount = nchunk * nE;
  for (int base = 0; base < ncount; base += 8 * kSortThreads) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * kSortThreads + tid;
      v[u] = i < ncount ? p.chunk_base[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * kSortThreads + tid;
      if (i < ncount && v[u]) atomicAdd(&s_count[i % nE], v[u]);
    }
  }
  __syncthreads();
  if (wv == 0) {
    int carry = 0;
    for (int base = 0; base < nE; base += kWave) {
      const int e = base + lane;
      const int c = e < nE ? s_count[e] : 0;
      const int pc = (c + BM - 1) / BM * BM;
      int incl = pc;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
      }
      if (e < nE) s_off[e] = carry + incl - pc;
      carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) s_off[nE] = carry;
  }
  __syncthreads();
  const int total = s_off[nE];
  const int nblk = total / BM;
  for (int e = tid; e < nE; e += kSortThreads) {
    p.counts[e] = s_count[e];
    p.offsets[e] = s_off[e];
    // chunk bases: the expert's offset plus the exclusive prefix of its counts
    // over the chunks, 16 chunks' loads in flight at a time
    int run = s_off[e];
    for (int c0 = 0; c0 < nchunk; c0 += 16) {
      int v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = c0 + u < nchunk ? p.chunk_base[(size_t)(c0 + u) * nE + e] : 0;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (c0 + u < nchunk) p.chunk_base[(size_t)(c0 + u) * nE + e] = run;
        run += v[u];
      }
    }
    for (int i = s_off[e] + s_count[e]; i < s_off[e + 1]; ++i) p.sorted[i] = p.P;
  }
  if (tid == 0) {
    p.offsets[nE] = total;
    *p.num_blocks = nblk;
  }
  const int max_blocks = p.capacity / BM;
  for (int b = tid; b < max_blocks; b += kSortThreads) {
    int be = -1;
    if (b < nblk) {
      int row = b * BM, lo = 0, hi = nE - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (s_off[mid] <= row) lo = mid; else hi = mid - 1;
      }
      be = lo;
    }
    p.block_expert[b] = be;
  }
  for (int i = total + tid; i < p.capacity; i += kSortThreads) p.sorted[i] = p.P;
}

__global__ __launch_bounds__(kSortThreads) void sort_scatter_kernel(SortParams p) {
  __shared__ int s_wave[kSortWaves][kMaxSortExperts];
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  for (int i = tid; i < kSortWaves * kMaxSortExperts; i += kSortThreads) (&s_wave[0][0])[i] = 0;
  const int pi = blockIdx.x * kChunk + tid;
  const bool valid = pi < p.P;
  const int e = valid ? p.ids[pi] : 0;
  uint64_t peers = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 10; ++bit) {
    const bool b = (e >> bit) & 1;
    const uint64_t bal = __ballot(b);
    peers &= b ? bal : ~bal;
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank = __popcll(peers & lt_mask);
  const int leader = valid ? (__ffsll((unsigned long long)peers) - 1) : -1;
  __syncthreads();
  if (valid && lane == leader) s_wave[wv][e] = __popcll(peers);
  __syncthreads();
  if (valid) {
    int pos = p.chunk_base[(size_t)blockIdx.x * p.n_experts + e] + rank;
    for (int w = 0; w < wv; ++w) pos += s_wave[w][e];
    p.sorted[pos] = pi;
  }
}

size_t sort_scratch_bytes(int P, int n_experts) {
  if (P <= kSmallSort) return 0;
  return (size_t)((P + kChunk - 1) / kChunk) * n_experts * sizeof(int32_t);
}

hipError_t launch_sort(const SortParams& p, hipStream_t s) {
  const long long zblocks = clear_blocks(p.zero_vec, kSortThreads);
  if (p.chunk_base == nullptr || p.P <= kSmallSort) {
    hipLaunchKernelGGL(sort_kernel, dim3(1 + (int)zblocks), dim3(kSortThreads), 0, s, p);
    return hipGetLastError();
  }
  const int nchunk = (p.P + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(sort_count_kernel, dim3(nchunk + (int)zblocks), dim3(kSortThreads), 0, s, p);
  hipLaunchKernelGGL(sort_scan_kernel, dim3(1), dim3(kSortThreads), 0, s, p);
  hipLaunchKernelGGL(sort_scatter_kernel, dim3(nchunk), dim3(kSortThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
