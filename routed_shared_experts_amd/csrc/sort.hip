// Token-by-expert sort with per-expert padding (vLLM PR 65207, "Purpose",
// commit 2, and the review's "moe_sorting without zeroing" experiment: the
// sort also clears the output accumulator unless an addend is present).
//
// Workgroup 0 (1024 threads) does the whole sort in LDS (sort_wg in
// prologue.hpp: histogram, padded scan and block map, stable ballot-ranked
// scatter); workgroups 1.. clear the requested region with 16-byte stores.
// Larger pair counts use the two-launch variant further below.
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

// ---- two-launch sort for large pair counts -----------------------------------
// A: per-chunk expert histograms (order-independent LDS atomics), one
//    workgroup per chunk of 1024 pairs;
// B: one workgroup per chunk again.  Each reads every chunk's histogram
//    (a few thousand words from L2) and derives what it needs itself: the
//    experts' totals, the padded exclusive scan over experts, and its own
//    chunk's base per expert (offset + the counts of the chunks before it);
//    then it places its pairs with the ballot-match ranking of the
//    single-workgroup sort.  The bookkeeping (counts, offsets, block map,
//    padding sentinels) is spread over all the workgroups.  No workgroup
//    waits for another, so there is no serial scan launch in between.
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

__global__ __launch_bounds__(kSortThreads) void sort_place_kernel(SortParams p) {
  __shared__ int s_wave[kSortWaves][kMaxSortExperts];
  __shared__ int s_tot[kMaxSortExperts];
  __shared__ int s_pre[kMaxSortExperts];
  __shared__ int s_off[kMaxSortExperts + 1];
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int nE = p.n_experts, BM = p.block_m;
  const int nchunk = (p.P + kChunk - 1) / kChunk;
  const int c = blockIdx.x;
  for (int i = tid; i < kSortWaves * kMaxSortExperts; i += kSortThreads) (&s_wave[0][0])[i] = 0;

  // 1. per expert: the total over all chunks and the sum over chunks < c
  //    (16 chunks' loads in flight at a time, coalesced over experts)
  for (int e = tid; e < nE; e += kSortThreads) {
    int tot = 0, pre = 0;
    for (int c0 = 0; c0 < nchunk; c0 += 16) {
      int v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = c0 + u < nchunk ? p.chunk_base[(size_t)(c0 + u) * nE + e] : 0;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        tot += v[u];
        pre += (c0 + u < c) ? v[u] : 0;
      }
    }
    s_tot[e] = tot;
    s_pre[e] = pre;
  }
  __syncthreads();
  // 2. padded exclusive scan over the experts (wave 0)
  if (wv == 0) {
    int carry = 0;
    for (int base = 0; base < nE; base += kWave) {
      const int e = base + lane;
      const int cnt = e < nE ? s_tot[e] : 0;
      const int pc = (cnt + BM - 1) / BM * BM;
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

  // 3. bookkeeping, spread over the workgroups (global thread index gi)
  const long long gi = (long long)c * kSortThreads + tid;
  const long long gstride = (long long)nchunk * kSortThreads;
  if (c == 0) {
    for (int e = tid; e < nE; e += kSortThreads) {
      p.counts[e] = s_tot[e];
      p.offsets[e] = s_off[e];
    }
    if (tid == 0) {
      p.offsets[nE] = total;
      *p.num_blocks = nblk;
    }
  }
  for (long long i = gi; i < (long long)nE * BM; i += gstride) {  // padding slots of each expert
    const int e = (int)(i / BM), j = (int)(i % BM);
    const int at = s_off[e] + s_tot[e] + j;
    if (at < s_off[e + 1]) p.sorted[at] = p.P;
  }
  const int max_blocks = p.capacity / BM;
  for (long long b = gi; b < max_blocks; b += gstride) {  // block -> expert
    int be = -1;
    if (b < nblk) {
      const int row = (int)b * BM;
      int lo = 0, hi = nE - 1;
      while (lo < hi) {  // last e with off[e] <= row
        const int mid = (lo + hi + 1) / 2;
        if (s_off[mid] <= row) lo = mid; else hi = mid - 1;
      }
      be = lo;
    }
    p.block_expert[b] = be;
  }
  for (long long i = total + gi; i < p.capacity; i += gstride) p.sorted[i] = p.P;  // unused tail

  // 4. this chunk's pairs: base = offset + earlier chunks, then the waves
  //    before this one, then the rank among equal experts in the wave
  const int pi = c * kChunk + tid;
  const bool valid = pi < p.P;
  const int e = valid ? p.ids[pi] : 0;
  uint64_t peers = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 10; ++bit) {
    const bool bb = (e >> bit) & 1;
    const uint64_t bal = __ballot(bb);
    peers &= bb ? bal : ~bal;
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank = __popcll(peers & lt_mask);
  const int leader = valid ? (__ffsll((unsigned long long)peers) - 1) : -1;
  if (valid && lane == leader) s_wave[wv][e] = __popcll(peers);
  __syncthreads();
  if (valid) {
    int pos = s_off[e] + s_pre[e] + rank;
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
  hipLaunchKernelGGL(sort_place_kernel, dim3(nchunk), dim3(kSortThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
