// Device building blocks of the stable counting sort of (token, choice) pairs by expert,
// shared by the bucketing kernels and the fused small-batch route+bucket kernel.
// Output order inside an expert is ascending pair index p = t*k + j. Counts come from LDS
// integer atomics (order-free sums); ranks come from wave ballots (lanes with the same
// expert, below this lane) plus a fixed-order prefix over waves and over chunks, so no
// ordering decision depends on timing.
#pragma once
#include "common.hpp"

namespace moe {
namespace bucket_dev {

constexpr int kBThreads = 256;

__device__ __forceinline__ int clamp_expert(int e, int E) { return (e >= 0 && e < E) ? e : -1; }

constexpr int kChunk = 4096;   // pairs per chunk (held in LDS while it is placed)

// All helpers take the workgroup size NTH (a multiple of 64) as a template parameter and
// must be called by every thread of the workgroup.

// ids[begin, end) -> lds[0, end - begin), end - begin <= kChunk. Every thread issues all
// of its loads (from clamped, valid addresses) before it stores any.
template <int NTH = kBThreads>
__device__ inline void load_ids(const int32_t* __restrict__ ids, int begin, int end, int* lds) {
  constexpr int kPer = kChunk / NTH;
  const int n = end - begin;
  if (n <= 0) return;
  int v[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) v[r] = ids[begin + min((int)threadIdx.x + r * NTH, n - 1)];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int i = threadIdx.x + r * NTH;
    if (i < n) lds[i] = v[r];
  }
}

// Exclusive scan of v over the workgroup's NTH threads; returns this thread's prefix and
// writes the total to *total. `tmp` holds NTH / 64 ints of LDS.
template <int NTH = kBThreads>
__device__ inline int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int inc = v;
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    int o = __shfl_up(inc, m, kWave);
    if (lane >= m) inc += o;
  }
  if (lane == kWave - 1) tmp[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NTH / kWave; ++w) {
    if (w < wave) base += tmp[w];
    tot += tmp[w];
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// Place the pairs [begin, end) stably, 256 at a time; their expert ids are in LDS at
// lid[p - begin]. run[e] (LDS) holds, on entry, the position where expert e's next pair
// goes; it is advanced as pairs are placed.
template <int NTH = kBThreads>
__device__ inline void stable_scatter(const int* lid, int begin, int end, int E,
                               int* run, int (*wcnt)[kMaxE], int32_t* __restrict__ perm,
                               int32_t* __restrict__ inv_perm, int* perm_lds = nullptr) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  for (int base = begin; base < end; base += NTH) {
    const int p = base + threadIdx.x;
    const bool valid = p < end;
    const int e = valid ? clamp_expert(lid[p - begin], E) : -1;
    const bool has = e >= 0;
    // lanes of this wave with the same expert
    uint64_t peers = __ballot(has);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      uint64_t bal = __ballot(has && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? bal : ~bal;
    }
    if (!has) peers = 0;
    const uint64_t below = lane ? (~0ull >> (kWave - lane)) : 0ull;
    const int rank = __popcll(peers & below);
    const int cnt = __popcll(peers);
    for (int i = threadIdx.x; i < (NTH / kWave) * kMaxE; i += NTH)
      (&wcnt[0][0])[i] = 0;
    __syncthreads();
    if (has && rank == cnt - 1) wcnt[wave][e] = cnt;   // the group's last lane reports
    __syncthreads();
    if (has) {
      int pre = 0;
      for (int w = 0; w < wave; ++w) pre += wcnt[w][e];
      const int pos = run[e] + pre + rank;
      perm[pos] = p;
      inv_perm[p] = pos;
      if (perm_lds) perm_lds[pos] = p;
    }
    __syncthreads();
    for (int x = threadIdx.x; x < E; x += NTH) {
      int s = 0;
      for (int w = 0; w < NTH / kWave; ++w) s += wcnt[w][x];
      run[x] += s;
    }
    __syncthreads();
  }
}

// Whole counting sort of n <= kChunk pairs by one NTH-thread workgroup. ids may point to
// global memory or to LDS. LDS: lid [n], hist, run [kMaxE], wcnt [NTH/64][kMaxE],
// tmp [NTH/64].
template <int NTH = kBThreads>
__device__ inline void bucket_one_block(const int32_t* __restrict__ ids, int n, int E,
                                 int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                 int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
                                 int* lid, int* hist, int* run, int (*wcnt)[kMaxE], int* tmp,
                                 int* perm_lds = nullptr) {
  for (int e = threadIdx.x; e < kMaxE; e += NTH) hist[e] = 0;
  if (n <= kWave) {
    // one wave holds every pair: counts, offsets, and a ballot rank inside each expert
    const int lane = threadIdx.x & (kWave - 1);
    const bool w0 = threadIdx.x < kWave;
    const int e = (w0 && lane < n) ? clamp_expert(ids[lane], E) : -1;
    __syncthreads();
    if (e >= 0) atomicAdd(&hist[e], 1);
    __syncthreads();
    const int c = threadIdx.x < E ? hist[threadIdx.x] : 0;
    int total;
    const int off = block_exclusive_scan<NTH>(c, tmp, &total);
    if (threadIdx.x < E) {
      counts[threadIdx.x] = c;
      offsets[threadIdx.x] = off;
      run[threadIdx.x] = off + c;
      hist[threadIdx.x] = c;
    }
    if (threadIdx.x == 0) offsets[E] = total;
    __syncthreads();
    if (w0) {
      const bool has = e >= 0;
      uint64_t peers = __ballot(has);
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const uint64_t bal = __ballot(has && ((e >> b) & 1));
        peers &= ((e >> b) & 1) ? bal : ~bal;
      }
      if (has) {
        const uint64_t below = lane ? (~0ull >> (kWave - lane)) : 0ull;
        const int pos = (run[e] - hist[e]) + __popcll(peers & below);
        perm[pos] = lane;
        inv_perm[lane] = pos;
        if (perm_lds) perm_lds[pos] = lane;
      }
    }
    __syncthreads();
    return;
  }
  load_ids<NTH>(ids, 0, n, lid);
  __syncthreads();
  for (int p = threadIdx.x; p < n; p += NTH) {
    int e = clamp_expert(lid[p], E);
    if (e >= 0) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  const int c = threadIdx.x < E ? hist[threadIdx.x] : 0;
  int total;
  const int off = block_exclusive_scan<NTH>(c, tmp, &total);
  if (threadIdx.x < E) {
    counts[threadIdx.x] = c;
    offsets[threadIdx.x] = off;
    run[threadIdx.x] = off;
  }
  if (threadIdx.x == 0) offsets[E] = total;
  __syncthreads();
  stable_scatter<NTH>(lid, 0, n, E, run, wcnt, perm, inv_perm, perm_lds);
}

}  // namespace bucket_dev
}  // namespace moe
