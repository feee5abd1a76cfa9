// Bucketing of the (token, choice) pairs by expert: a stable counting sort.
//
// Grouping tokens by expert so each expert's weights are loaded once per layer is the
// "Batched prefill" item of tinyserve's "How it works" list; the llama.cpp discussion's
// original post plans "expert bucketing + grouped GEMM" for prefill.
//
// Output order inside an expert is ascending pair index p = t*k + j. Nothing here lets an
// atomic decide an order: counts come from LDS integer atomics (order-free sums); ranks
// come from wave ballots (lanes with the same expert, below this lane) plus a fixed-order
// prefix over waves and over chunks.
//
// Small inputs (one chunk) use one workgroup. Larger ones use three launches:
//   count   per-chunk histograms              -> scratch [nchunks][E]
//   scan    per-(chunk, expert) bases, counts, offsets (one workgroup)
//   scatter per-chunk stable placement        -> perm, inv_perm
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kBThreads = 256;
constexpr int kChunk = 4096;   // pairs per chunk

__device__ __forceinline__ int clamp_expert(int e, int E) { return (e >= 0 && e < E) ? e : -1; }

// Exclusive scan of v over the workgroup's 256 threads; returns this thread's prefix and
// writes the total to *total. `tmp` holds 4 ints of LDS.
__device__ int block_exclusive_scan(int v, int* tmp, int* total) {
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
  for (int w = 0; w < kBThreads / kWave; ++w) {
    if (w < wave) base += tmp[w];
    tot += tmp[w];
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// Place the pairs [begin, end) stably, 256 at a time. run[e] (LDS) holds, on entry, the
// position where expert e's next pair goes; it is advanced as pairs are placed.
__device__ void stable_scatter(const int32_t* __restrict__ ids, int begin, int end, int E,
                               int* run, int (*wcnt)[kMaxE], int32_t* __restrict__ perm,
                               int32_t* __restrict__ inv_perm) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  for (int base = begin; base < end; base += kBThreads) {
    const int p = base + threadIdx.x;
    const bool valid = p < end;
    const int e = valid ? clamp_expert(ids[p], E) : -1;
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
    for (int i = threadIdx.x; i < (kBThreads / kWave) * kMaxE; i += kBThreads)
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
    }
    __syncthreads();
    for (int x = threadIdx.x; x < E; x += kBThreads) {
      int s = 0;
      for (int w = 0; w < kBThreads / kWave; ++w) s += wcnt[w][x];
      run[x] += s;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kBThreads) void k_bucket_single(const int32_t* __restrict__ ids,
                                                             int n, int E,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ perm,
                                                             int32_t* __restrict__ inv_perm) {
  __shared__ int hist[kMaxE];
  __shared__ int run[kMaxE];
  __shared__ int wcnt[kBThreads / kWave][kMaxE];
  __shared__ int tmp[4];
  for (int e = threadIdx.x; e < kMaxE; e += kBThreads) hist[e] = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < n; p += kBThreads) {
    int e = clamp_expert(ids[p], E);
    if (e >= 0) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  const int c = threadIdx.x < E ? hist[threadIdx.x] : 0;
  int total;
  const int off = block_exclusive_scan(c, tmp, &total);
  if (threadIdx.x < E) {
    counts[threadIdx.x] = c;
    offsets[threadIdx.x] = off;
    run[threadIdx.x] = off;
  }
  if (threadIdx.x == 0) offsets[E] = total;
  __syncthreads();
  stable_scatter(ids, 0, n, E, run, wcnt, perm, inv_perm);
}

__global__ __launch_bounds__(kBThreads) void k_bucket_count(const int32_t* __restrict__ ids,
                                                            int n, int E,
                                                            int32_t* __restrict__ chunk_cnt) {
  __shared__ int hist[kMaxE];
  for (int e = threadIdx.x; e < kMaxE; e += kBThreads) hist[e] = 0;
  __syncthreads();
  const int begin = blockIdx.x * kChunk;
  const int end = min(n, begin + kChunk);
  for (int p = begin + threadIdx.x; p < end; p += kBThreads) {
    int e = clamp_expert(ids[p], E);
    if (e >= 0) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kBThreads)
    chunk_cnt[(int64_t)blockIdx.x * E + e] = hist[e];
}

// chunk_cnt [nchunks][E] -> chunk base positions (in place), counts, offsets.
__global__ __launch_bounds__(kBThreads) void k_bucket_scan(int32_t* __restrict__ chunk_cnt,
                                                           int nchunks, int E,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets) {
  __shared__ int tmp[4];
  const int e = threadIdx.x;
  int c = 0;
  if (e < E)
    for (int z = 0; z < nchunks; ++z) c += chunk_cnt[(int64_t)z * E + e];
  int total;
  const int off = block_exclusive_scan(e < E ? c : 0, tmp, &total);
  if (e < E) {
    counts[e] = c;
    offsets[e] = off;
    int run = off;
    for (int z = 0; z < nchunks; ++z) {
      int v = chunk_cnt[(int64_t)z * E + e];
      chunk_cnt[(int64_t)z * E + e] = run;
      run += v;
    }
  }
  if (e == 0) offsets[E] = total;
}

__global__ __launch_bounds__(kBThreads) void k_bucket_scatter(const int32_t* __restrict__ ids,
                                                              int n, int E,
                                                              const int32_t* __restrict__ chunk_base,
                                                              int32_t* __restrict__ perm,
                                                              int32_t* __restrict__ inv_perm) {
  __shared__ int run[kMaxE];
  __shared__ int wcnt[kBThreads / kWave][kMaxE];
  for (int e = threadIdx.x; e < E; e += kBThreads)
    run[e] = chunk_base[(int64_t)blockIdx.x * E + e];
  __syncthreads();
  const int begin = blockIdx.x * kChunk;
  const int end = min(n, begin + kChunk);
  stable_scatter(ids, begin, end, E, run, wcnt, perm, inv_perm);
}

}  // namespace

size_t bucket_scratch_bytes(int n, int E) {
  const int nchunks = (n + kChunk - 1) / kChunk;
  if (nchunks <= 1) return 0;
  return (size_t)nchunks * E * sizeof(int32_t);
}

hipError_t launch_bucket(const int32_t* ids, int n, int E, int32_t* counts, int32_t* offsets,
                         int32_t* perm, int32_t* inv_perm, void* scratch, hipStream_t stream) {
  const int nchunks = (n + kChunk - 1) / kChunk;
  if (nchunks <= 1) {
    hipLaunchKernelGGL(k_bucket_single, dim3(1), dim3(kBThreads), 0, stream, ids, n, E, counts,
                       offsets, perm, inv_perm);
    return hipGetLastError();
  }
  int32_t* cc = (int32_t*)scratch;
  hipLaunchKernelGGL(k_bucket_count, dim3(nchunks), dim3(kBThreads), 0, stream, ids, n, E, cc);
  hipLaunchKernelGGL(k_bucket_scan, dim3(1), dim3(kBThreads), 0, stream, cc, nchunks, E, counts,
                     offsets);
  hipLaunchKernelGGL(k_bucket_scatter, dim3(nchunks), dim3(kBThreads), 0, stream, ids, n, E, cc,
                     perm, inv_perm);
  return hipGetLastError();
}

}  // namespace moe
