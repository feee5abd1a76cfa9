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
#include "bucket_dev.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

using namespace bucket_dev;

__global__ __launch_bounds__(kBThreads) void k_bucket_single(const int32_t* __restrict__ ids,
                                                             int n, int E,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ perm,
                                                             int32_t* __restrict__ inv_perm) {
  __shared__ int lid[kChunk];
  __shared__ int hist[kMaxE];
  __shared__ int run[kMaxE];
  __shared__ int wcnt[kBThreads / kWave][kMaxE];
  __shared__ int tmp[4];
  bucket_one_block(ids, n, E, counts, offsets, perm, inv_perm, lid, hist, run, wcnt, tmp);
}

__global__ __launch_bounds__(kBThreads) void k_bucket_count(const int32_t* __restrict__ ids,
                                                            int n, int E,
                                                            int32_t* __restrict__ chunk_cnt) {
  __shared__ int lid[kChunk];
  __shared__ int hist[kMaxE];
  for (int e = threadIdx.x; e < kMaxE; e += kBThreads) hist[e] = 0;
  const int begin = blockIdx.x * kChunk;
  const int end = min(n, begin + kChunk);
  load_ids(ids, begin, end, lid);
  __syncthreads();
  for (int p = threadIdx.x; p < end - begin; p += kBThreads) {
    int e = clamp_expert(lid[p], E);
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
  constexpr int kBatch = 16;
  const int e = threadIdx.x;
  const int ec = e < E ? e : 0;
  int c = 0;
  for (int z0 = 0; z0 < nchunks; z0 += kBatch) {
    int v[kBatch];
#pragma unroll
    for (int r = 0; r < kBatch; ++r) v[r] = chunk_cnt[(int64_t)min(z0 + r, nchunks - 1) * E + ec];
#pragma unroll
    for (int r = 0; r < kBatch; ++r)
      if (z0 + r < nchunks) c += v[r];
  }
  int total;
  const int off = block_exclusive_scan(e < E ? c : 0, tmp, &total);
  if (e < E) {
    counts[e] = c;
    offsets[e] = off;
    int run = off;
    for (int z0 = 0; z0 < nchunks; z0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int r = 0; r < kBatch; ++r) v[r] = chunk_cnt[(int64_t)min(z0 + r, nchunks - 1) * E + e];
#pragma unroll
      for (int r = 0; r < kBatch; ++r)
        if (z0 + r < nchunks) {
          chunk_cnt[(int64_t)(z0 + r) * E + e] = run;
          run += v[r];
        }
    }
  }
  if (e == 0) offsets[E] = total;
}

__global__ __launch_bounds__(kBThreads) void k_bucket_scatter(const int32_t* __restrict__ ids,
                                                              int n, int E,
                                                              const int32_t* __restrict__ chunk_base,
                                                              int32_t* __restrict__ perm,
                                                              int32_t* __restrict__ inv_perm) {
  __shared__ int lid[kChunk];
  __shared__ int run[kMaxE];
  __shared__ int wcnt[kBThreads / kWave][kMaxE];
  const int begin = blockIdx.x * kChunk;
  const int end = min(n, begin + kChunk);
  for (int e = threadIdx.x; e < E; e += kBThreads)
    run[e] = chunk_base[(int64_t)blockIdx.x * E + e];
  load_ids(ids, begin, end, lid);
  __syncthreads();
  stable_scatter(lid, begin, end, E, run, wcnt, perm, inv_perm);
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
