// Resident hits and misses.
//
// The llama.cpp discussion "fixed GPU expert working set with Native CPU miss execution"
// (original post) serves the selected experts that sit in the GPU pool from there and
// computes the others elsewhere, then merges the weighted outputs; it also proposes public
// hit/miss counters. Here an expert whose slot_map entry is kSlotMiss is not in the pool:
// the expert kernels give its pairs zero output (so the combine sums the resident pairs),
// k_miss_list lists the missed pairs for the caller, and k_merge_misses adds the caller's
// outputs for them.
#include "common.hpp"
#include "bucket_dev.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kMissThreads = 1024;

// One workgroup. Missed pairs are listed expert by expert (bucket order), so the list is
// their bucket positions in increasing order; miss_of_pair maps a pair to its list index.
__global__ __launch_bounds__(kMissThreads) void k_miss_list(
    const int32_t* __restrict__ slot_map, int E, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ perm, int n, int32_t* __restrict__ miss_pos,
    int32_t* __restrict__ miss_of_pair, int32_t* __restrict__ counters) {
  __shared__ int lo_l[kMaxE], cnt_l[kMaxE], base_l[kMaxE];
  __shared__ int tmp[kMissThreads / kWave];
  __shared__ int hit_e, miss_e;
  const int tid = threadIdx.x;
  if (tid == 0) {
    hit_e = 0;
    miss_e = 0;
  }
  int cnt = 0, lo = 0;
  bool miss = false;
  if (tid < E) {
    lo = offsets[tid];
    cnt = offsets[tid + 1] - lo;
    miss = slot_map[tid] == kSlotMiss;
  }
  int total;
  const int base = bucket_dev::block_exclusive_scan<kMissThreads>(miss ? cnt : 0, tmp, &total);
  if (tid < E) {
    lo_l[tid] = lo;
    cnt_l[tid] = miss ? cnt : 0;
    base_l[tid] = base;
    if (cnt > 0) atomicAdd(miss ? &miss_e : &hit_e, 1);   // integer sums: order-free
  }
  for (int p = tid; p < n; p += kMissThreads) miss_of_pair[p] = -1;
  __syncthreads();   // the -1 stores of this workgroup come before the indices below
  for (int e = 0; e < E; ++e) {
    const int c = cnt_l[e];
    for (int i = tid; i < c; i += kMissThreads) {
      const int pos = lo_l[e] + i, m = base_l[e] + i;
      miss_pos[m] = pos;
      miss_of_pair[perm[pos]] = m;
    }
  }
  if (tid == 0) {
    counters[0] = n - total;
    counters[1] = total;
    counters[2] = hit_e;
    counters[3] = miss_e;
  }
}

// out[t, 4c..4c+3] += w[t,j] * y_miss[m_j, 4c..4c+3] for the missed pairs j of token t, in
// increasing j. One thread per 4 columns of a token; grid (ceil(H/4/256), min(T, 65535)),
// tokens t = blockIdx.y, + gridDim.y, ...
__global__ __launch_bounds__(256) void k_merge_misses(float* __restrict__ out,
                                                      const float* __restrict__ y_miss,
                                                      const int32_t* __restrict__ miss_of_pair,
                                                      const float* __restrict__ topk_w, int T,
                                                      int k, int H) {
  const int c4 = blockIdx.x * blockDim.x + threadIdx.x;
  if (c4 * 4 >= H) return;
  for (int t = blockIdx.y; t < T; t += gridDim.y) {
    int m[kMaxK];
    float w[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {   // every load first (clamped to a valid pair)
      const int64_t p = (int64_t)t * k + min(j, k - 1);
      m[j] = miss_of_pair[p];
      w[j] = topk_w[p];
    }
    f32x4 acc = *(const f32x4*)(out + (int64_t)t * H + c4 * 4);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k && m[j] >= 0) {
        const f32x4 v = *(const f32x4*)(y_miss + (int64_t)m[j] * H + c4 * 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = fmaf(w[j], v[q], acc[q]);
      }
    }
    *(f32x4*)(out + (int64_t)t * H + c4 * 4) = acc;
  }
}

}  // namespace

hipError_t launch_miss_list(const int32_t* slot_map, int E, const int32_t* offsets,
                            const int32_t* perm, int n, int32_t* miss_pos,
                            int32_t* miss_of_pair, int32_t* counters, hipStream_t stream) {
  if (E < 1 || E > kMaxE || n < 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_miss_list, dim3(1), dim3(kMissThreads), 0, stream, slot_map, E, offsets,
                     perm, n, miss_pos, miss_of_pair, counters);
  return hipGetLastError();
}

hipError_t launch_merge_misses(float* out, const float* y_miss, const int32_t* miss_of_pair,
                               const float* topk_w, int T, int k, int H, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  if (k < 1 || k > kMaxK || H % 4) return hipErrorInvalidValue;
  dim3 grid((H / 4 + 255) / 256, min(T, kMaxGridY));
  hipLaunchKernelGGL(k_merge_misses, grid, dim3(256), 0, stream, out, y_miss, miss_of_pair,
                     topk_w, T, k, H);
  return hipGetLastError();
}

}  // namespace moe
