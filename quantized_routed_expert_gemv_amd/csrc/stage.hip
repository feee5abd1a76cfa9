// Staged prefill: the plan that maps a batch's used, non-resident experts to a window of
// staging slots, and the bulk copy of those experts into the window.
//
// The llama.cpp discussion "fixed GPU expert working set with Native CPU miss execution"
// ("Formal gate results") stages, per layer, the unique experts of a large prefill batch
// into shared VRAM windows, rewrites the mapping to those slots and runs the grouped
// quantized matmul on it; the tinyserve README ("How it works", item 6) loads each expert
// of a batch once. Both kernels read their sizes from device memory (the counts of the
// batch's bucketing, the plan's counters), so neither needs the host between routing and
// the grouped matmul.
#include <algorithm>

#include "common.hpp"
#include "bucket_dev.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kPlanThreads = 256;   // = kMaxE: one thread per expert

// One workgroup. Expert e needs staging if it has pairs and no slot; the i-th such expert
// (increasing e) takes slot first_slot + i while i < n_stage. slot_map_out may be slot_map:
// each thread reads its expert's entry before writing it.
__global__ __launch_bounds__(kPlanThreads) void k_stage_plan(
    const int32_t* __restrict__ counts, const int32_t* slot_map, int E, int first_slot,
    int n_stage, int32_t* slot_map_out, int32_t* __restrict__ copy_list,
    int32_t* __restrict__ counters) {
  __shared__ int tmp[kPlanThreads / kWave];
  const int e = threadIdx.x;
  int slot = kSlotMiss;
  bool need = false;
  if (e < E) {
    slot = slot_map[e];
    need = counts[e] > 0 && slot == kSlotMiss;
  }
  int total;
  const int rank = bucket_dev::block_exclusive_scan<kPlanThreads>(need ? 1 : 0, tmp, &total);
  if (e < E) {
    if (need && rank < n_stage) {
      slot = first_slot + rank;
      copy_list[rank] = e;
    }
    slot_map_out[e] = slot;
  }
  if (e == 0) {
    const int staged = min(total, n_stage);
    counters[0] = staged;
    counters[1] = total - staged;
  }
}

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;   // 16-byte pieces per thread in flight

// Grid (blocks per copy, max_copies): workgroup (x, i) copies its share of every plane of
// expert copy_list[i] (backing slot) into pool slot first_slot + i, if i < counters[0].
// Every plane's per-slot size is a multiple of 16 bytes.
__global__ __launch_bounds__(kCopyThreads) void k_stage_copy(StagePlanes pl,
                                                             const int32_t* __restrict__ copy_list,
                                                             const int32_t* __restrict__ counters,
                                                             int first_slot, int backing_slots,
                                                             uint32_t* __restrict__ err_flags) {
  const int i = blockIdx.y;
  if (i >= counters[0]) return;
  const int e = copy_list[i];
  if (e < 0 || e >= backing_slots) {
    if (threadIdx.x == 0 && blockIdx.x == 0 && err_flags) atomicOr(err_flags, 1u);
    return;
  }
  const int64_t stride = (int64_t)gridDim.x * kCopyThreads;
#pragma unroll 1
  for (int p = 0; p < kStagePlanes; ++p) {
    const int64_t n16 = pl.bytes[p] / 16;
    const u32x4* __restrict__ src = (const u32x4*)(pl.src[p] + (int64_t)e * pl.bytes[p]);
    u32x4* __restrict__ dst = (u32x4*)(pl.dst[p] + (int64_t)(first_slot + i) * pl.bytes[p]);
    for (int64_t c = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x; c < n16;
         c += stride * kCopyUnroll) {
      u32x4 v[kCopyUnroll];
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t cu = c + u * stride;
        if (cu < n16) v[u] = src[cu];
      }
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t cu = c + u * stride;
        if (cu < n16) dst[cu] = v[u];
      }
    }
  }
}

}  // namespace

hipError_t launch_stage_plan(const int32_t* counts, const int32_t* slot_map, int E,
                             int first_slot, int n_stage, int32_t* slot_map_out,
                             int32_t* copy_list, int32_t* counters, hipStream_t stream) {
  if (E < 1 || E > kPlanThreads || n_stage < 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_stage_plan, dim3(1), dim3(kPlanThreads), 0, stream, counts, slot_map, E,
                     first_slot, n_stage, slot_map_out, copy_list, counters);
  return hipGetLastError();
}

hipError_t launch_stage_copy(const StagePlanes& pl, const int32_t* copy_list,
                             const int32_t* counters, int first_slot, int max_copies,
                             int backing_slots, uint32_t* err_flags, hipStream_t stream) {
  if (max_copies <= 0) return hipSuccess;
  int64_t most = 0;
  for (int p = 0; p < kStagePlanes; ++p) {
    if (pl.bytes[p] % 16) return hipErrorInvalidValue;
    most = pl.bytes[p] > most ? pl.bytes[p] : most;
  }
  // enough workgroups per copy that the largest plane takes a few passes of the unrolled loop
  const int64_t per_wg = (int64_t)kCopyThreads * 16 * kCopyUnroll;
  const int bx = (int)std::min<int64_t>(std::max<int64_t>((most + per_wg - 1) / per_wg, 1), 512);
  hipLaunchKernelGGL(k_stage_copy, dim3(bx, max_copies), dim3(kCopyThreads), 0, stream, pl,
                     copy_list, counters, first_slot, backing_slots, err_flags);
  return hipGetLastError();
}

}  // namespace moe
