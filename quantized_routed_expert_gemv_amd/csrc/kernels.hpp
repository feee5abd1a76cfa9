// Host-side launchers of the layer's kernels (internal to the library; the public
// interface is include/moe.h). Every launcher only enqueues on `stream`.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace moe {

int route_ksplit(int T, int H);
hipError_t launch_route(const uint16_t* x, const uint16_t* wr, const float* bias, int T, int H,
                        int E, int k, int32_t* ids, float* w, float* partial,
                        hipStream_t stream);
// Route + bucket for T <= 16 (route_bucket_fusable): the split router, then one
// single-workgroup kernel that finishes the top-k and bucket-sorts the pairs.
bool route_bucket_fusable(int T, int E);
hipError_t launch_route_bucket_small(const uint16_t* x, const uint16_t* wr, const float* bias,
                                     int T, int H, int E, int k, float* partial, int32_t* ids,
                                     float* w, int32_t* counts, int32_t* offsets, int32_t* perm,
                                     int32_t* inv_perm, hipStream_t stream);

// Route, top-k and bucket for T <= 16, E <= 128 in one single-workgroup launch, which also
// writes the active-expert list act (1 + 4 * E int32; format in route.hip).
bool route_small_ok(int T, int E);
hipError_t launch_route_small(const uint16_t* x, const uint16_t* wr, const float* bias, int T,
                              int H, int E, int k, const int32_t* slot_map, int32_t* ids,
                              float* w, int32_t* counts, int32_t* offsets, int32_t* perm,
                              int32_t* inv_perm, int32_t* act, hipStream_t stream);

// Decode routing split in two: the router's partial logits over route_fused_split(H)
// slices of H (launch_router_partials), finished inside the gate/up kernel
// (launch_gate_up_route). For 1 <= T <= 4, T*E <= 256 and at least 2 slices.
bool route_fused_ok(int T, int H, int E);
int route_fused_split(int H);
// sync (nullable): n_sync int32 that the launch zeroes (the fused decode layer's
// synchronisation words).
hipError_t launch_router_partials(const uint16_t* x, const uint16_t* wr, int T, int H, int E,
                                  int ns, float* partial, hipStream_t stream,
                                  int32_t* sync = nullptr, int n_sync = 0);
// The partials finished by one workgroup (same order as the fused gate/up kernel), with
// or without the counting sort.
hipError_t launch_router_finish(const float* partial, int ns, const float* bias, int T, int E,
                                int k, int32_t* ids, float* w, int32_t* counts,
                                int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                                hipStream_t stream);

size_t bucket_scratch_bytes(int n, int E);
hipError_t launch_bucket(const int32_t* ids, int n, int E, int32_t* counts, int32_t* offsets,
                         int32_t* perm, int32_t* inv_perm, void* scratch, hipStream_t stream);

// act: the small-batch router's active-expert list, or NULL (then the kernel derives the
// active experts from offsets and slot_map).
hipError_t launch_gate_up_gemv(int fmt, const PoolView& gate, const PoolView& up,
                               const int32_t* slot_map, int n_slots, int E, const uint16_t* x,
                               int T, int k, int H, int I, const int32_t* offsets,
                               const int32_t* perm, uint16_t* h, uint32_t* err,
                               const int32_t* act, hipStream_t stream);
hipError_t launch_down_gemv(int fmt, const PoolView& down, const int32_t* slot_map, int n_slots,
                            int E, int T, int k, int H, int I, const int32_t* offsets,
                            const uint16_t* h, float* y, uint32_t* err, hipStream_t stream);
// Gate/up GEMV that first finishes a split router (see RouteIn); every workgroup derives
// its expert from the partials, workgroup 0 stores the routing.
hipError_t launch_gate_up_route(int fmt, const PoolView& gate, const PoolView& up,
                                const int32_t* slot_map, int n_slots, int E, const uint16_t* x,
                                int T, int k, int H, int I, const RouteIn& rin, uint16_t* h,
                                uint32_t* err, hipStream_t stream);
// Down projection + combine in one launch for T*k <= 8 (down_combine_small_ok); needs the
// small-batch router's active-expert list.
bool down_combine_small_ok(int T, int k, int E, int I);
// Whether the small-batch down kernel (rather than one workgroup per row group and expert)
// serves this shape: both the fused layer's tail and the stage down call follow it.
bool down_small_preferred(int fmt, int T, int k, int E, int I);
hipError_t launch_down_combine_small(int fmt, const PoolView& down, int n_slots, int E, int T,
                                     int k, int H, int I, const int32_t* act, const uint16_t* h,
                                     const int32_t* inv_perm, const float* topk_w, float* y,
                                     float* out, uint32_t* err, hipStream_t stream);
// Down projection + combine for the fused decode layer (1 <= T <= 4): one workgroup per
// (16-row group, active expert) of the gate/up kernel's active list; the last workgroup
// of each row group (by ticket) writes out. tickets: int32 [H/16], zeroed by the routed
// gate/up kernel of the same call.
// The fused decode layer (1 <= T <= 4, as route_fused_ok): after the router's partials,
// one persistent kernel finishes the routing, computes gate/up + SwiGLU, the down projection
// and the combine (k_gate_up_routed with a down phase). sync: sync_ints(H) int32, zeroed by
// launch_router_partials of the same call.
bool decode_fused_ok(int T, int H, int E);
hipError_t launch_decode_fused(int fmt, const PoolView& gate, const PoolView& up,
                               const PoolView& down, const int32_t* slot_map, int n_slots, int E,
                               const uint16_t* x, int T, int k, int H, int I, const RouteIn& rin,
                               uint16_t* h, float* y, float* out, int32_t* sync, uint32_t* err,
                               hipStream_t stream);
bool down_ticket_ok(int T, int k, int E);
hipError_t launch_down_ticket(int fmt, const PoolView& down, int n_slots, int E, int T, int k,
                              int H, int I, const int32_t* act, const uint16_t* h,
                              const int32_t* inv_perm, const float* topk_w, float* y,
                              float* out, int32_t* tickets, uint32_t* err, hipStream_t stream);
hipError_t launch_gate_up_grouped(int fmt, const PoolView& gate, const PoolView& up,
                                  const int32_t* slot_map, int n_slots, int E, const uint16_t* x,
                                  int T, int k, int H, int I, const int32_t* offsets,
                                  const int32_t* perm, uint16_t* h, uint32_t* err,
                                  hipStream_t stream);
hipError_t launch_down_grouped(int fmt, const PoolView& down, const int32_t* slot_map,
                               int n_slots, int E, int T, int k, int H, int I,
                               const int32_t* offsets, const uint16_t* h, float* y,
                               uint32_t* err, hipStream_t stream);

hipError_t launch_combine(const float* y, const int32_t* inv_perm, const float* w, int T, int k,
                          int H, float* out, hipStream_t stream);

hipError_t launch_pack(int fmt, int n_mats, int rows, int K, const void* sq, const void* ss,
                       void* dq, void* ds, hipStream_t stream);

// Resident hits and misses (csrc/miss.hip): the list of pairs routed to experts whose slot
// is kSlotMiss, and the merge of the caller's outputs for them.
hipError_t launch_miss_list(const int32_t* slot_map, int E, const int32_t* offsets,
                            const int32_t* perm, int n, int32_t* miss_pos,
                            int32_t* miss_of_pair, int32_t* counters, hipStream_t stream);
hipError_t launch_merge_misses(float* out, const float* y_miss, const int32_t* miss_of_pair,
                               const float* topk_w, int T, int k, int H, hipStream_t stream);

// Staged prefill (csrc/stage.hip): the window plan (mapping rewrite) and the bulk copy of
// the planned experts' planes from a backing store (indexed by expert) into the pool.
hipError_t launch_stage_plan(const int32_t* counts, const int32_t* slot_map, int E,
                             int first_slot, int n_stage, int32_t* slot_map_out,
                             int32_t* copy_list, int32_t* counters, hipStream_t stream);
constexpr int kStagePlanes = 6;   // gate, up, down x (codes, scales)
struct StagePlanes {
  const uint8_t* src[kStagePlanes];   // backing store: slot = expert index
  uint8_t* dst[kStagePlanes];         // pool
  int64_t bytes[kStagePlanes];        // bytes of one slot of each plane (multiple of 16)
};
hipError_t launch_stage_copy(const StagePlanes& pl, const int32_t* copy_list,
                             const int32_t* counters, int first_slot, int max_copies,
                             int backing_slots, uint32_t* err_flags, hipStream_t stream);

}  // namespace moe
