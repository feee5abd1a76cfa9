// C ABI of the routed MoE FFN layer (declared in include/moe.h): argument checking,
// workspace layout and dispatch to the kernels. No call allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/moe.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

moe_status ok() {
  g_err[0] = 0;
  return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool known_fmt(int fmt) {
  return fmt == MOE_W_MXFP4 || fmt == MOE_W_Q8_0 || fmt == MOE_W_Q4_K || fmt == MOE_W_Q5_K ||
         fmt == MOE_W_Q6_K;
}
// k-quant formats: the reduction dimension must be a multiple of the 256-element super-block
bool superblocked(int fmt) { return fmt == MOE_W_Q4_K || fmt == MOE_W_Q5_K || fmt == MOE_W_Q6_K; }

// Launch errors are read back with hipGetLastError; drop any error an earlier, unrelated
// HIP call left behind so it is not reported as this call's failure.
void clear_stale_error() { (void)hipGetLastError(); }

#define CHECK_PTR(p)                                                                 \
  do {                                                                               \
    if ((p) == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", #p);          \
    if (!aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); \
  } while (0)

moe_status check_shape(int32_t T, int32_t H, int32_t E, int32_t k) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %d < 0", T);
  if (H <= 0 || H % 32) return fail(MOE_ERR_INVALID_ARG, "H = %d is not a positive multiple of 32", H);
  if (E < 1 || E > moe::kMaxE) return fail(MOE_ERR_INVALID_ARG, "E = %d outside [1, %d]", E, moe::kMaxE);
  if (k < 1 || k > moe::kMaxK) return fail(MOE_ERR_INVALID_ARG, "k = %d outside [1, %d]", k, moe::kMaxK);
  if (k > E) return fail(MOE_ERR_INVALID_ARG, "k = %d > E = %d", k, E);
  if ((int64_t)T * k > 0x3FFFFFFF) return fail(MOE_ERR_INVALID_ARG, "T*k too large");
  return MOE_OK;
}

// The grouped GEMM addresses gathered activation rows (x, and h for the down projection)
// as 32-bit indices of 16-byte units, so each of x [T x H] and h [T*k x I] must hold fewer
// than 2^35 bf16 elements (64 GiB).
constexpr int64_t kMaxActElems = int64_t(1) << 35;
moe_status check_extent(int32_t T, int32_t k, int32_t H, int32_t I) {
  if ((int64_t)T * H >= kMaxActElems)
    return fail(MOE_ERR_INVALID_ARG, "x holds T*H = %lld elements, limit 2^35",
                (long long)T * H);
  if ((int64_t)T * k * I >= kMaxActElems)
    return fail(MOE_ERR_INVALID_ARG, "h holds T*k*I = %lld elements, limit 2^35",
                (long long)T * k * I);
  return MOE_OK;
}

moe_status check_pool(const moe_pool* pool) {
  if (pool == nullptr) return fail(MOE_ERR_INVALID_ARG, "pool is NULL");
  if (!known_fmt(pool->fmt))
    return fail(MOE_ERR_UNSUPPORTED, "unknown weight format %d", pool->fmt);
  if (pool->n_slots < 1) return fail(MOE_ERR_INVALID_ARG, "n_slots = %d < 1", pool->n_slots);
  if (pool->H <= 0 || pool->H % 32) return fail(MOE_ERR_INVALID_ARG, "pool H = %d", pool->H);
  if (pool->I <= 0 || pool->I % 32) return fail(MOE_ERR_INVALID_ARG, "pool I = %d", pool->I);
  if (superblocked(pool->fmt) && (pool->H % 256 || pool->I % 256))
    return fail(MOE_ERR_INVALID_ARG, "k-quant pools need H and I to be multiples of 256 (H = %d, I = %d)",
                pool->H, pool->I);
  CHECK_PTR(pool->gate_q);
  CHECK_PTR(pool->up_q);
  CHECK_PTR(pool->down_q);
  CHECK_PTR(pool->gate_s);
  CHECK_PTR(pool->up_s);
  CHECK_PTR(pool->down_s);
  return MOE_OK;
}

size_t plane_bytes(int fmt, int64_t rows, int64_t K, bool scales) {
  if (scales) return (size_t)moe::scale_plane_bytes(fmt, rows, K);
  return (size_t)moe::code_plane_bytes(fmt, rows, K);
}

void pool_views(const moe_pool* p, moe::PoolView* g, moe::PoolView* u, moe::PoolView* d) {
  const int fmt = p->fmt;
  const int64_t gq = plane_bytes(fmt, p->I, p->H, false), gs = plane_bytes(fmt, p->I, p->H, true);
  const int64_t dq = plane_bytes(fmt, p->H, p->I, false), ds = plane_bytes(fmt, p->H, p->I, true);
  *g = {(const uint8_t*)p->gate_q, (const uint8_t*)p->gate_s, gq, gs};
  *u = {(const uint8_t*)p->up_q, (const uint8_t*)p->up_s, gq, gs};
  *d = {(const uint8_t*)p->down_q, (const uint8_t*)p->down_s, dq, ds};
}

size_t route_scratch(int32_t T, int32_t H, int32_t E) {
  if (moe::route_fused_ok(T, H, E))          // split router, finished by a later kernel
    return (size_t)moe::route_fused_split(H) * T * E * sizeof(float);
  if (moe::route_small_ok(T, E)) return 0;   // one workgroup, no partials
  const int ks = moe::route_ksplit(T, H);
  return ks > 1 ? (size_t)ks * T * E * sizeof(float) : 0;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool use_gemv(int32_t path, int32_t T) {
  return path == MOE_PATH_GEMV || path == MOE_PATH_PERSISTENT ||
         (path == MOE_PATH_AUTO && T <= 16);
}

moe_status gate_up_dispatch(const moe_pool* pool, const int32_t* slot_map, int32_t E,
                            const uint16_t* x, int32_t T, int32_t k, const int32_t* offsets,
                            const int32_t* perm, uint16_t* h, uint32_t* err, int32_t path,
                            hipStream_t stream, const int32_t* act = nullptr) {
  clear_stale_error();
  moe::PoolView g, u, d;
  pool_views(pool, &g, &u, &d);
  if (use_gemv(path, T))
    return hip_status(moe::launch_gate_up_gemv(pool->fmt, g, u, slot_map, pool->n_slots, E, x, T,
                                               k, pool->H, pool->I, offsets, perm, h, err, act,
                                               stream),
                      "gate/up (GEMV)");
  return hip_status(moe::launch_gate_up_grouped(pool->fmt, g, u, slot_map, pool->n_slots, E, x, T,
                                                k, pool->H, pool->I, offsets, perm, h, err, stream),
                    "gate/up (grouped GEMM)");
}

moe_status down_dispatch(const moe_pool* pool, const int32_t* slot_map, int32_t E, int32_t T,
                         int32_t k, const int32_t* offsets, const uint16_t* h, float* y,
                         uint32_t* err, int32_t path, hipStream_t stream) {
  clear_stale_error();
  moe::PoolView g, u, d;
  pool_views(pool, &g, &u, &d);
  if (use_gemv(path, T))
    return hip_status(moe::launch_down_gemv(pool->fmt, d, slot_map, pool->n_slots, E, T, k,
                                            pool->H, pool->I, offsets, h, y, err, stream),
                      "down (GEMV)");
  return hip_status(moe::launch_down_grouped(pool->fmt, d, slot_map, pool->n_slots, E, T, k,
                                             pool->H, pool->I, offsets, h, y, err, stream),
                    "down (grouped GEMM)");
}

moe_status ffn_dispatch(const moe_pool* pool, const int32_t* slot_map, int32_t E,
                        const uint16_t* x, int32_t T, int32_t k, const int32_t* offsets,
                        const int32_t* perm, uint16_t* h, float* y, uint32_t* err,
                        int32_t path, hipStream_t stream) {
  moe_status s = gate_up_dispatch(pool, slot_map, E, x, T, k, offsets, perm, h, err, path, stream);
  if (s != MOE_OK) return s;
  return down_dispatch(pool, slot_map, E, T, k, offsets, h, y, err, path, stream);
}

// Shared argument checks of the expert-FFN entry points.
moe_status check_ffn_args(const moe_pool* pool, const int32_t* slot_map, int32_t E, int32_t T,
                          int32_t k, const int32_t* offsets, uint32_t* err_flags, int32_t path) {
  moe_status s = check_pool(pool);
  if (s != MOE_OK) return s;
  s = check_shape(T, pool->H, E, k);
  if (s != MOE_OK) return s;
  s = check_extent(T, k, pool->H, pool->I);
  if (s != MOE_OK) return s;
  if (path < MOE_PATH_AUTO || path > MOE_PATH_PERSISTENT)
    return fail(MOE_ERR_INVALID_ARG, "path = %d", path);
  if (T == 0) return MOE_OK;
  CHECK_PTR(slot_map);
  CHECK_PTR(offsets);
  if (err_flags != nullptr && ((uintptr_t)err_flags & 3))
    return fail(MOE_ERR_INVALID_ARG, "err_flags misaligned");
  return MOE_OK;
}

}  // namespace

// ---- moe_layer_noalloc: moe_layer with its workspace in a file-scope device array

// One array per device, held for the life of the process. In host code its name is only a
// stand-in for the symbol: kernels are given the device address that hipGetSymbolAddress
// returns for the current device, never the name itself.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_WS_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // address of `scratch` on each device, looked up once

// The device address of `scratch` on the device that `stream` belongs to, looked up (with
// that device current) on the first call for the device.
moe_status noalloc_workspace(hipStream_t stream, void** out) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t d = -1;
    e = hipStreamGetDevice(stream, &d);
    if (e != hipSuccess) return hip_status(e, "hipStreamGetDevice");
    dev = (int)d;
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_INVALID_ARG, "device %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e, "hipSetDevice");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = dev != cur ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (back != hipSuccess) return hip_status(back, "hipSetDevice (restore)");
    if (p == nullptr || ((uintptr_t)p & 255))
      return fail(MOE_ERR_HIP, "static workspace at %p is not 256-byte aligned", p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "unknown moe_status";
}

const char* moe_last_error(void) { return g_err; }

size_t moe_plane_bytes(int32_t fmt, int32_t rows, int32_t K, int32_t scales) {
  if (!known_fmt(fmt) || rows < 0 || K < 0 || (superblocked(fmt) && K % 256)) return 0;
  return plane_bytes(fmt, rows, K, scales != 0);
}

moe_status moe_pool_pack(int32_t fmt, int32_t n_mats, int32_t rows, int32_t K,
                         const void* src_q, const void* src_s, void* dst_q, void* dst_s,
                         void* stream) {
  if (!known_fmt(fmt)) return fail(MOE_ERR_UNSUPPORTED, "unknown weight format %d", fmt);
  if (n_mats < 0 || rows < 0 || K < 0) return fail(MOE_ERR_INVALID_ARG, "negative size");
  if (rows % 16) return fail(MOE_ERR_INVALID_ARG, "rows = %d is not a multiple of 16", rows);
  if (K % 32) return fail(MOE_ERR_INVALID_ARG, "K = %d is not a multiple of 32", K);
  if (superblocked(fmt) && K % 256)
    return fail(MOE_ERR_INVALID_ARG, "k-quants need K = %d to be a multiple of 256", K);
  if (n_mats == 0 || rows == 0 || K == 0) return ok();
  CHECK_PTR(src_q);
  CHECK_PTR(dst_q);
  if (src_s == nullptr || dst_s == nullptr) return fail(MOE_ERR_INVALID_ARG, "scale plane is NULL");
  if (fmt == MOE_W_Q8_0 && (((uintptr_t)src_s | (uintptr_t)dst_s) & 1))
    return fail(MOE_ERR_INVALID_ARG, "fp16 scale plane is not 2-byte aligned");
  clear_stale_error();
  return hip_status(moe::launch_pack(fmt, n_mats, rows, K, src_q, src_s, dst_q, dst_s,
                                     (hipStream_t)stream),
                    "pool pack");
}

size_t moe_route_scratch_bytes(int32_t T, int32_t H, int32_t E) {
  if (T <= 0 || H <= 0 || E <= 0) return 0;
  return route_scratch(T, H, E);
}

moe_status moe_route(const uint16_t* x, const uint16_t* w_router, const float* bias, int32_t T,
                     int32_t H, int32_t E, int32_t k, int32_t* topk_ids, float* topk_w,
                     void* scratch, size_t scratch_bytes, void* stream) {
  moe_status s = check_shape(T, H, E, k);
  if (s != MOE_OK) return s;
  if (T == 0) return ok();
  CHECK_PTR(x);
  CHECK_PTR(w_router);
  CHECK_PTR(topk_ids);
  CHECK_PTR(topk_w);
  if (bias != nullptr && ((uintptr_t)bias & 3)) return fail(MOE_ERR_INVALID_ARG, "bias misaligned");
  const size_t need = route_scratch(T, H, E);
  if (need) {
    CHECK_PTR(scratch);
    if (scratch_bytes < need)
      return fail(MOE_ERR_INVALID_ARG, "route scratch %zu bytes < %zu needed", scratch_bytes, need);
  }
  clear_stale_error();
  return hip_status(moe::launch_route(x, w_router, bias, T, H, E, k, topk_ids, topk_w,
                                      (float*)scratch, (hipStream_t)stream),
                    "route");
}

size_t moe_bucket_scratch_bytes(int32_t T, int32_t k, int32_t E) {
  if (T <= 0 || k <= 0 || E <= 0) return 0;
  return moe::bucket_scratch_bytes(T * k, E);
}

moe_status moe_bucket(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t* counts,
                      int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* scratch,
                      size_t scratch_bytes, void* stream) {
  moe_status s = check_shape(T, 32, E, k);
  if (s != MOE_OK) return s;
  CHECK_PTR(counts);
  CHECK_PTR(offsets);
  clear_stale_error();
  if (T == 0)   // empty input: one small kernel still writes all-zero counts and offsets
    return hip_status(moe::launch_bucket(nullptr, 0, E, counts, offsets, nullptr, nullptr,
                                         nullptr, (hipStream_t)stream),
                      "bucket");
  CHECK_PTR(topk_ids);
  CHECK_PTR(perm);
  CHECK_PTR(inv_perm);
  const size_t need = moe::bucket_scratch_bytes(T * k, E);
  if (need) {
    CHECK_PTR(scratch);
    if (scratch_bytes < need)
      return fail(MOE_ERR_INVALID_ARG, "bucket scratch %zu bytes < %zu needed", scratch_bytes, need);
  }
  return hip_status(moe::launch_bucket(topk_ids, T * k, E, counts, offsets, perm, inv_perm,
                                       scratch, (hipStream_t)stream),
                    "bucket");
}

moe_status moe_expert_ffn(const moe_pool* pool, const int32_t* slot_map, int32_t E,
                          const uint16_t* x, int32_t T, int32_t k, const int32_t* offsets,
                          const int32_t* perm, uint16_t* h, float* y, uint32_t* err_flags,
                          int32_t path, void* stream) {
  moe_status s = check_ffn_args(pool, slot_map, E, T, k, offsets, err_flags, path);
  if (s != MOE_OK || T == 0) return s == MOE_OK ? ok() : s;
  CHECK_PTR(x);
  CHECK_PTR(perm);
  CHECK_PTR(h);
  CHECK_PTR(y);
  return ffn_dispatch(pool, slot_map, E, x, T, k, offsets, perm, h, y, err_flags, path,
                      (hipStream_t)stream);
}

moe_status moe_expert_gate_up(const moe_pool* pool, const int32_t* slot_map, int32_t E,
                              const uint16_t* x, int32_t T, int32_t k, const int32_t* offsets,
                              const int32_t* perm, uint16_t* h, uint32_t* err_flags,
                              int32_t path, void* stream) {
  moe_status s = check_ffn_args(pool, slot_map, E, T, k, offsets, err_flags, path);
  if (s != MOE_OK || T == 0) return s == MOE_OK ? ok() : s;
  CHECK_PTR(x);
  CHECK_PTR(perm);
  CHECK_PTR(h);
  return gate_up_dispatch(pool, slot_map, E, x, T, k, offsets, perm, h, err_flags, path,
                          (hipStream_t)stream);
}

moe_status moe_expert_down(const moe_pool* pool, const int32_t* slot_map, int32_t E, int32_t T,
                           int32_t k, const int32_t* offsets, const uint16_t* h, float* y,
                           uint32_t* err_flags, int32_t path, void* stream) {
  moe_status s = check_ffn_args(pool, slot_map, E, T, k, offsets, err_flags, path);
  if (s != MOE_OK || T == 0) return s == MOE_OK ? ok() : s;
  CHECK_PTR(h);
  CHECK_PTR(y);
  return down_dispatch(pool, slot_map, E, T, k, offsets, h, y, err_flags, path,
                       (hipStream_t)stream);
}

moe_status moe_combine(const float* y, const int32_t* inv_perm, const float* topk_w, int32_t T,
                       int32_t k, int32_t H, float* out, void* stream) {
  moe_status s = check_shape(T, H, moe::kMaxE, k);
  if (s != MOE_OK) return s;
  if (T == 0) return ok();
  CHECK_PTR(y);
  CHECK_PTR(inv_perm);
  CHECK_PTR(topk_w);
  CHECK_PTR(out);
  clear_stale_error();
  return hip_status(moe::launch_combine(y, inv_perm, topk_w, T, k, H, out, (hipStream_t)stream),
                    "combine");
}

moe_status moe_miss_list(const int32_t* slot_map, int32_t E, const int32_t* offsets,
                         const int32_t* perm, int32_t T, int32_t k, int32_t* miss_pos,
                         int32_t* miss_of_pair, int32_t* counters, void* stream) {
  moe_status s = check_shape(T, 32, E, k);
  if (s != MOE_OK) return s;
  CHECK_PTR(slot_map);
  CHECK_PTR(offsets);
  CHECK_PTR(counters);
  if (T > 0) {
    CHECK_PTR(perm);
    CHECK_PTR(miss_pos);
    CHECK_PTR(miss_of_pair);
  }
  clear_stale_error();
  return hip_status(moe::launch_miss_list(slot_map, E, offsets, perm, T * k, miss_pos,
                                          miss_of_pair, counters, (hipStream_t)stream),
                    "miss list");
}

moe_status moe_merge_misses(float* out, const float* y_miss, const int32_t* miss_of_pair,
                            const float* topk_w, int32_t T, int32_t k, int32_t H,
                            void* stream) {
  moe_status s = check_shape(T, H, moe::kMaxE, k);
  if (s != MOE_OK) return s;
  if (T == 0) return ok();
  CHECK_PTR(out);
  CHECK_PTR(y_miss);
  CHECK_PTR(miss_of_pair);
  CHECK_PTR(topk_w);
  clear_stale_error();
  return hip_status(moe::launch_merge_misses(out, y_miss, miss_of_pair, topk_w, T, k, H,
                                             (hipStream_t)stream),
                    "merge misses");
}

moe_status moe_stage_plan(const int32_t* counts, const int32_t* slot_map, int32_t E,
                          int32_t first_slot, int32_t n_stage, int32_t* slot_map_out,
                          int32_t* copy_list, int32_t* counters, void* stream) {
  if (E < 1 || E > moe::kMaxE) return fail(MOE_ERR_INVALID_ARG, "E = %d outside [1, %d]", E, moe::kMaxE);
  if (first_slot < 0 || n_stage < 0)
    return fail(MOE_ERR_INVALID_ARG, "first_slot = %d, n_stage = %d", first_slot, n_stage);
  if ((int64_t)first_slot + n_stage > 0x7fffffff) return fail(MOE_ERR_INVALID_ARG, "window too large");
  CHECK_PTR(counts);
  CHECK_PTR(slot_map);
  CHECK_PTR(slot_map_out);
  CHECK_PTR(copy_list);
  CHECK_PTR(counters);
  clear_stale_error();
  return hip_status(moe::launch_stage_plan(counts, slot_map, E, first_slot, n_stage,
                                           slot_map_out, copy_list, counters,
                                           (hipStream_t)stream),
                    "stage plan");
}

moe_status moe_stage_copy(const moe_pool* pool, const moe_pool* backing,
                          const int32_t* copy_list, const int32_t* counters, int32_t first_slot,
                          int32_t max_copies, uint32_t* err_flags, void* stream) {
  moe_status s = check_pool(pool);
  if (s != MOE_OK) return s;
  s = check_pool(backing);
  if (s != MOE_OK) return s;
  if (backing->fmt != pool->fmt || backing->H != pool->H || backing->I != pool->I)
    return fail(MOE_ERR_INVALID_ARG, "backing store and pool differ in format or shape");
  if (first_slot < 0 || max_copies < 0 || (int64_t)first_slot + max_copies > pool->n_slots)
    return fail(MOE_ERR_INVALID_ARG, "window [%d, %d + %d) outside the pool's %d slots",
                first_slot, first_slot, max_copies, pool->n_slots);
  if (max_copies > moe::kMaxE)
    return fail(MOE_ERR_INVALID_ARG, "max_copies = %d > %d", max_copies, moe::kMaxE);
  if (max_copies == 0) return ok();
  CHECK_PTR(copy_list);
  CHECK_PTR(counters);
  const int fmt = pool->fmt, H = pool->H, I = pool->I;
  moe::StagePlanes pl;
  const void* src[6] = {backing->gate_q, backing->gate_s, backing->up_q,
                        backing->up_s,   backing->down_q, backing->down_s};
  const void* dst[6] = {pool->gate_q, pool->gate_s, pool->up_q,
                        pool->up_s,   pool->down_q, pool->down_s};
  for (int p = 0; p < moe::kStagePlanes; ++p) {
    const bool down = p >= 4, scales = p % 2 == 1;
    pl.src[p] = (const uint8_t*)src[p];
    pl.dst[p] = (uint8_t*)const_cast<void*>(dst[p]);
    pl.bytes[p] = (int64_t)plane_bytes(fmt, down ? H : I, down ? I : H, scales);
  }
  clear_stale_error();
  return hip_status(moe::launch_stage_copy(pl, copy_list, counters, first_slot, max_copies,
                                           backing->n_slots, err_flags, (hipStream_t)stream),
                    "stage copy");
}

moe_status moe_layer_workspace(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                               moe_ws_layout* out) {
  if (out == nullptr) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
  moe_status s = check_shape(T, H, E, k);
  if (s != MOE_OK) return s;
  if (I <= 0 || I % 32) return fail(MOE_ERR_INVALID_ARG, "I = %d", I);
  s = check_extent(T, k, H, I);
  if (s != MOE_OK) return s;
  const size_t n = (size_t)T * k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  out->topk_ids = take(n * 4);
  out->topk_w = take(n * 4);
  out->counts = take((size_t)E * 4);
  out->offsets = take((size_t)(E + 1) * 4);
  out->perm = take(n * 4);
  out->inv_perm = take(n * 4);
  out->h = take(n * I * 2);
  out->y = take(n * H * 4);
  const size_t rs = T > 0 ? route_scratch(T, H, E) : 0;
  const size_t bs = T > 0 ? moe::bucket_scratch_bytes((int)n, E) : 0;
  out->scratch = take(rs > bs ? rs : bs);
  out->act = take((size_t)moe::act_ints(E) * sizeof(int32_t));
  out->sync = take((size_t)moe::sync_ints(H) * sizeof(int32_t));
  out->total = off;
  return ok();
}

// Down projection and combine of the fused layer. With the small-batch active-expert list
// (act != NULL) and few pairs, one kernel does both.
static moe_status down_combine_tail(const moe_pool* pool, const int32_t* slot_map, int32_t E,
                                    int32_t T, int32_t k, const int32_t* offsets,
                                    const int32_t* act, const uint16_t* h,
                                    const int32_t* inv_perm, const float* w, float* y,
                                    float* out, uint32_t* err_flags, int32_t path,
                                    hipStream_t st, int32_t* tickets = nullptr) {
  const bool small = moe::down_small_preferred(pool->fmt, T, k, E, pool->I);
  if (act != nullptr && tickets != nullptr && use_gemv(path, T) && !small &&
      moe::down_ticket_ok(T, k, E)) {
    // decode: the tickets were zeroed by the routed gate/up kernel
    clear_stale_error();
    moe::PoolView g, u, d;
    pool_views(pool, &g, &u, &d);
    return hip_status(moe::launch_down_ticket(pool->fmt, d, pool->n_slots, E, T, k, pool->H,
                                              pool->I, act, h, inv_perm, w, y, out, tickets,
                                              err_flags, st),
                      "down+combine (tickets)");
  }
  if (act != nullptr && use_gemv(path, T) && small) {
    clear_stale_error();
    moe::PoolView g, u, d;
    pool_views(pool, &g, &u, &d);
    return hip_status(moe::launch_down_combine_small(pool->fmt, d, pool->n_slots, E, T, k, pool->H,
                                                     pool->I, act, h, inv_perm, w, y, out,
                                                     err_flags, st),
                      "down+combine");
  }
  moe_status s = down_dispatch(pool, slot_map, E, T, k, offsets, h, y, err_flags, path, st);
  if (s != MOE_OK) return s;
  clear_stale_error();
  return hip_status(moe::launch_combine(y, inv_perm, w, T, k, pool->H, out, st), "combine");
}

// Record a timing event; inside a stream capture it becomes an event-record node of the
// graph (so replays can still be timed).
static moe_status record_event(hipEvent_t ev, hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(st, &cs);
  if (e != hipSuccess) return hip_status(e, "event record: stream capture query");
  if (cs == hipStreamCaptureStatusActive)
    return hip_status(hipEventRecordWithFlags(ev, st, hipEventRecordExternal),
                      "event record (external, in capture)");
  return hip_status(hipEventRecord(ev, st), "event record");
}

static moe_status layer_impl(const moe_pool* pool, const int32_t* slot_map,
                             const uint16_t* w_router, const float* bias, const uint16_t* x,
                             int32_t T, int32_t E, int32_t k, float* out, void* workspace,
                             size_t workspace_bytes, uint32_t* err_flags, int32_t path,
                             void* stream, void* ev_begin, void* ev_end) {
  moe_status s = check_pool(pool);
  if (s != MOE_OK) return s;
  s = check_shape(T, pool->H, E, k);
  if (s != MOE_OK) return s;
  s = check_extent(T, k, pool->H, pool->I);
  if (s != MOE_OK) return s;
  if (path < MOE_PATH_AUTO || path > MOE_PATH_PERSISTENT)
    return fail(MOE_ERR_INVALID_ARG, "path = %d", path);
  if (T == 0) return ok();
  CHECK_PTR(slot_map);
  CHECK_PTR(w_router);
  CHECK_PTR(x);
  CHECK_PTR(out);
  if (bias != nullptr && ((uintptr_t)bias & 3)) return fail(MOE_ERR_INVALID_ARG, "bias misaligned");
  if (workspace == nullptr || ((uintptr_t)workspace & 255))
    return fail(MOE_ERR_INVALID_ARG, "workspace is NULL or not 256-byte aligned");
  if (err_flags != nullptr && ((uintptr_t)err_flags & 3))
    return fail(MOE_ERR_INVALID_ARG, "err_flags misaligned");
  moe_ws_layout L;
  s = moe_layer_workspace(T, pool->H, pool->I, E, k, &L);
  if (s != MOE_OK) return s;
  if (workspace_bytes < L.total)
    return fail(MOE_ERR_INVALID_ARG, "workspace %zu bytes < %zu needed", workspace_bytes, L.total);
  char* ws = (char*)workspace;
  int32_t* ids = (int32_t*)(ws + L.topk_ids);
  float* w = (float*)(ws + L.topk_w);
  int32_t* counts = (int32_t*)(ws + L.counts);
  int32_t* offsets = (int32_t*)(ws + L.offsets);
  int32_t* perm = (int32_t*)(ws + L.perm);
  int32_t* inv_perm = (int32_t*)(ws + L.inv_perm);
  uint16_t* h = (uint16_t*)(ws + L.h);
  float* y = (float*)(ws + L.y);
  void* scratch = ws + L.scratch;
  int32_t* act = (int32_t*)(ws + L.act);
  int32_t* sync = (int32_t*)(ws + L.sync);   // tickets first, then the hand-off counters
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  bool have_act = false;
  clear_stale_error();
  // route + bucket: for small batches the split router is finished (top-k and counting
  // sort) by one single-workgroup kernel; otherwise router, then the counting sort
  const bool gemv = use_gemv(path, T);
  if (moe::route_fused_ok(T, pool->H, E)) {
    // router partials over slices of H; the gate/up GEMV finishes the routing itself (or,
    // for the grouped path, one workgroup finishes it and bucket-sorts)
    const int ns = moe::route_fused_split(pool->H);
    const bool fused = path == MOE_PATH_PERSISTENT && moe::decode_fused_ok(T, pool->H, E);
    e = moe::launch_router_partials(x, w_router, T, pool->H, E, ns, (float*)scratch, st,
                                    fused ? sync : nullptr, moe::sync_ints(pool->H));
    if (e != hipSuccess) return hip_status(e, "router");
    if (fused) {
      // one persistent kernel: routing, gate/up + SwiGLU, down and combine
      if (ev_begin != nullptr) {
        s = record_event((hipEvent_t)ev_begin, st);
        if (s != MOE_OK) return s;
      }
      moe::PoolView g, u, d;
      pool_views(pool, &g, &u, &d);
      const moe::RouteIn rin{(const float*)scratch, ns, bias, T, ids, w, counts, offsets, perm,
                             inv_perm, act, nullptr, 0};
      clear_stale_error();
      e = moe::launch_decode_fused(pool->fmt, g, u, d, slot_map, pool->n_slots, E, x, T, k,
                                   pool->H, pool->I, rin, h, y, out, sync, err_flags, st);
      if (e != hipSuccess) return hip_status(e, "fused decode layer");
      if (ev_end != nullptr) return record_event((hipEvent_t)ev_end, st);
      return ok();
    }
    if (gemv) {
      if (ev_begin != nullptr) {
        s = record_event((hipEvent_t)ev_begin, st);
        if (s != MOE_OK) return s;
      }
      moe::PoolView g, u, d;
      pool_views(pool, &g, &u, &d);
      const moe::RouteIn rin{(const float*)scratch, ns, bias, T, ids, w, counts, offsets, perm,
                             inv_perm, act, sync, pool->H / 16};
      clear_stale_error();
      e = moe::launch_gate_up_route(pool->fmt, g, u, slot_map, pool->n_slots, E, x, T, k,
                                    pool->H, pool->I, rin, h, err_flags, st);
      if (e != hipSuccess) return hip_status(e, "route + gate/up (GEMV)");
      if (ev_end != nullptr) {
        s = record_event((hipEvent_t)ev_end, st);
        if (s != MOE_OK) return s;
      }
      return down_combine_tail(pool, slot_map, E, T, k, offsets, act, h, inv_perm, w, y, out,
                               err_flags, path, st, sync);
    }
    e = moe::launch_router_finish((const float*)scratch, ns, bias, T, E, k, ids, w, counts,
                                  offsets, perm, inv_perm, st);
    if (e != hipSuccess) return hip_status(e, "route+bucket");
  } else if (moe::route_small_ok(T, E)) {
    // one workgroup: router, top-k, counting sort and the active-expert list
    e = moe::launch_route_small(x, w_router, bias, T, pool->H, E, k, slot_map, ids, w, counts,
                                offsets, perm, inv_perm, act, st);
    if (e != hipSuccess) return hip_status(e, "route+bucket");
    have_act = true;
  } else if (moe::route_bucket_fusable(T, E)) {
    e = moe::launch_route_bucket_small(x, w_router, bias, T, pool->H, E, k, (float*)scratch, ids,
                                       w, counts, offsets, perm, inv_perm, st);
    if (e != hipSuccess) return hip_status(e, "route+bucket");
  } else {
    e = moe::launch_route(x, w_router, bias, T, pool->H, E, k, ids, w, (float*)scratch, st);
    if (e != hipSuccess) return hip_status(e, "route");
    e = moe::launch_bucket(ids, T * k, E, counts, offsets, perm, inv_perm, scratch, st);
    if (e != hipSuccess) return hip_status(e, "bucket");
  }
  if (ev_begin != nullptr) {
    s = record_event((hipEvent_t)ev_begin, st);
    if (s != MOE_OK) return s;
  }
  s = gate_up_dispatch(pool, slot_map, E, x, T, k, offsets, perm, h, err_flags, path, st,
                       have_act ? act : nullptr);
  if (s != MOE_OK) return s;
  if (ev_end != nullptr) {
    s = record_event((hipEvent_t)ev_end, st);
    if (s != MOE_OK) return s;
  }
  return down_combine_tail(pool, slot_map, E, T, k, offsets, have_act ? act : nullptr, h,
                           inv_perm, w, y, out, err_flags, path, st);
}

moe_status moe_layer(const moe_pool* pool, const int32_t* slot_map, const uint16_t* w_router,
                     const float* bias, const uint16_t* x, int32_t T, int32_t E, int32_t k,
                     float* out, void* workspace, size_t workspace_bytes, uint32_t* err_flags,
                     int32_t path, void* stream) {
  return layer_impl(pool, slot_map, w_router, bias, x, T, E, k, out, workspace, workspace_bytes,
                    err_flags, path, stream, nullptr, nullptr);
}

moe_status moe_layer_noalloc(const moe_pool* pool, const int32_t* slot_map,
                             const uint16_t* w_router, const float* bias, const uint16_t* x,
                             int32_t T, int32_t E, int32_t k, float* out, uint32_t* err_flags,
                             int32_t path, void* stream) {
  moe_status s = check_pool(pool);
  if (s != MOE_OK) return s;
  s = check_shape(T, pool->H, E, k);
  if (s != MOE_OK) return s;
  if (T == 0) return ok();
  moe_ws_layout L;
  s = moe_layer_workspace(T, pool->H, pool->I, E, k, &L);
  if (s != MOE_OK) return s;
  if (L.total > (size_t)MOE_NOALLOC_WS_BYTES)
    return fail(MOE_ERR_INVALID_ARG,
                "moe_layer_noalloc: the layer needs %zu bytes of workspace, more than the "
                "%zu-byte static workspace (T = %d; use moe_layer with a caller workspace)",
                L.total, (size_t)MOE_NOALLOC_WS_BYTES, T);
  void* ws = nullptr;
  s = noalloc_workspace((hipStream_t)stream, &ws);
  if (s != MOE_OK) return s;
  return layer_impl(pool, slot_map, w_router, bias, x, T, E, k, out, ws, MOE_NOALLOC_WS_BYTES,
                    err_flags, path, stream, nullptr, nullptr);
}

moe_status moe_layer_timed(const moe_pool* pool, const int32_t* slot_map,
                           const uint16_t* w_router, const float* bias, const uint16_t* x,
                           int32_t T, int32_t E, int32_t k, float* out, void* workspace,
                           size_t workspace_bytes, uint32_t* err_flags, int32_t path,
                           void* stream, void* ev_gate_up_begin, void* ev_gate_up_end) {
  return layer_impl(pool, slot_map, w_router, bias, x, T, E, k, out, workspace, workspace_bytes,
                    err_flags, path, stream, ev_gate_up_begin, ev_gate_up_end);
}

}  // extern "C"
