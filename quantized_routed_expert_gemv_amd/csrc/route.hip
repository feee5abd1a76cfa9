// Router GEMV + top-k + softmax over the chosen k.
//
// The router stays on the GPU (llama.cpp discussion "fixed GPU expert working set with
// Native CPU miss execution", original post); GPT-OSS-20B routes each token to 4 of 32
// experts (tinyserve README, "Performance").
//
// logits[t, e] = sum_h x[t, h] * Wr[e, h] (+ bias[e]) is a [T x H] x [H x E] contraction.
// It runs on bf16 MFMA (v_mfma_f32_16x16x32_bf16): bf16 products are exact in fp32 and
// accumulate in fp32. A workgroup owns 16 tokens and all E experts; its 4 waves split the
// reduction dimension and their partial tiles are summed in LDS in a fixed order, so the
// result is deterministic. For small T the reduction dimension is also split across
// workgroups and a later kernel (a single-workgroup finish, or every workgroup of the
// decode gate/up kernel) sums the partials in a fixed order, takes the top-k and, in the
// fused layer, also bucket-sorts the pairs; the decode split runs one wave per slice
// (k_router_part), whose few steps need no reduction across waves. A kernel
// boundary, not an arrival counter, hands the partials over: on this chip a device-scope
// release in every workgroup writes back the whole L2 of its XCD, which costs far more
// than a launch.
#include "common.hpp"
#include "bucket_dev.hpp"
#include "kernels.hpp"
#include "topk_dev.hpp"

namespace moe {

namespace {

constexpr int kRouteTok = 16;   // tokens per workgroup (one MFMA row tile)
constexpr int kRouteWaves = 4;
constexpr int kMaxSplit = kMaxRouteSplit;   // largest split of the reduction dimension

// Partial logits of tokens [t0, t0 + 16) over this workgroup's share (split z of nsplit) of
// the reduction dimension, summed over the NW waves in a fixed order into red[0][token][e]
// (red holds 4 wave slots: with 8 waves, wave w + 4 first adds its tile to wave w's).
// Each wave issues the loads of RB 32-wide steps before the MFMAs that consume them; rows
// past T or E are loaded from a valid row and zeroed when consumed.
template <int NF, int NW, int RB>
__device__ void router_tile(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                            int T, int H, int E, int t0, int z, int nsplit,
                            float (*red)[kRouteTok][NF * 16]) {
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nsteps = H / 32;
  // splits cover whole pairs of 32-wide steps, so no 128-byte line of a row is split
  // between two workgroups (which may sit on different XCDs and both fetch it)
  const int npairs = (nsteps + 1) / 2;
  const int s_begin = 2 * (int)((int64_t)npairs * z / nsplit);
  const int s_end = min(nsteps, 2 * (int)((int64_t)npairs * (z + 1) / nsplit));
  const int row = lane & 15;        // token (A) / expert (B) within the 16-tile
  const int kq = (lane >> 4) * 8;   // this lane's 8-element slice of the 32-step
  const bool tok_ok = t0 + row < T;
  const uint16_t* xr = x + (int64_t)(tok_ok ? t0 + row : 0) * H + kq;
  const uint16_t* wrow[NF];
  bool e_ok[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    e_ok[f] = f * 16 + row < E;
    wrow[f] = wr + (int64_t)(e_ok[f] ? f * 16 + row : 0) * H + kq;
  }
  f32x4 acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4 zero = {0, 0, 0, 0};
  for (int s0 = s_begin + wave; s0 < s_end; s0 += NW * RB) {
    u32x4 a[RB], bq[RB][NF];
    bool ok[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int s = s0 + r * NW;
      ok[r] = s < s_end;
      const int ss = ok[r] ? s : s_begin;
      a[r] = *(const u32x4*)(xr + ss * 32);
#pragma unroll
      for (int f = 0; f < NF; ++f) bq[r][f] = *(const u32x4*)(wrow[f] + ss * 32);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, (ok[r] && tok_ok) ? a[r] : zero);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const bf16x8 bv = __builtin_bit_cast(bf16x8, e_ok[f] ? bq[r][f] : zero);
        acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[f], 0, 0, 0);
      }
    }
  }
  // lane holds D[token 4*(lane/16)+v][expert 16f + lane%16]
  if (wave < 4) {
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][4 * (lane >> 4) + v][f * 16 + row] = acc[f][v];
  }
  __syncthreads();
  if (NW == 8 && wave >= 4) {
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave - 4][4 * (lane >> 4) + v][f * 16 + row] += acc[f][v];
  }
  if (NW == 8) __syncthreads();
  for (int i = threadIdx.x; i < kRouteTok * NF * 16; i += NW * kWave) {
    int tt = i / (NF * 16), e = i % (NF * 16);
    float sum = red[0][tt][e];
#pragma unroll
    for (int q = 1; q < 4; ++q) sum += red[q][tt][e];
    red[0][tt][e] = sum;
  }
  __syncthreads();
}

// Steps per load batch for NF expert tiles: as many as fit in about 144 VGPRs
// (4 VGPRs per 16-byte operand, 1 + NF operands per step).
template <int NF>
constexpr int router_rb() { return 144 / (4 * (1 + NF)) > 0 ? 144 / (4 * (1 + NF)) : 1; }

template <int NF>   // NF = ceil(E / 16) expert tiles
__global__ __launch_bounds__(256) void k_router(const uint16_t* __restrict__ x,
                                                const uint16_t* __restrict__ wr,
                                                const float* __restrict__ bias, int T, int H,
                                                int E, int k, float* __restrict__ partial,
                                                int32_t* __restrict__ ids,
                                                float* __restrict__ w) {
  __shared__ float red[kRouteWaves][kRouteTok][NF * 16];
  __shared__ TopkScratch tks[kRouteWaves];
  const int wave = threadIdx.x / kWave;
  const int t0 = blockIdx.x * kRouteTok;
  router_tile<NF, kRouteWaves, router_rb<NF>()>(x, wr, T, H, E, t0, blockIdx.y, gridDim.y, red);
  if (gridDim.y > 1) {
    float* dst = partial + (int64_t)blockIdx.y * T * E;
    for (int i = threadIdx.x; i < kRouteTok * E; i += blockDim.x) {
      int tt = i / E, e = i % E;
      if (t0 + tt < T) dst[(int64_t)(t0 + tt) * E + e] = red[0][tt][e];
    }
    return;
  }
  if (bias != nullptr) {
    for (int i = threadIdx.x; i < kRouteTok * E; i += blockDim.x) {
      int tt = i / E, e = i % E;
      red[0][tt][e] += bias[e];
    }
    __syncthreads();
  }
  for (int tt = wave; tt < kRouteTok; tt += kRouteWaves) {
    if (t0 + tt >= T) break;
    wave_topk_softmax(&red[0][tt][0], E, k, ids + (int64_t)(t0 + tt) * k,
                      w + (int64_t)(t0 + tt) * k, tks[wave]);
  }
}

// Partial logits of the split router for a small batch (T <= 16): one wave per slice z of
// the reduction dimension (the slices of router_tile, whole pairs of 32-wide steps) and
// group blockIdx.y of NF 16-expert tiles, its steps accumulated in increasing order in one
// MFMA chain and stored from registers as partial[z][t][e]. A slice holds at most a few
// steps, so the wave issues the loads of RB steps before the MFMAs that consume them; rows
// past T or E are loaded from a valid row and zeroed when consumed. Splitting the experts
// over workgroups as well keeps each wave's share of the router weights to a few KB, so
// the read is spread over many CUs.
template <int NF>
__global__ __launch_bounds__(kWave) void k_router_part(const uint16_t* __restrict__ x,
                                                       const uint16_t* __restrict__ wr, int T,
                                                       int H, int E, float* __restrict__ partial,
                                                       int32_t* __restrict__ sync, int n_sync) {
  // a slice of the fused decode split is at most 2 pairs of steps
  constexpr int RB = router_rb<NF>() < 4 ? router_rb<NF>() : 4;
  const int lane = threadIdx.x;
  const int z = blockIdx.x, nsplit = gridDim.x;
  const int nsteps = H / 32;
  const int npairs = (nsteps + 1) / 2;
  const int s_begin = 2 * (int)((int64_t)npairs * z / nsplit);
  const int s_end = min(nsteps, 2 * (int)((int64_t)npairs * (z + 1) / nsplit));
  const int row = lane & 15;        // token (A) / expert (B) within the 16-tile
  const int kq = (lane >> 4) * 8;   // this lane's 8-element slice of the 32-step
  const bool tok_ok = row < T;
  const int e0 = (int)blockIdx.y * NF * 16;   // first expert of this workgroup's tiles
  const uint16_t* xr = x + (int64_t)(tok_ok ? row : 0) * H + kq;
  const uint16_t* wrow[NF];
  bool e_ok[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    e_ok[f] = e0 + f * 16 + row < E;
    wrow[f] = wr + (int64_t)(e_ok[f] ? e0 + f * 16 + row : 0) * H + kq;
  }
  f32x4 acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4 zero = {0, 0, 0, 0};
  for (int s0 = s_begin; s0 < s_end; s0 += RB) {
    u32x4 a[RB], bq[RB][NF];
    bool ok[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int s = s0 + r;
      ok[r] = s < s_end;
      const int ss = ok[r] ? s : s_begin;
      a[r] = *(const u32x4*)(xr + ss * 32);
#pragma unroll
      for (int f = 0; f < NF; ++f) bq[r][f] = *(const u32x4*)(wrow[f] + ss * 32);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      if (!ok[r]) continue;
      const bf16x8 av = __builtin_bit_cast(bf16x8, tok_ok ? a[r] : zero);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const bf16x8 bv = __builtin_bit_cast(bf16x8, e_ok[f] ? bq[r][f] : zero);
        acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[f], 0, 0, 0);
      }
    }
  }
  // the next kernel's synchronisation words start at zero
  if (z == 0 && blockIdx.y == 0)
    for (int i = lane; i < n_sync; i += kWave) sync[i] = 0;
  // lane holds D[token 4*(lane/16)+v][expert e0 + 16f + lane%16]
  float* dst = partial + (int64_t)z * T * E;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int e = e0 + f * 16 + row;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = 4 * (lane >> 4) + v;
      if (t < T && e < E) dst[(int64_t)t * E + e] = acc[f][v];
    }
  }
}

// Finish a split router for a small batch (T <= 16) in one workgroup: load every split's
// partial logits (all loads issued before any is used), sum them in increasing split order,
// add the bias, take top-k and softmax per token, and, with BUCKET, bucket-sort the pairs.
// partial: [ksplit][T][E]; ksplit * T * E <= kFinishCap.
constexpr int kFinishCap = 8192;
template <bool BUCKET>
__global__ __launch_bounds__(256) void k_router_finish(
    const float* __restrict__ partial, int ksplit, const float* __restrict__ bias, int T, int E,
    int k, int32_t* __restrict__ ids, float* __restrict__ w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm) {
  __shared__ float flat[kFinishCap];
  __shared__ float lg[kRouteTok][kMaxE];
  __shared__ int ids_l[kRouteTok * kMaxK];
  __shared__ TopkScratch tks[kRouteWaves];
  __shared__ int lid[BUCKET ? kRouteTok * kMaxK : 1];
  __shared__ int hist[BUCKET ? kMaxE : 1], run[BUCKET ? kMaxE : 1];
  __shared__ int wcnt[BUCKET ? kRouteWaves : 1][kMaxE];
  __shared__ int tmp[4];
  const int wave = threadIdx.x / kWave;
  const int te = T * E;
  const int n = ksplit * te;
  constexpr int kBatch = 8;
  for (int base = threadIdx.x; base < n; base += 256 * kBatch) {
    float v[kBatch];
#pragma unroll
    for (int r = 0; r < kBatch; ++r) v[r] = partial[min(base + r * 256, n - 1)];
#pragma unroll
    for (int r = 0; r < kBatch; ++r)
      if (base + r * 256 < n) flat[base + r * 256] = v[r];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < te; i += 256) {
    float v[kMaxSplit];
#pragma unroll
    for (int z = 0; z < kMaxSplit; ++z) v[z] = flat[min(z, ksplit - 1) * te + i];
    lg[i / E][i % E] = finish_logit(v, ksplit, bias != nullptr ? bias[i % E] : 0.f);
  }
  __syncthreads();
  for (int tt = wave; tt < T; tt += kRouteWaves)
    wave_topk_softmax(lg[tt], E, k, ids + (int64_t)tt * k, w + (int64_t)tt * k, tks[wave],
                      ids_l + tt * k);
  if constexpr (BUCKET) {
    __syncthreads();
    bucket_dev::bucket_one_block<256>(ids_l, T * k, E, counts, offsets, perm, inv_perm, lid,
                                      hist, run, wcnt, tmp);
  }
}

// Route and bucket a small batch (T <= 16, E <= 128) in one workgroup of 8 waves: every
// router load is in flight at once, then top-k and softmax per token, the counting sort of
// the pairs, and the list of active experts the expert FFN reads:
//   act[0] = number of non-empty buckets; for j < act[0], entry j at act[1 + 8j]:
//   {expert e, slot_map[e], offsets[e], offsets[e + 1], token of the expert's first four
//    pairs (-1 where it has fewer)}   (experts in increasing order).
// Without BUCKET only ids and w are written (the stand-alone router for small batches, so
// that it sums in exactly the same order as the fused layer does).
constexpr int kSmallWaves = 8;
template <int NF, bool BUCKET>
__global__ __launch_bounds__(kSmallWaves * kWave) void k_route_small(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int T, int H, int E, int k,
    const int32_t* __restrict__ slot_map, int32_t* __restrict__ ids, float* __restrict__ w,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv_perm, int32_t* __restrict__ act) {
  constexpr int NTH = kSmallWaves * kWave;
  __shared__ float red[4][kRouteTok][NF * 16];
  __shared__ int ids_l[kRouteTok * kMaxK];
  __shared__ int lid[kRouteTok * kMaxK];
  __shared__ int perm_l[kRouteTok * kMaxK];
  __shared__ TopkScratch tks[kSmallWaves];
  __shared__ int hist[kMaxE], run[kMaxE], wcnt[kSmallWaves][kMaxE], tmp[kSmallWaves];
  const int wave = threadIdx.x / kWave;
  const int tid = threadIdx.x;
  // per-expert values needed at the end, loaded together with the router operands
  const int ec = tid < E ? tid : 0;
  const float bv = bias != nullptr ? bias[ec] : 0.f;
  const int sv = BUCKET ? slot_map[ec] : 0;
  router_tile<NF, kSmallWaves, router_rb<NF>()>(x, wr, T, H, E, 0, 0, 1, red);
  if (bias != nullptr && tid < E)
    for (int tt = 0; tt < T; ++tt) red[0][tt][tid] += bv;
  __syncthreads();
  for (int tt = wave; tt < T; tt += kSmallWaves)
    wave_topk_softmax(&red[0][tt][0], E, k, ids + (int64_t)tt * k, w + (int64_t)tt * k,
                      tks[wave], ids_l + tt * k);
  if constexpr (!BUCKET) return;
  __syncthreads();
  bucket_dev::bucket_one_block<NTH>(ids_l, T * k, E, counts, offsets, perm, inv_perm, lid, hist,
                                    run, wcnt, tmp, perm_l);
  __syncthreads();
  // after the counting sort: hist[e] = count, run[e] = offsets[e] + count
  const bool ne = tid < E && hist[tid] > 0;
  int total;
  const int rank = bucket_dev::block_exclusive_scan<NTH>(ne ? 1 : 0, tmp, &total);
  if (ne) {
    int32_t* a = act + 1 + kActStride * rank;
    const int lo = run[tid] - hist[tid], hi = run[tid];
    a[0] = tid;
    a[1] = sv;
    a[2] = lo;
    a[3] = hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[4 + i] = lo + i < hi ? perm_l[lo + i] / k : -1;
  }
  if (tid == 0) act[0] = total;
}

}  // namespace

int route_ksplit(int T, int H) {
  if (T > kRouteTok) return 1;
  int ks = (H / 32) / 4;
  ks = min(ks, kMaxSplit);
  ks = min(ks, kFinishCap / (T * kMaxE));
  return max(ks, 1);
}

int route_fused_split(int H) { return min(kMaxRouteSplit, max(1, (H / 32) / 2)); }

bool route_fused_ok(int T, int H, int E) {
  // T * k <= kFuseMaxPairs follows from T <= kFuseMaxT and k <= kMaxK
  return T >= 1 && T <= kFuseMaxT && T * E <= kFuseMaxTE && H <= kRouteMaxH &&
         route_fused_split(H) >= 2;
}

hipError_t launch_router_partials(const uint16_t* x, const uint16_t* wr, int T, int H, int E,
                                  int ns, float* partial, hipStream_t stream, int32_t* sync,
                                  int n_sync) {
  if (T < 1 || T > kRouteTok || ns < 2 || ns > kMaxSplit) return hipErrorInvalidValue;
  const int ntiles = (E + 15) / 16;
  if (E < 1 || ntiles > 16) return hipErrorInvalidValue;
  // one 16-expert tile per workgroup: ns x ntiles single-wave workgroups
  hipLaunchKernelGGL(k_router_part<1>, dim3(ns, ntiles), dim3(kWave), 0, stream, x, wr, T, H, E,
                     partial, sync, sync != nullptr ? n_sync : 0);
  return hipGetLastError();
}

hipError_t launch_router_finish(const float* partial, int ns, const float* bias, int T, int E,
                                int k, int32_t* ids, float* w, int32_t* counts,
                                int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                                hipStream_t stream) {
  if (T < 1 || T > kRouteTok || ns * T * E > kFinishCap) return hipErrorInvalidValue;
  if (counts != nullptr)
    hipLaunchKernelGGL(k_router_finish<true>, dim3(1), dim3(256), 0, stream, partial, ns, bias,
                       T, E, k, ids, w, counts, offsets, perm, inv_perm);
  else
    hipLaunchKernelGGL(k_router_finish<false>, dim3(1), dim3(256), 0, stream, partial, ns, bias,
                       T, E, k, ids, w, nullptr, nullptr, nullptr, nullptr);
  return hipGetLastError();
}

bool route_bucket_fusable(int T, int E) { return T >= 1 && T <= kRouteTok; }

bool route_small_ok(int T, int E) { return T >= 1 && T <= kRouteTok && E <= 128; }

hipError_t launch_route_small(const uint16_t* x, const uint16_t* wr, const float* bias, int T,
                              int H, int E, int k, const int32_t* slot_map, int32_t* ids,
                              float* w, int32_t* counts, int32_t* offsets, int32_t* perm,
                              int32_t* inv_perm, int32_t* act, hipStream_t stream) {
  if (!route_small_ok(T, E)) return hipErrorInvalidValue;
  const bool bucket = counts != nullptr;
#define MOE_SMALL_CASE(N)                                                                       \
  case N:                                                                                      \
    if (bucket)                                                                                \
      hipLaunchKernelGGL((k_route_small<N, true>), dim3(1), dim3(kSmallWaves * kWave), 0,       \
                         stream, x, wr, bias, T, H, E, k, slot_map, ids, w, counts, offsets,    \
                         perm, inv_perm, act);                                                  \
    else                                                                                       \
      hipLaunchKernelGGL((k_route_small<N, false>), dim3(1), dim3(kSmallWaves * kWave), 0,      \
                         stream, x, wr, bias, T, H, E, k, slot_map, ids, w, counts, offsets,    \
                         perm, inv_perm, act);                                                  \
    break;
  switch ((E + 15) / 16) {
    MOE_SMALL_CASE(1) MOE_SMALL_CASE(2) MOE_SMALL_CASE(3) MOE_SMALL_CASE(4)
    MOE_SMALL_CASE(5) MOE_SMALL_CASE(6) MOE_SMALL_CASE(7) MOE_SMALL_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef MOE_SMALL_CASE
  return hipGetLastError();
}

hipError_t launch_route_impl(const uint16_t* x, const uint16_t* wr, const float* bias, int T,
                             int H, int E, int k, int32_t* ids, float* w, float* partial,
                             int32_t* counts, int32_t* offsets, int32_t* perm,
                             int32_t* inv_perm, bool bucket, hipStream_t stream) {
  const int ks = route_ksplit(T, H);
  dim3 grid((T + kRouteTok - 1) / kRouteTok, ks);
#define MOE_ROUTER_CASE(N)                                                                  \
  case N:                                                                                  \
    hipLaunchKernelGGL(k_router<N>, grid, dim3(256), 0, stream, x, wr, bias, T, H, E, k,   \
                       partial, ids, w);                                                   \
    break;
  switch ((E + 15) / 16) {
    MOE_ROUTER_CASE(1) MOE_ROUTER_CASE(2) MOE_ROUTER_CASE(3) MOE_ROUTER_CASE(4)
    MOE_ROUTER_CASE(5) MOE_ROUTER_CASE(6) MOE_ROUTER_CASE(7) MOE_ROUTER_CASE(8)
    MOE_ROUTER_CASE(9) MOE_ROUTER_CASE(10) MOE_ROUTER_CASE(11) MOE_ROUTER_CASE(12)
    MOE_ROUTER_CASE(13) MOE_ROUTER_CASE(14) MOE_ROUTER_CASE(15) MOE_ROUTER_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef MOE_ROUTER_CASE
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || ks == 1) return err;
  if (bucket)
    hipLaunchKernelGGL(k_router_finish<true>, dim3(1), dim3(256), 0, stream, partial, ks, bias,
                       T, E, k, ids, w, counts, offsets, perm, inv_perm);
  else
    hipLaunchKernelGGL(k_router_finish<false>, dim3(1), dim3(256), 0, stream, partial, ks, bias,
                       T, E, k, ids, w, nullptr, nullptr, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_route(const uint16_t* x, const uint16_t* wr, const float* bias, int T, int H,
                        int E, int k, int32_t* ids, float* w, float* partial,
                        hipStream_t stream) {
  if (route_fused_ok(T, H, E)) {   // same partials, same finishing order as the fused layer
    const int ns = route_fused_split(H);
    hipError_t e = launch_router_partials(x, wr, T, H, E, ns, partial, stream);
    if (e != hipSuccess) return e;
    return launch_router_finish(partial, ns, bias, T, E, k, ids, w, nullptr, nullptr, nullptr,
                                nullptr, stream);
  }
  if (route_small_ok(T, E))   // same kernel, same summation order as the fused layer
    return launch_route_small(x, wr, bias, T, H, E, k, nullptr, ids, w, nullptr, nullptr,
                              nullptr, nullptr, nullptr, stream);
  return launch_route_impl(x, wr, bias, T, H, E, k, ids, w, partial, nullptr, nullptr, nullptr,
                           nullptr, false, stream);
}

hipError_t launch_route_bucket_small(const uint16_t* x, const uint16_t* wr, const float* bias,
                                     int T, int H, int E, int k, float* partial, int32_t* ids,
                                     float* w, int32_t* counts, int32_t* offsets, int32_t* perm,
                                     int32_t* inv_perm, hipStream_t stream) {
  if (!route_bucket_fusable(T, E)) return hipErrorInvalidValue;
  if (route_ksplit(T, H) == 1) {   // nothing to finish: router, then the counting sort
    hipError_t e = launch_route(x, wr, bias, T, H, E, k, ids, w, partial, stream);
    if (e != hipSuccess) return e;
    return launch_bucket(ids, T * k, E, counts, offsets, perm, inv_perm, nullptr, stream);
  }
  return launch_route_impl(x, wr, bias, T, H, E, k, ids, w, partial, counts, offsets, perm,
                           inv_perm, true, stream);
}

}  // namespace moe
