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
// workgroups (grid.y) and a second kernel sums the partials in a fixed order.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kRouteTok = 16;   // tokens per workgroup (one MFMA row tile)
constexpr int kRouteWaves = 4;

// Top-k of one token's E logits held in LDS, by one wave. Ties go to the lower index;
// NaN counts as -inf. Writes ids and softmax weights over the chosen k.
__device__ void wave_topk_softmax(const float* logit, int E, int k, int32_t* ids_out,
                                  float* w_out) {
  const int lane = threadIdx.x & (kWave - 1);
  float v[kMaxE / kWave];
#pragma unroll
  for (int i = 0; i < kMaxE / kWave; ++i) {
    int e = lane + i * kWave;
    float x = e < E ? logit[e] : -INFINITY;
    v[i] = (x != x) ? -INFINITY : x;
  }
  uint32_t taken = 0;   // bit i: v[i] already chosen
  float chosen_v[kMaxK];
  int chosen_e[kMaxK];
  for (int j = 0; j < k; ++j) {
    // best of this lane: largest value, lowest index among equals (indices grow with i)
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxE / kWave; ++i) {
      int e = lane + i * kWave;
      bool ok = e < E && !((taken >> i) & 1u);
      if (ok && (v[i] > bv || (v[i] == bv && e < be))) { bv = v[i]; be = e; }
    }
    // wave arg-max on the key (value desc, index asc)
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      float ov = __shfl_xor(bv, m, kWave);
      int oe = __shfl_xor(be, m, kWave);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
    chosen_v[j] = bv;
    chosen_e[j] = be;
    if ((be & (kWave - 1)) == lane) taken |= 1u << (be / kWave);
  }
  if (lane == 0) {
    float z[kMaxK];
    float sum = 0.f;
    for (int j = 0; j < k; ++j) { z[j] = expf(chosen_v[j] - chosen_v[0]); sum += z[j]; }
    for (int j = 0; j < k; ++j) { ids_out[j] = chosen_e[j]; w_out[j] = z[j] / sum; }
  }
}

template <int NF>   // NF = ceil(E / 16) expert tiles
__global__ __launch_bounds__(256) void k_router(const uint16_t* __restrict__ x,
                                                const uint16_t* __restrict__ wr,
                                                const float* __restrict__ bias, int T, int H,
                                                int E, int k, float* __restrict__ partial,
                                                int32_t* __restrict__ ids,
                                                float* __restrict__ w) {
  __shared__ float red[kRouteWaves][kRouteTok][NF * 16];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int t0 = blockIdx.x * kRouteTok;
  const int nsteps = H / 32;
  const int ksplit = gridDim.y;
  const int s_begin = (int)((int64_t)nsteps * blockIdx.y / ksplit);
  const int s_end = (int)((int64_t)nsteps * (blockIdx.y + 1) / ksplit);

  const int row = lane & 15;        // token (A) / expert (B) within the 16-tile
  const int kq = (lane >> 4) * 8;   // this lane's 8-element slice of the 32-step
  const int tok = t0 + row;
  const bool tok_ok = tok < T;
  const uint16_t* xr = x + (int64_t)(tok_ok ? tok : 0) * H + kq;

  f32x4 acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int s = s_begin + wave; s < s_end; s += kRouteWaves) {
    u32x4 a = tok_ok ? *(const u32x4*)(xr + s * 32) : u32x4{0, 0, 0, 0};
    bf16x8 av = __builtin_bit_cast(bf16x8, a);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      int e = f * 16 + row;
      u32x4 b = e < E ? *(const u32x4*)(wr + (int64_t)e * H + kq + s * 32) : u32x4{0, 0, 0, 0};
      acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, b),
                                                      acc[f], 0, 0, 0);
    }
  }
  // lane holds D[token 4*(lane/16)+v][expert 16f + lane%16]
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][4 * (lane >> 4) + v][f * 16 + row] = acc[f][v];
  __syncthreads();
  // fixed-order sum over waves
  for (int i = threadIdx.x; i < kRouteTok * NF * 16; i += blockDim.x) {
    int tt = i / (NF * 16), e = i % (NF * 16);
    float sum = red[0][tt][e];
#pragma unroll
    for (int q = 1; q < kRouteWaves; ++q) sum += red[q][tt][e];
    red[0][tt][e] = sum;
  }
  __syncthreads();
  if (ksplit > 1) {
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
                      w + (int64_t)(t0 + tt) * k);
  }
}

// Sum the split-K partial logits in a fixed order, add the bias, take top-k.
__global__ __launch_bounds__(256) void k_router_finish(const float* __restrict__ partial,
                                                       int ksplit, const float* __restrict__ bias,
                                                       int T, int E, int k,
                                                       int32_t* __restrict__ ids,
                                                       float* __restrict__ w) {
  __shared__ float lg[4][kMaxE];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  for (int e = lane; e < E; e += kWave) {
    float sum = partial[(int64_t)t * E + e];
    for (int z = 1; z < ksplit; ++z) sum += partial[((int64_t)z * T + t) * E + e];
    if (bias != nullptr) sum += bias[e];
    lg[wave][e] = sum;
  }
  // the wave's own LDS row: lanes of one wave are in lock-step on wave64 hardware, but
  // make the ordering explicit anyway
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  wave_topk_softmax(lg[wave], E, k, ids + (int64_t)t * k, w + (int64_t)t * k);
}

}  // namespace

int route_ksplit(int T, int H) {
  const int nsteps = H / 32;
  if (T > 64) return 1;
  int ks = nsteps / 4;
  if (ks < 1) ks = 1;
  if (ks > 32) ks = 32;
  return ks;
}

hipError_t launch_route(const uint16_t* x, const uint16_t* wr, const float* bias, int T, int H,
                        int E, int k, int32_t* ids, float* w, float* partial,
                        hipStream_t stream) {
  const int ks = route_ksplit(T, H);
  dim3 grid((T + kRouteTok - 1) / kRouteTok, ks);
  const int nf = (E + 15) / 16;
#define MOE_ROUTER_CASE(N)                                                                  \
  case N:                                                                                  \
    hipLaunchKernelGGL(k_router<N>, grid, dim3(256), 0, stream, x, wr, bias, T, H, E, k, \
                       partial, ids, w);                                                   \
    break;
  switch (nf) {
    MOE_ROUTER_CASE(1) MOE_ROUTER_CASE(2) MOE_ROUTER_CASE(3) MOE_ROUTER_CASE(4)
    MOE_ROUTER_CASE(5) MOE_ROUTER_CASE(6) MOE_ROUTER_CASE(7) MOE_ROUTER_CASE(8)
    MOE_ROUTER_CASE(9) MOE_ROUTER_CASE(10) MOE_ROUTER_CASE(11) MOE_ROUTER_CASE(12)
    MOE_ROUTER_CASE(13) MOE_ROUTER_CASE(14) MOE_ROUTER_CASE(15) MOE_ROUTER_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef MOE_ROUTER_CASE
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || ks == 1) return err;
  hipLaunchKernelGGL(k_router_finish, dim3((T + 3) / 4), dim3(256), 0, stream, partial, ks,
                     bias, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe
