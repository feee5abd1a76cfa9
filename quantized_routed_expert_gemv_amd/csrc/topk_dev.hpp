// Per-token top-k + softmax over the chosen k, by one wave; shared by the router kernels
// and by the decode gate/up kernel that finishes a split router itself.
#pragma once
#include "common.hpp"

namespace moe {

typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

// LDS scratch of one wave for wave_topk_softmax.
struct TopkScratch {
  __attribute__((aligned(16))) uint64_t keys[kMaxE];
  float zs[kMaxK];
};

// Unsigned key that orders like the float: NaN counts as -inf and -0 as +0.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (x != x) u = 0xff800000u;        // -inf
  if (u == 0x80000000u) u = 0u;       // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Softmax over the k chosen logits zs[0..k) (LDS, in rank order), by one wave:
// z_j = exp(L_j - L_0), sum = z_0 + z_1 + ... (increasing j), w_j = z_j / sum.
__device__ __forceinline__ void wave_softmax_chosen(const float* zs, int k, float* w_out) {
  const int lane = threadIdx.x & (kWave - 1);
  const float l0 = zs[0];
  const float z = lane < k ? expf(zs[lane < k ? lane : 0] - l0) : 0.f;
  float sum = 0.f;
  for (int j = 0; j < k; ++j) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), j));
  if (lane < k) w_out[lane] = z / sum;
}

// The key of expert e with logit x: order_key(x) above, then the lower index first.
__device__ __forceinline__ uint64_t topk_key(float x, int e) {
  return ((uint64_t)order_key(x) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
}

// Largest 32-bit value of the wave, in every lane: running maxima within each 16-lane row
// (row_shr 1, 2, 4, 8), then across rows (row_bcast 15 into rows 1 and 3, row_bcast 31 into
// rows 2 and 3), so that lane 63 holds the maximum, read back as a scalar.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// The float an order_key was made from (-0 comes back as +0, NaN as -inf: the values the key
// orders by).
__device__ __forceinline__ float key_value(uint32_t okey) {
  return __uint_as_float((okey & 0x80000000u) ? (okey & 0x7fffffffu) : ~okey);
}

template <int SLOTS>
__device__ void wave_topk_softmax_impl(const float* logit, int E, int k, int32_t* ids_out,
                                       float* w_out, TopkScratch& sc, int* ids_lds) {
  const int lane = threadIdx.x & (kWave - 1);
  const int E4 = (E + 3) & ~3;
  uint64_t key[SLOTS];
  float val[SLOTS];
  int rank[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int e = lane + i * kWave;
    float x = e < E ? logit[e] : -INFINITY;
    x = (x != x) ? -INFINITY : x;
    val[i] = x;
    key[i] = e < E ? topk_key(x, e) : 0ull;
    if (SLOTS == 1 || e < E4) sc.keys[e] = key[i];   // one slot: all 64 keys written
    rank[i] = 0;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  // every key against every key, as LDS broadcasts (padding keys are 0, below every real
  // key)
  if constexpr (SLOTS == 1) {
    // all 64 slots hold a key: read them in one batch, no loop-carried LDS latency
    u64x2 kv[kWave / 2];
#pragma unroll
    for (int q = 0; q < kWave / 2; ++q) kv[q] = *(const u64x2*)&sc.keys[2 * q];
#pragma unroll
    for (int q = 0; q < kWave / 2; ++q)
      rank[0] += (int)(kv[q][0] > key[0]) + (int)(kv[q][1] > key[0]);
  } else {
    for (int e2 = 0; e2 < E4; e2 += 4) {
      const u64x2 a = *(const u64x2*)&sc.keys[e2];
      const u64x2 b = *(const u64x2*)&sc.keys[e2 + 2];
#pragma unroll
      for (int i = 0; i < SLOTS; ++i)
        rank[i] += (int)(a[0] > key[i]) + (int)(a[1] > key[i]) + (int)(b[0] > key[i]) +
                   (int)(b[1] > key[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int e = lane + i * kWave;
    if (e < E && rank[i] < k) {
      ids_out[rank[i]] = e;
      sc.zs[rank[i]] = val[i];
      if (ids_lds) ids_lds[rank[i]] = e;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  wave_softmax_chosen(sc.zs, k, w_out);
}

// Top-k of one token's E logits (LDS), by one wave. Ties go to the lower index; NaN counts
// as -inf and -0 equals +0. Each logit gets the unique key (value order, then lower index
// first) and its rank
//   rank(e) = #{e' : L[e'] > L[e], or L[e'] == L[e] and e' < e}
// is the number of keys above its own; the experts of rank j < k are the choices, in
// order. The softmax over the chosen k is z_j = exp(L_j - L_0),
// sum = z_0 + z_1 + ... (increasing j), w_j = z_j / sum.
// sc: LDS scratch private to the wave. Writes ids and weights (and, if ids_lds is given, a
// copy of the ids).
__device__ inline void wave_topk_softmax(const float* logit, int E, int k, int32_t* ids_out,
                                         float* w_out, TopkScratch& sc,
                                         int* ids_lds = nullptr) {
  if (E <= kWave) wave_topk_softmax_impl<1>(logit, E, k, ids_out, w_out, sc, ids_lds);
  else if (E <= 2 * kWave) wave_topk_softmax_impl<2>(logit, E, k, ids_out, w_out, sc, ids_lds);
  else wave_topk_softmax_impl<kMaxE / kWave>(logit, E, k, ids_out, w_out, sc, ids_lds);
}

// Logit of one (token, expert) from a split router's partials: the splits are added in
// increasing split order, then the bias. Every kernel that finishes a split router uses
// this order, so they all agree bit for bit.
//   partial [ns][T*E] fp32, i = t*E + e.
//   v[z] = partial of split z (z < ns <= MAXS).
template <int MAXS>
__device__ __forceinline__ float finish_logit(const float (&v)[MAXS], int ns, float bias) {
  float sum = v[0];
#pragma unroll
  for (int z = 1; z < MAXS; ++z)
    if (z < ns) sum += v[z];
  return sum + bias;
}

}  // namespace moe
