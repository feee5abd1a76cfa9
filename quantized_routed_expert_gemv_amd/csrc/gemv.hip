// Expert FFN for few tokens (decode): dequant-fused split-K GEMV on the native blocks.
//
// Each selected expert's forward is a gate, an up and a down projection computed directly
// on the quantized bytes, with no bf16 copy of the weights (tinyserve README, "How it
// works" item 2, and "What we tried and ruled out": full dequantization at load). With
// few tokens per expert the work is a stream of the selected experts' bytes from HBM, so
// the kernel is built around that stream:
//   * one workgroup = one 16-row group of one active expert; its 4 waves split the
//     reduction dimension K;
//   * in the pool's tiled layout one 64-lane 16-byte load is one contiguous KiB holding
//     16 rows x 4 MXFP4 blocks (or 16 rows x 2 Q8_0 blocks): every HBM line is used once;
//   * codes are widened in registers (gfx950 v_cvt_scalef32_pk_bf16_fp4 for MXFP4, exact
//     int8 -> bf16 for Q8_0) and reduced with v_dot2_f32_bf16 into fp32;
//   * partial sums meet through xor-shuffles and a fixed-order LDS sum over the 4 waves,
//     so results do not depend on timing.
// Gate and up are read in the same pass and SwiGLU is applied before h is written
// (rounded once to bf16); the down projection writes fp32 y.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kGThreads = 256;
constexpr int kGWaves = kGThreads / kWave;
constexpr int kUnroll = 2;     // chunks in flight per wave per iteration

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }

// Find the j-th expert (in expert order) with a non-empty bucket; -1 if there are fewer.
// Every lane of the calling wave gets the result.
__device__ int find_active_expert(const int32_t* __restrict__ offsets, int E, int j) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int base = 0; base < E; base += kWave) {
    const int e = base + lane;
    const bool ne = e < E && offsets[e + 1] > offsets[e];
    const uint64_t bal = __ballot(ne);
    const int cnt = __popcll(bal);
    if (j < cnt) {
      const uint64_t below = lane ? (~0ull >> (kWave - lane)) : 0ull;
      const bool mine = ne && __popcll(bal & below) == j;
      const uint64_t hit = __ballot(mine);
      return base + __ffsll((unsigned long long)hit) - 1;
    }
    j -= cnt;
  }
  return -1;
}

// Per-lane share of one chunk for one matrix: the lane's row, the lane's block (MXFP4:
// 32 codes; Q8_0: 16 codes = half a block), converted once and dotted with each token.
template <int FMT>
struct Chunk {
  u32x4 q;
  uint32_t s;
};

template <int FMT>
__device__ __forceinline__ void load_chunk(Chunk<FMT>& c, const uint8_t* q, const uint8_t* s,
                                           bool ok) {
  if (ok) {
    c.q = ld16(q);
    if constexpr (FMT == kMXFP4) c.s = *s;
    else c.s = *(const uint16_t*)s;
  } else {
    c.q = u32x4{0, 0, 0, 0};
    c.s = 0;
  }
}

// Weights of the chunk as bf16 pairs (MXFP4: 16 pairs, scale folded in; Q8_0: 8 pairs,
// scale applied later to the fp32 partial).
template <int FMT>
__device__ __forceinline__ void widen(const Chunk<FMT>& c, bf16x2* w) {
  if constexpr (FMT == kMXFP4) {
    const float sc = e8m0_to_f32(c.s);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      w[4 * d + 0] = fp4x2_to_bf16x2<0>(c.q[d], sc);
      w[4 * d + 1] = fp4x2_to_bf16x2<1>(c.q[d], sc);
      w[4 * d + 2] = fp4x2_to_bf16x2<2>(c.q[d], sc);
      w[4 * d + 3] = fp4x2_to_bf16x2<3>(c.q[d], sc);
    }
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      float f[4];
      i8x4_to_f32(c.q[d], f);
      w[2 * d + 0] = __builtin_bit_cast(bf16x2, pack_bf16x2_exact(f[0], f[1]));
      w[2 * d + 1] = __builtin_bit_cast(bf16x2, pack_bf16x2_exact(f[2], f[3]));
    }
  }
}

template <int FMT>
__device__ __forceinline__ float dot_chunk(const bf16x2* w, const uint32_t* xv, uint32_t s,
                                           float acc) {
  if constexpr (FMT == kMXFP4) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc = dot2_bf16(w[i], xv[i], acc);
    return acc;
  } else {
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) part = dot2_bf16(w[i], xv[i], part);
    return fmaf(fp16_to_f32((uint16_t)s), part, acc);
  }
}

// Geometry of the lane within a 1 KiB chunk of the tiled layout.
template <int FMT>
struct LaneMap {
  // MXFP4: unit = 16 B = one block of one row; lane l -> row l%16, block 4c + l/16
  // Q8_0 : unit = 32 B = one block of one row; lane l -> row (l/2)%16, block 2c + l/32,
  //        half l%2 of the block
  static constexpr int kBlocksPerChunk = FMT == kMXFP4 ? 4 : 2;
  static constexpr int kXWords = FMT == kMXFP4 ? 16 : 8;     // u32 of x per lane per chunk
  __device__ static int row(int lane) { return FMT == kMXFP4 ? (lane & 15) : ((lane >> 1) & 15); }
  __device__ static int blk(int lane) { return FMT == kMXFP4 ? (lane >> 4) : (lane >> 5); }
  __device__ static int xoff(int lane) { return FMT == kMXFP4 ? 0 : (lane & 1) * 16; }
};

template <int FMT, bool GATED, int NT>
__global__ __launch_bounds__(kGThreads) void k_gemv(
    const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as, int64_t a_qslot,
    int64_t a_sslot, const uint8_t* __restrict__ bq, const uint8_t* __restrict__ bs,
    const int32_t* __restrict__ slot_map, int n_slots, int E,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm, int k,
    const uint16_t* __restrict__ src, int K, int rows, uint16_t* __restrict__ h_out,
    float* __restrict__ y_out, uint32_t* __restrict__ err_flags) {
  using LM = LaneMap<FMT>;
  constexpr int kM = GATED ? 2 : 1;
  __shared__ float red[kGWaves][NT][kM][16];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int rg = blockIdx.x;
  const int e = find_active_expert(offsets, E, blockIdx.y);
  if (e < 0) return;
  const int lo = offsets[e], hi = offsets[e + 1];
  const int slot = slot_map[e];
  const int r0 = rg * 16;
  if (slot < 0 || slot >= n_slots) {
    for (int i = threadIdx.x; i < (hi - lo) * 16; i += kGThreads) {
      const int pos = lo + i / 16, r = r0 + i % 16;
      if (GATED) h_out[(int64_t)pos * rows + r] = 0;
      else y_out[(int64_t)pos * rows + r] = 0.f;
    }
    if (threadIdx.x == 0 && err_flags) atomicOr(err_flags, 1u);
    return;
  }
  const int nb = K / 32;
  const int nc = (nb + LM::kBlocksPerChunk - 1) / LM::kBlocksPerChunk;
  const int64_t cb = code_bytes_per_block(FMT), sb = scale_bytes_per_block(FMT);
  // start of this row group in the code / scale planes, plus the lane's 16-byte slot
  const int64_t unit0 = (int64_t)rg * nb * 16;
  const uint8_t* qa = aq + slot * a_qslot + unit0 * cb + lane * 16;
  const uint8_t* qb = GATED ? bq + slot * a_qslot + unit0 * cb + lane * 16 : nullptr;
  const int lane_unit = FMT == kMXFP4 ? lane : (lane >> 1);
  const uint8_t* sa = as + slot * a_sslot + (unit0 + lane_unit) * sb;
  const uint8_t* sbp = GATED ? bs + slot * a_sslot + (unit0 + lane_unit) * sb : nullptr;
  const int lblk = LM::blk(lane);

  for (int c0 = lo; c0 < hi; c0 += NT) {
    const uint16_t* xr[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int pos = min(c0 + i, hi - 1);
      const int64_t row = GATED ? (int64_t)(perm[pos] / k) : (int64_t)pos;
      xr[i] = src + row * K + LM::xoff(lane);
    }
    float acc[kM][NT];
#pragma unroll
    for (int m = 0; m < kM; ++m)
#pragma unroll
      for (int i = 0; i < NT; ++i) acc[m][i] = 0.f;

    for (int c = wave; c < nc; c += kGWaves * kUnroll) {
      Chunk<FMT> ca[kUnroll], cbk[kUnroll];
      uint32_t xv[kUnroll][NT][LM::kXWords];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int cc = c + u * kGWaves;
        const int b = cc * LM::kBlocksPerChunk + lblk;
        const bool ok = cc < nc && b < nb;
        const int64_t qoff = (int64_t)cc * 1024;
        const int64_t soff = (int64_t)cc * (FMT == kMXFP4 ? 64 : 64);
        load_chunk<FMT>(ca[u], qa + qoff, sa + soff, ok);
        if constexpr (GATED) load_chunk<FMT>(cbk[u], qb + qoff, sbp + soff, ok);
#pragma unroll
        for (int i = 0; i < NT; ++i) {
#pragma unroll
          for (int w4 = 0; w4 < LM::kXWords / 4; ++w4) {
            u32x4 v = ok ? ld16(xr[i] + b * 32 + w4 * 8) : u32x4{0, 0, 0, 0};
            xv[u][i][4 * w4 + 0] = v[0];
            xv[u][i][4 * w4 + 1] = v[1];
            xv[u][i][4 * w4 + 2] = v[2];
            xv[u][i][4 * w4 + 3] = v[3];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        bf16x2 w[16];
        widen<FMT>(ca[u], w);
#pragma unroll
        for (int i = 0; i < NT; ++i) acc[0][i] = dot_chunk<FMT>(w, xv[u][i], ca[u].s, acc[0][i]);
        if constexpr (GATED) {
          widen<FMT>(cbk[u], w);
#pragma unroll
          for (int i = 0; i < NT; ++i)
            acc[kM - 1][i] = dot_chunk<FMT>(w, xv[u][i], cbk[u].s, acc[kM - 1][i]);
        }
      }
    }
    // lanes that share a row: MXFP4 {l, l^16, l^32, l^48}; Q8_0 {l, l^1, l^32, l^33}
#pragma unroll
    for (int m = 0; m < kM; ++m)
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        float v = acc[m][i];
        if constexpr (FMT == kMXFP4) {
          v += wave_xor(v, 16);
          v += wave_xor(v, 32);
        } else {
          v += wave_xor(v, 1);
          v += wave_xor(v, 32);
        }
        acc[m][i] = v;
      }
    const bool writer = FMT == kMXFP4 ? (lane < 16) : (lane < 32 && (lane & 1) == 0);
    if (writer) {
      const int r = LM::row(lane);
#pragma unroll
      for (int m = 0; m < kM; ++m)
#pragma unroll
        for (int i = 0; i < NT; ++i) red[wave][i][m][r] = acc[m][i];
    }
    __syncthreads();
    if (threadIdx.x < NT * 16) {
      const int i = threadIdx.x / 16, r = threadIdx.x % 16;
      const int pos = c0 + i;
      if (pos < hi) {
        float v[kM];
#pragma unroll
        for (int m = 0; m < kM; ++m) {
          float sum = red[0][i][m][r];
#pragma unroll
          for (int q = 1; q < kGWaves; ++q) sum += red[q][i][m][r];
          v[m] = sum;
        }
        if constexpr (GATED) h_out[(int64_t)pos * rows + r0 + r] = f32_to_bf16_rne(silu_mul(v[0], v[1]));
        else y_out[(int64_t)pos * rows + r0 + r] = v[0];
      }
    }
    __syncthreads();
  }
}

template <int FMT, bool GATED>
hipError_t launch_gemv_t(const PoolView& a, const PoolView& b, const int32_t* slot_map,
                         int n_slots, int E, const int32_t* offsets, const int32_t* perm,
                         int T, int k, const uint16_t* src, int K, int rows, uint16_t* h,
                         float* y, uint32_t* err, hipStream_t stream) {
  const int n_act = min(E, T * k);
  dim3 grid(rows / 16, n_act);
#define MOE_GEMV_CASE(N)                                                                     \
  hipLaunchKernelGGL((k_gemv<FMT, GATED, N>), grid, dim3(kGThreads), 0, stream, a.q, a.s,    \
                     a.q_slot, a.s_slot, b.q, b.s, slot_map, n_slots, E, offsets, perm, k,   \
                     src, K, rows, h, y, err)
  if (T <= 1) MOE_GEMV_CASE(1);
  else if (T <= 2) MOE_GEMV_CASE(2);
  else MOE_GEMV_CASE(4);
#undef MOE_GEMV_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_gemv(int fmt, const PoolView& gate, const PoolView& up,
                               const int32_t* slot_map, int n_slots, int E, const uint16_t* x,
                               int T, int k, int H, int I, const int32_t* offsets,
                               const int32_t* perm, uint16_t* h, uint32_t* err,
                               hipStream_t stream) {
  if (fmt == kMXFP4)
    return launch_gemv_t<kMXFP4, true>(gate, up, slot_map, n_slots, E, offsets, perm, T, k, x, H,
                                       I, h, nullptr, err, stream);
  return launch_gemv_t<kQ8_0, true>(gate, up, slot_map, n_slots, E, offsets, perm, T, k, x, H, I,
                                    h, nullptr, err, stream);
}

hipError_t launch_down_gemv(int fmt, const PoolView& down, const int32_t* slot_map, int n_slots,
                            int E, int T, int k, int H, int I, const int32_t* offsets,
                            const uint16_t* h, float* y, uint32_t* err, hipStream_t stream) {
  if (fmt == kMXFP4)
    return launch_gemv_t<kMXFP4, false>(down, down, slot_map, n_slots, E, offsets, nullptr, T, k,
                                        h, I, H, nullptr, y, err, stream);
  return launch_gemv_t<kQ8_0, false>(down, down, slot_map, n_slots, E, offsets, nullptr, T, k, h,
                                     I, H, nullptr, y, err, stream);
}

}  // namespace moe
