// Expert FFN for many tokens (prefill): grouped GEMM on bf16 MFMA over the experts' blocks.
//
// Once tokens are grouped by expert (tinyserve README, "How it works" item 6) each expert's
// work is a dense contraction [n_e x K] x [K x N]; the llama.cpp discussion's follow-up
// ("Formal gate results") runs it as a grouped quantized matmul after the mapping rewrite.
// Here one launch covers every expert:
//   * the workgroup grid is sized for the worst case, sum_e ceil(n_e / BM) <= T*k/BM + E
//     row tiles, times the column tiles; each workgroup finds its (expert, row tile) from
//     the bucket offsets and exits if it has none, so the host never reads the counts;
//   * A rows are gathered through perm on load (gate/up: x[perm[pos] / k]; down: h[pos]),
//     staged in LDS one 128-wide K step at a time, and prefetched into registers one step
//     ahead;
//   * B comes straight from the tiled pool: a 64-lane 16-byte load is 16 weight rows x 4
//     MXFP4 blocks, exactly the operand shape of four v_mfma_f32_16x16x32_bf16 (the 32-wide
//     K of one MFMA is a fixed permutation of the step's 128 K indices, applied to A and B
//     alike); codes are widened to bf16 in registers with the block scale folded in, which is
//     exact for MXFP4. For Q8_0 each MFMA covers exactly one block, its int8 codes are exact
//     in bf16, and the block scale d multiplies the fp32 MFMA result before accumulation;
//   * gate and up tiles of the same columns live in the same wave, so SwiGLU is applied in
//     registers and h is written once, rounded to bf16; the down projection writes fp32 y.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kTThreads = 256;
constexpr int kBM = 128;          // pairs per tile
constexpr int kBK = 128;          // K per pipeline step
constexpr int kLdsStride = kBK * 2 + 16;   // bytes per A row in LDS (padded)

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ u32x2 ldg8(const void* p) { return *(const u32x2*)p; }

// Which (expert, first position) a row tile index maps to; returns false if none.
__device__ bool map_row_tile(const int32_t* __restrict__ offsets, int E, int mt, int* e_out,
                             int* m0_out, int* tmp4, int* sh) {
  const int e = threadIdx.x;
  int lo = 0, n = 0;
  if (e < E) {
    lo = offsets[e];
    n = offsets[e + 1] - lo;
  }
  const int nt = (n + kBM - 1) / kBM;
  // exclusive scan of nt over the workgroup
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int inc = nt;
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    int o = __shfl_up(inc, m, kWave);
    if (lane >= m) inc += o;
  }
  if (lane == kWave - 1) tmp4[wave] = inc;
  if (threadIdx.x == 0) sh[0] = -1;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += tmp4[w];
  const int cum = base + inc - nt;
  if (e < E && mt >= cum && mt < cum + nt) {
    sh[0] = e;
    sh[1] = lo + (mt - cum) * kBM;
  }
  __syncthreads();
  *e_out = sh[0];
  *m0_out = sh[1];
  return sh[0] >= 0;
}

template <int FMT>
struct BFrag;   // one n-fragment's share of a K step, per lane

template <>
struct BFrag<kMXFP4> {
  u32x4 q;        // 32 codes of one block of one row
  uint32_t s;     // its E8M0 scale
  bool ok;
};
template <>
struct BFrag<kQ8_0> {
  u32x2 q[4];     // 8 codes from each of the step's 4 blocks
  uint32_t s[4];  // fp16 scale bits of each block
  uint32_t okm;   // bit j: block j exists
};

// Load the lane's B share of step c for the row group rg (MXFP4: block 4c + lane/16 of row
// lane%16; Q8_0: codes 8*(lane/16).. of blocks 4c..4c+3 of row lane%16). Loads are issued
// unconditionally (from the matrix base when out of range) and masked when consumed, so
// none of them waits for another.
template <int FMT>
__device__ __forceinline__ void load_b(BFrag<FMT>& f, const uint8_t* q, const uint8_t* s,
                                       int rg, int nb, int c, bool row_ok) {
  const int lane = threadIdx.x & (kWave - 1);
  if constexpr (FMT == kMXFP4) {
    const int b = 4 * c + (lane >> 4);
    f.ok = row_ok && b < nb;
    const int64_t unit = f.ok ? ((int64_t)rg * nb + b) * 16 + (lane & 15) : 0;
    f.q = ldg16(q + unit * 16);
    f.s = s[unit];
  } else {
    f.okm = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = 4 * c + j;
      const bool ok = row_ok && b < nb;
      f.okm |= (uint32_t)ok << j;
      const int64_t unit = ok ? ((int64_t)rg * nb + b) * 16 + (lane & 15) : 0;
      f.q[j] = ldg8(q + unit * 32 + 8 * (lane >> 4));
      f.s[j] = *(const uint16_t*)(s + unit * 2);
    }
  }
}

template <int FMT, bool GATED>
__global__ __launch_bounds__(kTThreads) void k_ggemm(
    const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as, int64_t qslot,
    int64_t sslot, const uint8_t* __restrict__ bq, const uint8_t* __restrict__ bs,
    const int32_t* __restrict__ slot_map, int n_slots, int E,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm, int k,
    const uint16_t* __restrict__ src, int K, int N, int n_ntiles,
    uint16_t* __restrict__ h_out, float* __restrict__ y_out, uint32_t* __restrict__ err_flags) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[kBM * kLdsStride];
  __shared__ int tmp4[4];
  __shared__ int sh[2];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int wm = wave >> 1, wn = wave & 1;
  const int mt = blockIdx.x / n_ntiles;
  const int nt = blockIdx.x % n_ntiles;
  int e, m0;
  if (!map_row_tile(offsets, E, mt, &e, &m0, tmp4, sh)) return;
  const int mend = offsets[e + 1];
  const int slot = slot_map[e];
  // columns of this workgroup: GATED -> 64 gate + the same 64 up columns; else 128
  const int n0 = GATED ? nt * 64 : nt * 128;
  if (slot < 0 || slot >= n_slots) {
    const int ncols = GATED ? 64 : 128;
    for (int i = threadIdx.x; i < kBM * ncols; i += kTThreads) {
      const int pos = m0 + i / ncols, n = n0 + i % ncols;
      if (pos < mend && n < N) {
        if (GATED) h_out[(int64_t)pos * N + n] = 0;
        else y_out[(int64_t)pos * N + n] = 0.f;
      }
    }
    if (threadIdx.x == 0 && err_flags) atomicOr(err_flags, 1u);
    return;
  }
  const int nb = K / 32;
  const int nsteps = (K + kBK - 1) / kBK;

  // ---- A staging: thread handles 16-byte piece (tid % 16) of rows tid/16 + 16 j
  const int piece = threadIdx.x & 15;
  const int rbase = threadIdx.x >> 4;
  int64_t arow[8];
  int prow[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)   // all perm loads first (clamped to the tile's first row)
    prow[j] = GATED ? perm[min(m0 + rbase + 16 * j, mend - 1)] : 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int pos = m0 + rbase + 16 * j;
    if (pos < mend) arow[j] = GATED ? (int64_t)(prow[j] / k) * K : (int64_t)pos * K;
    else arow[j] = -1;
  }
  u32x4 areg[8];
  uint32_t aok = 0;   // bit j: areg[j] holds real data (else it is stored as zeros)
  auto load_a = [&](int c) {
    const int kk = c * kBK + piece * 8;
    aok = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool ok = arow[j] >= 0 && kk < K;
      aok |= (uint32_t)ok << j;
      areg[j] = ldg16(src + (ok ? arow[j] + kk : 0));
    }
  };

  // ---- B: 4 n-fragments per wave
  const uint8_t* q0 = aq + (int64_t)slot * qslot;
  const uint8_t* s0 = as + (int64_t)slot * sslot;
  const uint8_t* q1 = GATED ? bq + (int64_t)slot * qslot : q0;
  const uint8_t* s1 = GATED ? bs + (int64_t)slot * sslot : s0;
  int frg[4];
  bool fok[4];
  const uint8_t* fq[4];
  const uint8_t* fs[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    int col0;
    if (GATED) {
      col0 = n0 + 32 * wn + 16 * (f & 1);
      fq[f] = f < 2 ? q0 : q1;
      fs[f] = f < 2 ? s0 : s1;
    } else {
      col0 = n0 + 64 * wn + 16 * f;
      fq[f] = q0;
      fs[f] = s0;
    }
    frg[f] = col0 / 16;
    fok[f] = col0 < N;
  }
  BFrag<FMT> bcur[4], bnext[4];

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_a(0);
#pragma unroll
  for (int f = 0; f < 4; ++f) load_b<FMT>(bcur[f], fq[f], fs[f], frg[f], nb, 0, fok[f]);

  const int g = lane >> 4;
  const int mrow = lane & 15;
  for (int c = 0; c < nsteps; ++c) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *(u32x4*)(lds_a + (rbase + 16 * j) * kLdsStride + piece * 16) =
          ((aok >> j) & 1) ? areg[j] : u32x4{0, 0, 0, 0};
    __syncthreads();
    if (c + 1 < nsteps) {
      load_a(c + 1);
#pragma unroll
      for (int f = 0; f < 4; ++f) load_b<FMT>(bnext[f], fq[f], fs[f], frg[f], nb, c + 1, fok[f]);
    }
    if constexpr (FMT == kMXFP4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x8 bv[4];
#pragma unroll
        for (int f = 0; f < 4; ++f)
          bv[f] = fp4x8_to_bf16x8(bcur[f].q[i], bcur[f].ok ? e8m0_to_f32(bcur[f].s) : 0.f);
#pragma unroll
        for (int mf = 0; mf < 4; ++mf) {
          const int row = 64 * wm + 16 * mf + mrow;
          const bf16x8 av =
              __builtin_bit_cast(bf16x8, *(const u32x4*)(lds_a + row * kLdsStride + (32 * g + 8 * i) * 2));
#pragma unroll
          for (int f = 0; f < 4; ++f)
            acc[mf][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[f], acc[mf][f], 0, 0, 0);
        }
      }
    } else {
      // one MFMA per 32-wide block; lane supplies K = 32 j + 8 g .. + 7 of block j
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 bv[4];
        float ds[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          bv[f] = i8x8_to_bf16x8(bcur[f].q[j][0], bcur[f].q[j][1]);
          ds[f] = ((bcur[f].okm >> j) & 1) ? fp16_to_f32((uint16_t)bcur[f].s[j]) : 0.f;
        }
#pragma unroll
        for (int mf = 0; mf < 4; ++mf) {
          const int row = 64 * wm + 16 * mf + mrow;
          const bf16x8 av =
              __builtin_bit_cast(bf16x8, *(const u32x4*)(lds_a + row * kLdsStride + (32 * j + 8 * g) * 2));
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[f], f32x4{0.f, 0.f, 0.f, 0.f},
                                                              0, 0, 0);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[mf][f][v] = fmaf(ds[f], t[v], acc[mf][f][v]);
          }
        }
      }
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) bcur[f] = bnext[f];
  }

  // ---- epilogue: lane holds D[row 4*(lane/16) + v][col lane%16] of each 16x16 tile
#pragma unroll
  for (int mf = 0; mf < 4; ++mf) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int pos = m0 + 64 * wm + 16 * mf + 4 * g + v;
      if (pos >= mend) continue;
      if constexpr (GATED) {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int n = n0 + 32 * wn + 16 * f + mrow;
          if (n < N)
            h_out[(int64_t)pos * N + n] = f32_to_bf16_rne(silu_mul(acc[mf][f][v], acc[mf][f + 2][v]));
        }
      } else {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int n = n0 + 64 * wn + 16 * f + mrow;
          if (n < N) y_out[(int64_t)pos * N + n] = acc[mf][f][v];
        }
      }
    }
  }
}

template <int FMT, bool GATED>
hipError_t launch_ggemm_t(const PoolView& a, const PoolView& b, const int32_t* slot_map,
                          int n_slots, int E, const int32_t* offsets, const int32_t* perm,
                          int T, int k, const uint16_t* src, int K, int N, uint16_t* h,
                          float* y, uint32_t* err, hipStream_t stream) {
  const int pairs = T * k;
  const int max_mtiles = (pairs + kBM - 1) / kBM + min(E, pairs);
  const int n_ntiles = GATED ? (N + 63) / 64 : (N + 127) / 128;
  const int64_t grid = (int64_t)max_mtiles * n_ntiles;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_ggemm<FMT, GATED>), dim3((unsigned)grid), dim3(kTThreads), 0, stream,
                     a.q, a.s, a.q_slot, a.s_slot, b.q, b.s, slot_map, n_slots, E, offsets, perm,
                     k, src, K, N, n_ntiles, h, y, err);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_grouped(int fmt, const PoolView& gate, const PoolView& up,
                                  const int32_t* slot_map, int n_slots, int E, const uint16_t* x,
                                  int T, int k, int H, int I, const int32_t* offsets,
                                  const int32_t* perm, uint16_t* h, uint32_t* err,
                                  hipStream_t stream) {
  if (fmt == kMXFP4)
    return launch_ggemm_t<kMXFP4, true>(gate, up, slot_map, n_slots, E, offsets, perm, T, k, x,
                                        H, I, h, nullptr, err, stream);
  return launch_ggemm_t<kQ8_0, true>(gate, up, slot_map, n_slots, E, offsets, perm, T, k, x, H,
                                     I, h, nullptr, err, stream);
}

hipError_t launch_down_grouped(int fmt, const PoolView& down, const int32_t* slot_map,
                               int n_slots, int E, int T, int k, int H, int I,
                               const int32_t* offsets, const uint16_t* h, float* y,
                               uint32_t* err, hipStream_t stream) {
  if (fmt == kMXFP4)
    return launch_ggemm_t<kMXFP4, false>(down, down, slot_map, n_slots, E, offsets, nullptr, T,
                                         k, h, I, H, nullptr, y, err, stream);
  return launch_ggemm_t<kQ8_0, false>(down, down, slot_map, n_slots, E, offsets, nullptr, T, k,
                                      h, I, H, nullptr, y, err, stream);
}

}  // namespace moe
