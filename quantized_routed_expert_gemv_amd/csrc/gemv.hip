// Expert FFN for few tokens (decode): dequant-fused split-K GEMV on the native blocks.
//
// Each selected expert's forward is a gate, an up and a down projection computed directly
// on the quantized bytes, with no bf16 copy of the weights (tinyserve README, "How it
// works" item 2, and "What we tried and ruled out": full dequantization at load). With
// few tokens per expert the work is a stream of the selected experts' bytes from HBM, so
// the kernel is built around keeping that stream in flight:
//   * one workgroup = one 16-row group of one active expert; its 4 waves split K;
//   * in the pool's tiled layout one 64-lane 16-byte load is one contiguous KiB holding
//     16 rows x 4 MXFP4 blocks (or 16 rows x 2 Q8_0 blocks): every HBM line is used once;
//   * each wave issues the loads of up to 8 such chunks per matrix before it consumes any,
//     so at the workloads' sizes a workgroup has its whole share of the expert in flight
//     after one round trip; the activations for the same K range are staged in LDS once
//     per workgroup and read back as broadcasts;
//   * codes are widened in registers (gfx950 v_cvt_scalef32_pk_bf16_fp4 for MXFP4, exact
//     int8 -> bf16 for Q8_0) and reduced with v_dot2_f32_bf16 into fp32;
//   * partial sums meet through xor-shuffles and a fixed-order LDS sum over the 4 waves,
//     so results do not depend on timing.
// Gate and up are read in the same pass and SwiGLU is applied before h is written
// (rounded once to bf16); the down projection writes fp32 y.
#include <type_traits>

#include "common.hpp"
#include "bucket_dev.hpp"
#include "kernels.hpp"
#include "topk_dev.hpp"

namespace moe {

namespace {

constexpr int kGThreads = 256;
constexpr int kGWaves = kGThreads / kWave;
constexpr int kU = 8;          // chunks per wave per batch (all loads issued first)
constexpr int kRoutedMaxWG = 1024;   // workgroups of the routed gate/up kernel (4 per CU)

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }
// Expert weights are streamed once per call: nontemporal loads keep them from displacing
// the activations and small tables in the caches (and stream measurably faster).
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

// 16 bytes read device-coherently (two agent-scope 8-byte loads): data another workgroup
// of the same kernel stored with agent-scope stores, possibly on another XCD.
__device__ __forceinline__ u32x4 ld16_coherent(const void* p) {
  const uint64_t* q = (const uint64_t*)p;
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
}

// Find the j-th expert (in expert order) with a non-empty bucket; -1 if there are fewer.
// *n_active receives the number of non-empty buckets. Every lane of the wave gets both.
__device__ int find_active_expert(const int32_t* __restrict__ offsets, int E, int j,
                                  int* n_active) {
  const int lane = threadIdx.x & (kWave - 1);
  int found = -1, total = 0;
  for (int base = 0; base < E; base += kWave) {
    const int e = base + lane;
    const bool ne = e < E && offsets[e + 1] > offsets[e];
    const uint64_t bal = __ballot(ne);
    const int cnt = __popcll(bal);
    if (found < 0 && j >= total && j < total + cnt) {
      const uint64_t below = lane ? (~0ull >> (kWave - lane)) : 0ull;
      const bool mine = ne && __popcll(bal & below) == j - total;
      const uint64_t hit = __ballot(mine);
      found = base + __ffsll((unsigned long long)hit) - 1;
    }
    total += cnt;
  }
  *n_active = total;
  return found;
}

// One lane's share of one chunk of one matrix (16 bytes of codes and the block scale).
// Loads are issued unconditionally (from a valid address when the chunk lies past the end
// of the row) and masked when consumed: a guarded load would make the compiler wait for it
// before issuing the next one.
struct Chunk {
  u32x4 q;
  uint32_t s;    // the block's scale record
  uint32_t s2;   // k-quants: its super-block's d | dmin << 16
  u32x2 h;       // Q5_K: the block's high-bit dword; Q6_K: its two high-part dwords
  bool ok;
};

template <int FMT>
__device__ __forceinline__ void load_chunk(Chunk& c, const uint8_t* q, const uint8_t* s,
                                           const uint8_t* s2, const uint8_t* hq, bool ok) {
  c.q = ld16_stream(q);
  if constexpr (FMT == kMXFP4) c.s = __builtin_nontemporal_load(s);
  else c.s = __builtin_nontemporal_load((const uint16_t*)s);
  if constexpr (kquant(FMT)) c.s2 = __builtin_nontemporal_load((const uint32_t*)s2);
  else c.s2 = 0;
  if constexpr (FMT == kQ5_K) c.h = u32x2{__builtin_nontemporal_load((const uint32_t*)hq), 0u};
  else if constexpr (FMT == kQ6_K) c.h = __builtin_nontemporal_load((const u32x2*)hq);
  else c.h = u32x2{0u, 0u};
  c.ok = ok;
}

// Where a lane's high-bit dwords start (Q5_K, Q6_K; other formats: unused). plane: the
// matrix's code plane for the slot; unit: the lane's unit of chunk 0. Chunk c is
// 64 * hi_bytes_per_block further.
template <int FMT>
__device__ __forceinline__ const uint8_t* hi_base(const uint8_t* plane, int rows, int K,
                                                  int64_t unit) {
  if constexpr (hi_bytes_per_block(FMT) == 0) return plane;
  return plane + hi_region(rows, K) + unit * hi_bytes_per_block(FMT);
}

// Where a lane's super-block records start (Q4_K; other formats: unused). plane: the
// matrix's scale plane for the slot; rows x K: the matrix; rg: the row group. The record of
// chunk c (blocks 4c .. 4c+3, all in super-block c/2) is 64 bytes per super-block further.
template <int FMT>
__device__ __forceinline__ const uint8_t* super_base(const uint8_t* plane, int rows, int K,
                                                     int rg, int lane) {
  if constexpr (!kquant(FMT)) return plane;
  const int nsb = K / (32 * kSuperBlocks);
  return plane + super_region(rows, K) +
         ((int64_t)rg * nsb * kRowGroup + (lane & 15)) * kSuperBytes;
}

// Weights of the chunk as bf16 pairs (MXFP4: 16 pairs, scale folded in; Q8_0: 8 pairs,
// scale applied later to the fp32 partial; Q4_K: 16 pairs of the codes q, scale and min
// applied later; Q5_K: 16 pairs of the low nibbles, then 16 pairs of 16 x the high bits,
// pair i + 16 covering the same elements as pair i).
template <int FMT>
__device__ __forceinline__ void widen(const Chunk& c, bf16x2* w) {
  if constexpr (kquant(FMT)) {
#pragma unroll
    for (int d = 0; d < 4; ++d) u4x8_split_to_bf16(c.q[d], w + 4 * d);
    if constexpr (FMT == kQ5_K) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        // bytes 0/1 are the E4M3 codes of 0 and 2^-9; scale 2^13 gives 0 or 16, exactly
        const uint32_t lo = (c.h[0] >> (2 * d)) & 0x01010101u;
        const uint32_t hi = (c.h[0] >> (2 * d + 1)) & 0x01010101u;
        w[16 + 4 * d + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 8192.0f, false);
        w[16 + 4 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 8192.0f, true);
        w[16 + 4 * d + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 8192.0f, false);
        w[16 + 4 * d + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 8192.0f, true);
      }
    } else if constexpr (FMT == kQ6_K) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        // bytes 0..3 are the E4M3 codes of 0 .. 3 * 2^-9; scale 2^13 gives 16 x the high part
        const uint32_t g = c.h[d >> 1];
        const int sh = 4 * (d & 1);
        const uint32_t lo = (g >> sh) & 0x03030303u;
        const uint32_t hi = (g >> (sh + 2)) & 0x03030303u;
        w[16 + 4 * d + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 8192.0f, false);
        w[16 + 4 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 8192.0f, true);
        w[16 + 4 * d + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 8192.0f, false);
        w[16 + 4 * d + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 8192.0f, true);
      }
    }
  } else if constexpr (FMT == kMXFP4) {
    const float sc = c.ok ? e8m0_to_f32(c.s) : 0.f;
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

// A k-quant block. Q4_K / Q5_K: with P = sum x q and S = sum x over the block,
// sum x w = a P - c S where a = d sc and c = dmin m (both exact in fp32); P runs over the
// chunk's pairs (Q5_K: the low nibbles' pairs, then the high bits'). Q6_K: per 16-element
// half h, a_h (P_h - 32 S_h) with a_h = d sc_h (exact). sx: S (Q6_K: S_0, S_1).
template <int FMT>
__device__ __forceinline__ float kq_block(const bf16x2* w, const uint32_t* xv, uint32_t s,
                                          uint32_t s2, const float* sx, float acc) {
  if constexpr (FMT == kQ6_K) {
    const float d = fp16_to_f32((uint16_t)s2);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float p = 0.f;
#pragma unroll
      for (int i = 8 * h; i < 8 * h + 8; ++i) {
        p = dot2_bf16(w[i], xv[i], p);
        p = dot2_bf16(w[16 + i], xv[i], p);
      }
      const float a = d * (float)(int8_t)(s >> (8 * h));
      acc = fmaf(a, fmaf(-32.f, sx[h], p), acc);
    }
    return acc;
  } else {
    constexpr int kPairs = FMT == kQ5_K ? 32 : 16;
    float p = 0.f;
#pragma unroll
    for (int i = 0; i < kPairs; ++i) p = dot2_bf16(w[i], xv[i & 15], p);
    const float a = fp16_to_f32((uint16_t)s2) * (float)(s & 0xFFu);
    const float c = fp16_to_f32((uint16_t)(s2 >> 16)) * (float)((s >> 8) & 0xFFu);
    return fmaf(-c, sx[0], fmaf(a, p, acc));
  }
}

// s: the block's scale record (0 for a masked chunk: it then adds nothing); s2: a
// k-quant's super-block record.
template <int FMT>
__device__ __forceinline__ float dot_chunk(const bf16x2* w, const uint32_t* xv, uint32_t s,
                                           uint32_t s2, float acc) {
  if constexpr (kquant(FMT)) {
    // block sums (Q6_K: of each half), in the order block_sums() takes them
    float sx[2] = {0.f, 0.f};
    constexpr int kWordsPerSum = 16 / sums_per_block(FMT);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      sx[i / kWordsPerSum] = dot2_bf16(0x3F803F80u, xv[i], sx[i / kWordsPerSum]);   // (1, 1)
    return kq_block<FMT>(w, xv, s, s2, sx, acc);
  } else if constexpr (FMT == kMXFP4) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc = dot2_bf16(w[i], xv[i], acc);
    return acc;
  } else {
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) part = dot2_bf16(w[i], xv[i], part);
    return fmaf(fp16_to_f32((uint16_t)s), part, acc);   // s is 0 for masked chunks
  }
}

// dot_chunk with the block sums given (k-quants; other formats ignore them). Sums taken as
// block_sums() computes them give the same result as dot_chunk bit for bit.
template <int FMT>
__device__ __forceinline__ float dot_chunk_s(const bf16x2* w, const uint32_t* xv, uint32_t s,
                                             uint32_t s2, const float* sx, float acc) {
  if constexpr (kquant(FMT)) {
    return kq_block<FMT>(w, xv, s, s2, sx, acc);
  } else {
    return dot_chunk<FMT>(w, xv, s, s2, acc);
  }
}

// MXFP4 with 2 to 4 tokens: a chunk is 4 MFMAs (v_mfma_f32_16x16x32_bf16) instead of one
// dot2 pass per token, which leaves the kernel bound by HBM rather than by VALU issue. MFMA
// q takes from lane l (row l%16, block l/16 of the chunk) elements 8q .. 8q+7 of its block
// as B, and from the same lane the same K of token l%16 as A (zero past the tokens): the
// 32-wide K of MFMA q is a fixed choice of the chunk's 128, applied to both. The result,
// D[token][row], sits in lanes l < 16, tokens 0..3 of row l.
constexpr bool mma_path(int fmt, int nt) { return fmt == kMXFP4 && nt >= 2 && nt <= 4; }

// A fragments of a chunk: token row xr (LDS) at the lane's K offset, or zeros.
__device__ __forceinline__ void mma_a(const uint16_t* xr, bool live, bf16x8* av) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 v = *(const u32x4*)(xr + 8 * q);
    av[q] = __builtin_bit_cast(bf16x8, live ? v : u32x4{0u, 0u, 0u, 0u});
  }
}

// One widened MXFP4 chunk (w: 16 bf16 pairs in K order) into D.
__device__ __forceinline__ f32x4 mma_chunk(const bf16x2* w, const bf16x8* av, f32x4 acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bf16x8 b = {w[4 * q][0], w[4 * q][1], w[4 * q + 1][0], w[4 * q + 1][1],
                      w[4 * q + 2][0], w[4 * q + 2][1], w[4 * q + 3][0], w[4 * q + 3][1]};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[q], b, acc, 0, 0, 0);
  }
  return acc;
}

// Sums of the 32 bf16 values of a block at p (LDS) -- one sum, or one per 16-element half
// (Q6_K) -- into out, in the order dot_chunk takes them for the k-quants.
template <int FMT>
__device__ __forceinline__ void block_sums(const uint16_t* p, float* out) {
  constexpr int kWordsPerSum = 16 / sums_per_block(FMT);
  float sx[2] = {0.f, 0.f};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 v = *(const u32x4*)(p + q * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sx[(4 * q + i) / kWordsPerSum] = dot2_bf16(0x3F803F80u, v[i], sx[(4 * q + i) / kWordsPerSum]);
  }
#pragma unroll
  for (int h = 0; h < sums_per_block(FMT); ++h) out[h] = sx[h];
}

// Geometry of a lane within a 1 KiB chunk of the tiled layout.
//   MXFP4: unit = 16 B = one block of one row; lane l -> row l%16, block 4c + l/16
//   Q8_0 : unit = 32 B = one block of one row; lane l -> row (l/2)%16, block 2c + l/32,
//          half l%2 of the block
template <int FMT>
struct LaneMap {
  static constexpr bool k16 = unit16(FMT);
  static constexpr int kBlocksPerChunk = k16 ? 4 : 2;
  static constexpr int kKPerChunk = 32 * kBlocksPerChunk;     // K elements per chunk
  static constexpr int kXWords = k16 ? 16 : 8;                // u32 of x per lane per chunk
  static constexpr int kScaleChunk = 64 * (kquant(FMT) ? 2 : 1);   // scale bytes per chunk
  static constexpr int kWPairs = hi_bytes_per_block(FMT) ? 32 : 16;   // widened pairs per chunk
  static constexpr int kHiChunk = 64 * (int)hi_bytes_per_block(FMT);  // high-bit bytes per chunk
  __device__ static int row(int lane) { return k16 ? (lane & 15) : ((lane >> 1) & 15); }
  __device__ static int blk(int lane) { return k16 ? (lane >> 4) : (lane >> 5); }
  // K offset of the lane's codes inside its chunk
  __device__ static int koff(int lane) {
    return k16 ? (lane >> 4) * 32 : (lane >> 5) * 32 + (lane & 1) * 16;
  }
};

// Where a workgroup learns its expert, bucket range and tokens:
//   kSrcOffsets  bucket offsets (+ perm) from a previous stage
//   kSrcAct      the small-batch router's active-expert list
constexpr int kSrcOffsets = 0, kSrcAct = 1;

// RU: chunks per wave per batch (kU, or fewer where the row needs no more).
// TICKET (down projection from the active list, every expert's pairs within NT <= 4): the
// workgroups of a row group, one per active expert, finish with the combine of that row
// group (DownTail): wave 0 stores the unit's y rows device-coherently, waits for them and
// takes the row group's ticket; the last one to draw reads every pair's y row back and
// writes out[t] = sum_j w[t, j] y[inv_perm[t k + j]] in increasing j, as k_combine does.
template <int FMT, bool GATED, int SRC, int NT, int RU = kU, bool TICKET = false>
__global__ __launch_bounds__(kGThreads) void k_gemv(
    const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as, int64_t a_qslot,
    int64_t a_sslot, const uint8_t* __restrict__ bq, const uint8_t* __restrict__ bs,
    const int32_t* __restrict__ slot_map, int n_slots, int E,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm, int k,
    const uint16_t* __restrict__ src, int K, int rows, uint16_t* __restrict__ h_out,
    float* __restrict__ y_out, uint32_t* __restrict__ err_flags, const int32_t* __restrict__ act,
    DownTail tail) {
  static_assert(!TICKET || (!GATED && SRC == kSrcAct && NT <= 4), "ticket combine: down, <= 4 pairs");
  using LM = LaneMap<FMT>;
  constexpr int kM = GATED ? 2 : 1;
  constexpr int kSlice = kGWaves * RU * LM::kKPerChunk;   // K elements staged per batch
  constexpr int kSlicePieces = NT * (kSlice / 8);   // 16-byte pieces staged per batch
  __shared__ __attribute__((aligned(16))) uint16_t xs[NT][kSlice];
  __shared__ float red[kGWaves][NT][kM][16];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int rg = blockIdx.x;
  int e, lo, hi, slot;
  int atok[4] = {0, 0, 0, 0};
  int n_act = 0;
  if constexpr (SRC == kSrcAct) {
    // the small-batch router's active list: one round trip for expert, slot, range, tokens
    const int32_t* a = act + 1 + kActStride * blockIdx.y;
    n_act = act[0];
    e = a[0];
    slot = a[1];
    lo = a[2];
    hi = a[3];
#pragma unroll
    for (int i = 0; i < 4; ++i) atok[i] = a[4 + i];
    if ((int)blockIdx.y >= n_act) return;
  } else {
    int n_active;
    e = find_active_expert(offsets, E, blockIdx.y, &n_active);
    if (e < 0) return;
    lo = offsets[e];
    hi = offsets[e + 1];
    slot = slot_map[e];
  }
  const int r0 = rg * 16;
  if (slot < 0 || slot >= n_slots) {
    for (int i = threadIdx.x; i < (hi - lo) * 16; i += kGThreads) {
      const int pos = lo + i / 16, r = r0 + i % 16;
      if (GATED) h_out[(int64_t)pos * rows + r] = 0;
      else if (TICKET) __hip_atomic_store(&y_out[(int64_t)pos * rows + r], 0.f, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);   // wave 0 (<= 64 values)
      else y_out[(int64_t)pos * rows + r] = 0.f;
    }
    if (threadIdx.x == 0 && err_flags && slot != kSlotMiss) atomicOr(err_flags, 1u);
  } else {
    const int nb = K / 32;
    const int nc = (nb + LM::kBlocksPerChunk - 1) / LM::kBlocksPerChunk;
    constexpr int64_t cb = code_bytes_per_block(FMT), sb = scale_bytes_per_block(FMT);
    const int64_t unit0 = (int64_t)rg * nb * 16;
    const uint8_t* qa = aq + slot * a_qslot + unit0 * cb + lane * 16;
    const uint8_t* qb = GATED ? bq + slot * a_qslot + unit0 * cb + lane * 16 : nullptr;
    const int lane_unit = unit16(FMT) ? lane : (lane >> 1);
    const uint8_t* sa = as + slot * a_sslot + (unit0 + lane_unit) * sb;
    const uint8_t* sbp = GATED ? bs + slot * a_sslot + (unit0 + lane_unit) * sb : nullptr;
    const uint8_t* sa2 = super_base<FMT>(as + slot * a_sslot, rows, K, rg, lane);
    const uint8_t* sbp2 = GATED ? super_base<FMT>(bs + slot * a_sslot, rows, K, rg, lane) : nullptr;
    const uint8_t* ha = hi_base<FMT>(aq + slot * a_qslot, rows, K, unit0 + lane);
    const uint8_t* hb = GATED ? hi_base<FMT>(bq + slot * a_qslot, rows, K, unit0 + lane) : nullptr;
    const int lblk = LM::blk(lane);
    const int koff = LM::koff(lane);

    for (int c0 = lo; c0 < hi; c0 += NT) {
      // activation row of each token of this chunk (clamped to a valid row past the end)
      const uint16_t* xrow[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const int pos = min(c0 + i, hi - 1);
        int64_t row = pos;
        if constexpr (GATED) {
          // first chunk of the bucket: tokens come with the active list (past the bucket's
          // end, any valid row: those results are never stored)
          if (SRC != kSrcOffsets && i < 4 && c0 == lo) row = c0 + i < hi ? atok[i & 3] : atok[0];
          else row = perm[pos] / k;
        }
        xrow[i] = src + row * K;
      }
      constexpr bool kMma = mma_path(FMT, NT);
      float acc[kM][NT];
      f32x4 acc4[kM];
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        acc4[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NT; ++i) acc[m][i] = 0.f;
      }

      for (int cbase = 0; cbase < nc; cbase += kGWaves * RU) {
        // 1. the batch's K range of every token's activation row (L2-resident): loads first,
        //    LDS writes after the weight loads are issued
        // 16-byte pieces per thread (threads past the slice's pieces stage none)
        constexpr int kPieces = (kSlicePieces + kGThreads - 1) / kGThreads;
        const int k0 = cbase * LM::kKPerChunk;
        u32x4 xp[kPieces];
        bool xok[kPieces];
#pragma unroll
        for (int it = 0; it < kPieces; ++it) {
          const int idx0 = threadIdx.x + it * kGThreads;
          const int idx = idx0 < kSlicePieces ? idx0 : 0;
          const int i = idx / (kSlice / 8), q = idx % (kSlice / 8);
          const int kk = k0 + q * 8;
          xok[it] = idx0 < kSlicePieces && c0 + i < hi && kk < K;
          xp[it] = ld16(xrow[i] + (xok[it] ? kk : 0));
        }
        // 2. this wave's weight chunks of the batch, all in flight at once
        Chunk ca[RU], cbk[RU];
#pragma unroll
        for (int u = 0; u < RU; ++u) {
          const int c = cbase + wave + kGWaves * u;
          const int b = c * LM::kBlocksPerChunk + lblk;
          const bool ok = c < nc && b < nb;
          const int cs = ok ? c : 0;      // chunk 0 of the row group always exists
          load_chunk<FMT>(ca[u], qa + (int64_t)cs * 1024, sa + (int64_t)cs * LM::kScaleChunk,
                          sa2 + (int64_t)(cs >> 1) * 64, ha + (int64_t)cs * LM::kHiChunk, ok);
          if constexpr (GATED)
            load_chunk<FMT>(cbk[u], qb + (int64_t)cs * 1024, sbp + (int64_t)cs * LM::kScaleChunk,
                            sbp2 + (int64_t)(cs >> 1) * 64, hb + (int64_t)cs * LM::kHiChunk, ok);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the whole batch of loads ahead of its use
        __syncthreads();
#pragma unroll
        for (int it = 0; it < kPieces; ++it) {
          const int idx = threadIdx.x + it * kGThreads;
          const int i = idx / (kSlice / 8), q = idx % (kSlice / 8);
          if (idx < kSlicePieces) *(u32x4*)&xs[i][q * 8] = xok[it] ? xp[it] : u32x4{0, 0, 0, 0};
        }
        __syncthreads();
        // 3. consume (chunks past the end of the row carry a zero scale and add nothing)
        if constexpr (kMma) {
          const int tm = lane & 15;   // the lane's token row of A
#pragma unroll
          for (int u = 0; u < RU; ++u) {
            const int c = cbase + wave + kGWaves * u;
            const int xo = (c - cbase) * LM::kKPerChunk + koff;
            bf16x8 av[4];
            mma_a(&xs[tm < NT ? tm : 0][xo], tm < NT, av);
            bf16x2 w[LM::kWPairs];
            widen<FMT>(ca[u], w);
            acc4[0] = mma_chunk(w, av, acc4[0]);
            if constexpr (GATED) {
              widen<FMT>(cbk[u], w);
              acc4[kM - 1] = mma_chunk(w, av, acc4[kM - 1]);
            }
          }
          continue;
        }
#pragma unroll
        for (int u = 0; u < RU; ++u) {
          const int c = cbase + wave + kGWaves * u;
          const int xo = (c - cbase) * LM::kKPerChunk + koff;
          bf16x2 w[LM::kWPairs];
          uint32_t xv[LM::kXWords];
          widen<FMT>(ca[u], w);
#pragma unroll
          for (int i = 0; i < NT; ++i) {
#pragma unroll
            for (int q = 0; q < LM::kXWords / 4; ++q) {
              const u32x4 v = *(const u32x4*)&xs[i][xo + q * 8];
              xv[4 * q + 0] = v[0];
              xv[4 * q + 1] = v[1];
              xv[4 * q + 2] = v[2];
              xv[4 * q + 3] = v[3];
            }
            acc[0][i] = dot_chunk<FMT>(w, xv, ca[u].ok ? ca[u].s : 0u, ca[u].s2, acc[0][i]);
          }
          if constexpr (GATED) {
            widen<FMT>(cbk[u], w);
#pragma unroll
            for (int i = 0; i < NT; ++i) {
#pragma unroll
              for (int q = 0; q < LM::kXWords / 4; ++q) {
                const u32x4 v = *(const u32x4*)&xs[i][xo + q * 8];
                xv[4 * q + 0] = v[0];
                xv[4 * q + 1] = v[1];
                xv[4 * q + 2] = v[2];
                xv[4 * q + 3] = v[3];
              }
              acc[kM - 1][i] = dot_chunk<FMT>(w, xv, cbk[u].ok ? cbk[u].s : 0u, cbk[u].s2, acc[kM - 1][i]);
            }
          }
        }
      }
      if constexpr (kMma) {
        // D: lane l < 16 holds tokens 0..3 of row l
        if (lane < 16) {
#pragma unroll
          for (int m = 0; m < kM; ++m)
#pragma unroll
            for (int i = 0; i < NT; ++i) red[wave][i][m][lane] = acc4[m][i];
        }
      } else {
        // lanes that share a row: MXFP4 {l, l^16, l^32, l^48}; Q8_0 {l, l^1, l^32, l^33}
#pragma unroll
        for (int m = 0; m < kM; ++m)
#pragma unroll
          for (int i = 0; i < NT; ++i) {
            float v = acc[m][i];
            if constexpr (unit16(FMT)) {
              v += wave_xor(v, 16);
              v += wave_xor(v, 32);
            } else {
              v += wave_xor(v, 1);
              v += wave_xor(v, 32);
            }
            acc[m][i] = v;
          }
        const bool writer = unit16(FMT) ? (lane < 16) : (lane < 32 && (lane & 1) == 0);
        if (writer) {
          const int r = LM::row(lane);
#pragma unroll
          for (int m = 0; m < kM; ++m)
#pragma unroll
            for (int i = 0; i < NT; ++i) red[wave][i][m][r] = acc[m][i];
        }
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
          else if constexpr (TICKET)
            __hip_atomic_store(&y_out[(int64_t)pos * rows + r0 + r], v[0], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
          else y_out[(int64_t)pos * rows + r0 + r] = v[0];
        }
      }
      __syncthreads();
    }
  }
  if constexpr (TICKET) {
    // wave 0 holds every y store of this unit: once they have completed, the row group's
    // ticket; the workgroup that draws ticket n_act - 1 is the last of the group
    if (wave != 0) return;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    int ticket = 0;
    if (lane == 0)
      ticket = __hip_atomic_fetch_add(&tail.tickets[rg], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ticket = __builtin_amdgcn_readfirstlane(ticket);
    if (ticket != n_act - 1) return;
    if (lane < tail.T * 16) {
      const int t = lane >> 4, r = lane & 15;
      float yv[kMaxK], wv[kMaxK];
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {   // every load issued before the first use
        const int p = t * k + (j < k ? j : 0);
        const int pos = tail.inv_perm[p];
        wv[j] = tail.w[p];
        yv[j] = __hip_atomic_load(&y_out[(int64_t)pos * rows + r0 + r], __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
      }
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j)
        if (j < k) a = fmaf(wv[j], yv[j], a);
      tail.out[(int64_t)t * rows + r0 + r] = a;
    }
  }
}

// Down projection (and, with COMBINE, the combine) for a small batch (T*k <= 8 pairs) in
// one launch, with no atomics: a workgroup owns 16 output columns (one row group of the
// down matrices) for every active expert and every token. Its 8 waves split the (expert,
// chunk) work, each with all of its chunk loads in flight; the h rows of all pairs sit in
// LDS. Per pair and column the wave partials are summed in increasing wave order and
// written to y; COMBINE then merges them per token in increasing j exactly like the
// stand-alone combine kernel. The active experts come from the small-batch router's list
// (act) or, when act is NULL, from offsets and slot_map.
constexpr int kDCWaves = 8;
constexpr int kDCMaxPairs = 8;
constexpr int kDCMaxH = 57344 / 2;   // bf16 elements of h staged in LDS (pairs x I)
constexpr int kDCU = 12;             // chunks per wave per load batch

// NP: most pairs of one expert (every pair of an expert is a different token, so NP >= T
// suffices); the per-expert accumulators and the unrolled chunk loop are sized by it.
// DCU: chunks per wave per load batch (one token: as many as the wave's share needs, at
// most kDCU).
template <int FMT, bool COMBINE, int NP, int DCU = kDCU>
__global__ __launch_bounds__(kDCWaves * kWave) void k_down_small(
    const uint8_t* __restrict__ dq, const uint8_t* __restrict__ ds, int64_t qslot,
    int64_t sslot, int n_slots, int E, const int32_t* __restrict__ act,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ slot_map,
    const uint16_t* __restrict__ h, int T, int k, int H, int I, const int32_t* __restrict__ inv_perm,
    const float* __restrict__ topk_w, float* __restrict__ y, float* __restrict__ out,
    uint32_t* __restrict__ err_flags) {
  using LM = LaneMap<FMT>;
  constexpr int NTH = kDCWaves * kWave;
  __shared__ __attribute__((aligned(16))) uint16_t hs[kDCMaxH];
  __shared__ float red[kDCWaves][kDCMaxPairs][16];
  __shared__ float yl[kDCMaxPairs][16];
  __shared__ int actl[1 + kActStride * kDCMaxPairs];
  __shared__ float tw_l[kDCMaxPairs];
  __shared__ int ip_l[kDCMaxPairs];
  __shared__ int tmp[kDCWaves];
  // Q4_K: the block sums of the staged h rows
  __shared__ float hsum_l[kquant(FMT) ? kDCMaxH / 32 * sums_per_block(FMT) : 1];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int rg = blockIdx.x;
  const int r0 = rg * 16;
  const int np = T * k;
  const int nb = I / 32;
  const int nc = (nb + LM::kBlocksPerChunk - 1) / LM::kBlocksPerChunk;
  constexpr int64_t cb = code_bytes_per_block(FMT), sb = scale_bytes_per_block(FMT);
  const int64_t unit0 = (int64_t)rg * nb * 16;
  const int lane_unit = unit16(FMT) ? lane : (lane >> 1);
  const int lblk = LM::blk(lane);
  const int koff = LM::koff(lane);
  // 1. one round trip: the active list (or the offsets), every h row, the gate weights and
  //    the inverse permutation (independent loads, issued together)
  const int na_ints = 1 + kActStride * min(min(np, E), kDCMaxPairs);   // entries that exist
  int av = 0, olo = 0, ohi = 0, osl = 0;
  if (act != nullptr) {
    av = act[min(lane, na_ints - 1)];   // every wave reads the list's first 64 ints itself
  } else {
    const int ec = threadIdx.x < E ? threadIdx.x : 0;
    olo = offsets[ec];
    ohi = offsets[ec + 1];
    osl = slot_map[ec];
  }
  constexpr int kHPieces = kDCMaxH / 8 / NTH;    // 16-byte pieces per thread (upper bound)
  const int hp = np * I / 8;                     // pieces actually present
  u32x4 hv[kHPieces];
#pragma unroll
  for (int r = 0; r < kHPieces; ++r)
    hv[r] = *(const u32x4*)(h + (int64_t)min((int)threadIdx.x + r * NTH, hp - 1) * 8);
  float twv = 0.f;
  int ipv = 0;
  if constexpr (COMBINE) {
    const int pc = min((int)threadIdx.x, np - 1);
    twv = topk_w[pc];
    ipv = inv_perm[pc];
  }
  // 2. with the list in registers each wave knows its (expert j, share q) and issues its
  //    first batch of weight loads before the h rows reach LDS
  int n_act = 0, per = 1, j = 0, q = 0, slot = 0, lo = 0, hi = 0;
  if (act != nullptr) {
    n_act = __builtin_amdgcn_readlane(av, 0);   // lane 0 holds act[0]
    n_act = min(max(n_act, 1), kDCWaves);
    per = kDCWaves / n_act;
    j = wave % n_act;
    q = wave / n_act;
    slot = __builtin_amdgcn_readlane(av, 1 + kActStride * j + 1);
    lo = min(max(__builtin_amdgcn_readlane(av, 1 + kActStride * j + 2), 0), np);
    hi = min(max(__builtin_amdgcn_readlane(av, 1 + kActStride * j + 3), lo), np);
  }
  bool busy = q < per;
  bool valid = slot >= 0 && slot < n_slots;
  const uint8_t* qa = dq + (valid ? slot : 0) * qslot + unit0 * cb + lane * 16;
  const uint8_t* sa = ds + (valid ? slot : 0) * sslot + (unit0 + lane_unit) * sb;
  const uint8_t* sa2 = super_base<FMT>(ds + (valid ? slot : 0) * sslot, H, I, rg, lane);
  const uint8_t* ha = hi_base<FMT>(dq + (valid ? slot : 0) * qslot, H, I, unit0 + lane);
  Chunk ch[DCU];
  auto load_batch = [&](int cbase) {
#pragma unroll
    for (int u = 0; u < DCU; ++u) {
      const int c = cbase + u * per;
      const int b = c * LM::kBlocksPerChunk + lblk;
      const bool ok = c < nc && b < nb;
      const int cs = ok ? c : 0;
      load_chunk<FMT>(ch[u], qa + (int64_t)cs * 1024, sa + (int64_t)cs * LM::kScaleChunk,
                      sa2 + (int64_t)(cs >> 1) * 64, ha + (int64_t)cs * LM::kHiChunk, ok);
    }
  };
  if (act != nullptr && busy && valid) load_batch(q);
  __builtin_amdgcn_sched_barrier(0);
  // 3. h rows, list and combine inputs into LDS
  if (act != nullptr) {
    if (wave == 0 && lane < na_ints) actl[lane] = av;
  } else {
    const bool ne = (int)threadIdx.x < E && ohi > olo;
    int total;
    const int rank = bucket_dev::block_exclusive_scan<kDCWaves * kWave>(ne ? 1 : 0, tmp, &total);
    if (ne && rank < kDCMaxPairs) {
      int* a = &actl[1 + kActStride * rank];
      a[0] = threadIdx.x;
      a[1] = osl;
      a[2] = olo;
      a[3] = ohi;
    }
    if (threadIdx.x == 0) actl[0] = total;
  }
  if constexpr (COMBINE) {
    if ((int)threadIdx.x < np) {
      tw_l[threadIdx.x] = twv;
      ip_l[threadIdx.x] = ipv;
    }
  }
#pragma unroll
  for (int r = 0; r < kHPieces; ++r) {
    const int i = threadIdx.x + r * NTH;
    if (i < hp) *(u32x4*)&hs[i * 8] = hv[r];
  }
  __syncthreads();
  if constexpr (kquant(FMT)) {
    for (int i = threadIdx.x; i < np * I / 32; i += NTH)
      block_sums<FMT>(&hs[i * 32], &hsum_l[i * sums_per_block(FMT)]);
    __syncthreads();
  }
  if (act == nullptr) {
    n_act = actl[0];
    per = kDCWaves / n_act;
    j = wave % n_act;
    q = wave / n_act;
    const int* ent = &actl[1 + kActStride * j];
    slot = ent[1];
    lo = ent[2];
    hi = ent[3];
    busy = q < per;
    valid = slot >= 0 && slot < n_slots;
    qa = dq + (valid ? slot : 0) * qslot + unit0 * cb + lane * 16;
    sa = ds + (valid ? slot : 0) * sslot + (unit0 + lane_unit) * sb;
    sa2 = super_base<FMT>(ds + (valid ? slot : 0) * sslot, H, I, rg, lane);
    ha = hi_base<FMT>(dq + (valid ? slot : 0) * qslot, H, I, unit0 + lane);
    if (busy && valid) load_batch(q);
  }
  // 4. consume each batch as it arrives, then load the next
  static_assert(NP >= 1 && NP <= kDCMaxPairs, "pairs per expert");
  float acc[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) acc[p] = 0.f;
  if (busy && valid) {
    for (int cbase = q;;) {
#pragma unroll
      for (int u = 0; u < DCU; ++u) {
        const int c = cbase + u * per;
        const int kx = ch[u].ok ? c * LM::kKPerChunk + koff : 0;   // masked lanes: any valid row part
        bf16x2 w[LM::kWPairs];
        uint32_t xv[LM::kXWords];
        widen<FMT>(ch[u], w);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          if (lo + p < hi) {
            const uint16_t* hrow = &hs[(lo + p) * I + kx];
#pragma unroll
            for (int qq = 0; qq < LM::kXWords / 4; ++qq) {
              const u32x4 v = *(const u32x4*)(hrow + qq * 8);
              xv[4 * qq + 0] = v[0];
              xv[4 * qq + 1] = v[1];
              xv[4 * qq + 2] = v[2];
              xv[4 * qq + 3] = v[3];
            }
            const float* sx = &hsum_l[kquant(FMT) ? ((lo + p) * (I / 32) + kx / 32) * sums_per_block(FMT) : 0];
            acc[p] = dot_chunk_s<FMT>(w, xv, ch[u].ok ? ch[u].s : 0u, ch[u].s2, sx, acc[p]);
          }
        }
      }
      cbase += per * DCU;
      if (cbase >= nc) break;
      load_batch(cbase);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // 5. rows of the wave's partials, then fixed-order sums over the waves of each expert
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    float v = acc[p];
    if constexpr (unit16(FMT)) {
      v += wave_xor(v, 16);
      v += wave_xor(v, 32);
    } else {
      v += wave_xor(v, 1);
      v += wave_xor(v, 32);
    }
    acc[p] = v;
  }
  const bool writer = unit16(FMT) ? (lane < 16) : (lane < 32 && (lane & 1) == 0);
  if (writer) {
    const int r = LM::row(lane);
#pragma unroll
    for (int p = 0; p < NP; ++p) red[wave][p][r] = acc[p];
  }
  __syncthreads();
  if (threadIdx.x < np * 16) {
    const int pos = threadIdx.x / 16, r = threadIdx.x % 16;
    // the expert owning this bucket position, and its waves j, j + n_act, ...
    int jj = 0;
    for (int t = 0; t < n_act; ++t)
      if (pos >= actl[1 + kActStride * t + 2] && pos < actl[1 + kActStride * t + 3]) jj = t;
    const int plo = actl[1 + kActStride * jj + 2];
    const int ps = actl[1 + kActStride * jj + 1];
    float sum = 0.f;
    if (ps >= 0 && ps < n_slots) {
      sum = red[jj][pos - plo][r];
      for (int ww = jj + n_act; ww < per * n_act; ww += n_act) sum += red[ww][pos - plo][r];
    }
    yl[pos][r] = sum;
    y[(int64_t)pos * H + r0 + r] = sum;
  }
  if (!valid && busy && q == 0 && lane == 0 && err_flags && slot != kSlotMiss)
    atomicOr(err_flags, 1u);
  if constexpr (!COMBINE) return;
  __syncthreads();
  // 6. combine, in increasing j, as k_combine does
  if (threadIdx.x < T * 16) {
    const int t = threadIdx.x / 16, r = threadIdx.x % 16;
    float a = 0.f;
    for (int jj = 0; jj < k; ++jj) {
      const int p = t * k + jj;
      a = fmaf(tw_l[p], yl[ip_l[p]][r], a);
    }
    out[(int64_t)t * H + r0 + r] = a;
  }
}

// Decode gate/up that first finishes a split router (1 <= T <= 4 tokens, H <= kRouteMaxH).
//
// The router's partial logits (one set per slice of H) come from the previous kernel.
// Every workgroup finishes the routing itself from them -- sum in split order, top-k per
// token, counting sort of the T*k pairs, list of active experts -- so no workgroup waits
// for another; workgroup 0 also stores the routing for the stages after this kernel. Each
// workgroup then serves units (row group, active expert) blockIdx.x, + gridDim.x, ...
// Everything that does not depend on the routing (the partials, the slot map, the bias and
// the tokens' activation rows) is loaded in one round trip at the start; then the expert's
// gate and up rows of this row group are streamed and each chunk is consumed as it
// arrives. Chunk order, per-lane accumulation and the reduction are those of k_gemv, so
// the two give bit-identical h.
// RU: chunks per wave per load batch (0: by format and token count). At one token the
// launch picks, for every format, whichever of 4, 6 and the format's default leaves the
// fewest masked slots in the row's batches (the larger on a tie); some masked slots may
// remain (gpt-oss MXFP4: 23 chunks in 24 slots).
//
// RUD > 0: the fused decode layer. The workgroups stay for the down projection and the
// combine: each gate/up unit stores its h rows device-coherently and then counts itself
// done for its expert (FusedDown); after its gate/up units a workgroup serves down units
// (16-row group of out, active expert) v = blockIdx.x, + gridDim.x, ...: it issues the
// unit's first batch of down weights (RUD chunks per wave), waits until every gate/up unit
// of the expert is done, reads the expert's h rows device-coherently and finishes as the
// ticket-combining down kernel does (k_gemv with TICKET). The grid must fit on the device
// at once (the launcher caps it at the co-resident workgroup count), since a down unit
// waits on gate/up units of other workgroups; the waits are bounded (FusedDown).
template <int FMT, int NT, int RU = 0, int RUD = 0>
__global__ __launch_bounds__(kGThreads, 3) void k_gate_up_routed(
    const uint8_t* __restrict__ gq, const uint8_t* __restrict__ gsc,
    const uint8_t* __restrict__ uq, const uint8_t* __restrict__ usc, int64_t qslot,
    int64_t sslot, const int32_t* __restrict__ slot_map, int n_slots, int E, int k,
    const uint16_t* __restrict__ x, int H, int I, uint16_t* __restrict__ h_out,
    uint32_t* __restrict__ err_flags, RouteIn rin, FusedDown fd) {
  constexpr bool kFused = RUD > 0;
  using LM = LaneMap<FMT>;
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) uint16_t xs[NT * kRouteMaxH];
  __shared__ float lg_l[kFuseMaxTE];
  __shared__ int slot_l[kMaxE];
  __shared__ TopkScratch tk_l[NT];
  __shared__ int ids_l[kFuseMaxPairs];
  __shared__ float w_l[kFuseMaxPairs];
  __shared__ __attribute__((aligned(16))) int key_l[kFuseMaxPairs];
  __shared__ int perm_l[kFuseMaxPairs], inv_l[kFuseMaxPairs], tokp_l[kFuseMaxPairs];
  __shared__ unsigned long long hit_l[kMaxE / 64];
  __shared__ int act_l[kFuseMaxPairs][kActStride];
  __shared__ int nact_l;
  __shared__ float red[kGWaves][NT][2][16];
  // Q4_K: the block sums of the tokens' activation rows, shared by every row of every unit
  __shared__ float xsum_l[kquant(FMT) ? NT * kRouteMaxH / 32 * sums_per_block(FMT) : 1];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int T = rin.T, TE = T * E, ns = rin.ns, n = T * k;

  // 1. one round trip: partials of logit tid, slot and bias of expert tid, activation rows
  const int ic = tid < TE ? tid : 0;
  float v[kMaxRouteSplit];
#pragma unroll
  for (int z = 0; z < kMaxRouteSplit; ++z) v[z] = rin.partial[(int64_t)min(z, ns - 1) * TE + ic];
  const int ec = tid < E ? tid : 0;
  const int sm = slot_map[ec];
  const float bz = rin.bias != nullptr ? rin.bias[ic % E] : 0.f;
  constexpr int kXP = NT * kRouteMaxH / 8 / kGThreads;   // 16-byte pieces per thread
  const int xp_n = T * H / 8;
  u32x4 xv[kXP];
#pragma unroll
  for (int r = 0; r < kXP; ++r)
    xv[r] = *(const u32x4*)(x + (int64_t)min(tid + r * kGThreads, xp_n - 1) * 8);
  if (tid < kMaxE / 64) hit_l[tid] = 0ull;
  if (tid < E) slot_l[tid] = sm;
  if (tid < TE) lg_l[tid] = finish_logit(v, ns, bz);
#pragma unroll
  for (int r = 0; r < kXP; ++r) {
    const int i = tid + r * kGThreads;
    if (i < xp_n) *(u32x4*)&xs[i * 8] = xv[r];
  }
  __syncthreads();
  if constexpr (kquant(FMT)) {   // read after the routing's barriers
    const int nbx = H / 32;
    for (int i = tid; i < T * nbx; i += kGThreads)
      block_sums<FMT>(&xs[i * 32], &xsum_l[i * sums_per_block(FMT)]);
  }

  // steps 2 and 3 for any T (used unless the one-token path below applies)
  auto route_general = [&]() {
    // 2. top-k + softmax, wave t for token t
    if (wave < T) wave_topk_softmax(&lg_l[wave * E], E, k, ids_l + wave * k, w_l + wave * k, tk_l[wave]);
    __syncthreads();

    // 3. counting sort of the n = T*k pairs by wave 0. Pair p (expert e_p) has the unique key
    //    32*e_p + p; its bucket position is the number of smaller keys, its expert's range
    //    [lo, hi) the numbers of keys below 32*e_p and below 32*(e_p + 1), and its expert's
    //    index among the active ones the number of hit experts below e_p.
    if (wave == 0) {
      const bool has = lane < n;
      const int ep = has ? ids_l[lane] : 0;
      const int key = has ? ep * kFuseMaxPairs + lane : 0x7fffffff;
      if (lane < kFuseMaxPairs) key_l[lane] = key;
      if (has) atomicOr(&hit_l[ep >> 6], 1ull << (ep & 63));
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      const int klo = ep * kFuseMaxPairs, khi = klo + kFuseMaxPairs;
      int pos = 0, lo = 0, hi = 0;
      for (int q = 0; q < n; q += 4) {
        const i32x4 kq = *(const i32x4*)&key_l[q];
  #pragma unroll
        for (int c = 0; c < 4; ++c) {
          pos += kq[c] < key ? 1 : 0;
          lo += kq[c] < klo ? 1 : 0;
          hi += kq[c] < khi ? 1 : 0;
        }
      }
      const int hw = ep >> 6;
      int aidx = __popcll(hit_l[hw] & ((1ull << (ep & 63)) - 1ull));
      int nact = 0;
  #pragma unroll
      for (int w = 0; w < kMaxE / 64; ++w) {
        const int c = __popcll(hit_l[w]);
        nact += c;
        aidx += w < hw ? c : 0;
      }
      if (has) {
        perm_l[pos] = lane;
        inv_l[lane] = pos;
        tokp_l[pos] = (lane >= k ? 1 : 0) + (lane >= 2 * k ? 1 : 0) + (lane >= 3 * k ? 1 : 0);  // lane / k, T <= 4
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      if (has && pos == lo) {   // the first pair of its expert writes the expert's entry
        int* a = act_l[aidx];
        a[0] = ep;
        a[1] = slot_l[ep];
        a[2] = lo;
        a[3] = hi;
  #pragma unroll
        for (int i = 0; i < 4; ++i) a[4 + i] = lo + i < hi ? tokp_l[lo + i] : -1;
      }
      if (lane == 0) nact_l = nact;
    }
  };
  // 2'. one token, by wave 0 alone in registers: k rounds, each taking the largest
  //     remaining logit (its order_key, a 32-bit wave maximum) and, among equal ones, the
  //     lowest expert index (ballots of the slots in expert order, the first set lane): the
  //     largest remaining key of wave_topk_softmax, i.e. the key of rank r, so the same
  //     choices in the same order; then the softmax of the chosen logits exactly as
  //     wave_softmax_chosen computes it.
  // 3'. the k pairs of the one token (distinct experts): pair j goes to position
  //     #{j' : e_j' < e_j}, and is its expert's only pair.
  auto route_one_token = [&](auto slots) {
    constexpr int SLOTS = decltype(slots)::value;
    if (wave != 0) return;
    // order_key of expert s * 64 + lane's logit (every real key is at least order_key(-inf),
    // which is not 0); 0 for experts past E and for experts already taken
    uint32_t key[SLOTS];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int e = s * kWave + lane;
      float x = e < E ? lg_l[e] : -INFINITY;
      x = (x != x) ? -INFINITY : x;
      key[s] = e < E ? order_key(x) : 0u;
    }
    uint32_t mkey = 0u;   // lane r < k: the order_key and expert chosen in round r
    int ej = 0x7fffffff;
    for (int r = 0; r < k; ++r) {
      uint32_t m = key[0];
#pragma unroll
      for (int s = 1; s < SLOTS; ++s) m = max(m, key[s]);
      m = wave_max_u32(m);
      int sel = -1;   // wave-uniform: the lowest expert whose key is m
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        const uint64_t b = __builtin_amdgcn_ballot_w64(key[s] == m);
        if (sel < 0 && b != 0ull) sel = s * kWave + (int)__builtin_ctzll(b);
      }
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) key[s] = s * kWave + lane == sel ? 0u : key[s];
      if (lane == r) {
        mkey = m;
        ej = sel;
      }
    }
    if (lane >= k) ej = 0x7fffffff;
    // the value the key orders by: the logit itself, except that -0 comes back as +0,
    // which gives the same differences below
    const float val = lane < k ? key_value(mkey) : 0.f;
    const float l0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(val), 0));
    const float z = lane < k ? expf(val - l0) : 0.f;
    float sum = 0.f;
    for (int j = 0; j < k; ++j) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), j));
    int pos = 0;
    for (int q = 0; q < k; ++q) pos += __builtin_amdgcn_readlane(ej, q) < ej ? 1 : 0;
    if (lane < k) {
      ids_l[lane] = ej;
      w_l[lane] = z / sum;
      perm_l[pos] = lane;
      inv_l[lane] = pos;
      int* a = act_l[pos];
      a[0] = ej;
      a[1] = slot_l[ej];
      a[2] = pos;
      a[3] = pos + 1;
      a[4] = 0;
      a[5] = -1;
      a[6] = -1;
      a[7] = -1;
    }
    if (lane == 0) nact_l = k;
  };
  if constexpr (NT == 1) {   // NT == 1 means T == 1
    if (E <= kWave) route_one_token(std::integral_constant<int, 1>{});
    else if (E <= 2 * kWave) route_one_token(std::integral_constant<int, 2>{});
    else route_one_token(std::integral_constant<int, kMaxE / kWave>{});
  } else {
    route_general();
  }
  __syncthreads();
  const int na = nact_l;
  if (blockIdx.x == 0) {   // publish the routing
    if (tid < n) {
      rin.ids[tid] = ids_l[tid];
      rin.w[tid] = w_l[tid];
      rin.perm[tid] = perm_l[tid];
      rin.inv_perm[tid] = inv_l[tid];
    }
    for (int e = tid; e <= E; e += kGThreads) {   // E + 1 offsets (E may equal the block)
      int c = 0, o = 0;
      for (int q = 0; q < n; ++q) {
        const int eq = ids_l[q];
        c += eq == e ? 1 : 0;
        o += eq < e ? 1 : 0;
      }
      if (e < E) rin.counts[e] = c;
      rin.offsets[e] = o;
    }
    for (int i = tid; i < na * kActStride; i += kGThreads) rin.act[1 + i] = (&act_l[0][0])[i];
    if (tid == 0) rin.act[0] = na;
    if (!kFused && rin.tickets != nullptr)   // the down kernel's tickets start at zero
      for (int i = tid; i < rin.n_tickets; i += kGThreads) rin.tickets[i] = 0;
  }
  // 4. the workgroup's units u = blockIdx.x, + gridDim.x, ...: unit u is row group
  //    u % n_rg of active expert u / n_rg (the routing above is paid once per workgroup)
  const int n_rg = I / 16;
  const int nb = H / 32;
  const int nc = (nb + LM::kBlocksPerChunk - 1) / LM::kBlocksPerChunk;
  constexpr int64_t cb = code_bytes_per_block(FMT), sb = scale_bytes_per_block(FMT);
  const int lane_unit = unit16(FMT) ? lane : (lane >> 1);
  const int lblk = LM::blk(lane);
  const int koff = LM::koff(lane);
  for (int unit = blockIdx.x;; unit += gridDim.x) {
    const int j = unit / n_rg;
    if (j >= na) break;
    const int rg = unit % n_rg;
    const int slot = act_l[j][1];
    // the bucket range as the routing above wrote it, kept inside [0, n) and to at most NT
    // pairs whatever it holds, so that no store below can leave h
    const int lo = min(max(act_l[j][2], 0), n);
    const int np = min(max(act_l[j][3] - lo, 0), min(NT, n - lo));
    const int r0 = rg * 16;
    // fused: once wave 0's h stores of the unit have completed, the unit counts itself
    // done for its expert
    auto publish = [&]() {
      if (kFused && wave == 0) {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        if (lane == 0) {
          // the unit that completes its sub-counter adds one to the expert's ready count
          const int q = rg % kHandoffSplit;
          const int old = __hip_atomic_fetch_add(&fd.counters[j * kHandoffSplit + q], 1,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (old == handoff_units(n_rg, q) - 1)
            __hip_atomic_fetch_add(&fd.ready[j * kReadyStride], 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    };
    if (slot < 0 || slot >= n_slots) {
      for (int i = tid; i < np * 16; i += kGThreads) {   // wave 0: np * 16 <= 64
        uint16_t* dst = &h_out[(int64_t)(lo + i / 16) * I + r0 + i % 16];
        if constexpr (kFused) __hip_atomic_store(dst, (uint16_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else *dst = 0;
      }
      if (tid == 0 && err_flags && slot != kSlotMiss) atomicOr(err_flags, 1u);
      publish();
      continue;
    }
    // stream this row group of the expert's gate and up rows
    const int64_t unit0 = (int64_t)rg * nb * 16;
    const uint8_t* qa = gq + slot * qslot + unit0 * cb + lane * 16;
    const uint8_t* qb = uq + slot * qslot + unit0 * cb + lane * 16;
    const uint8_t* sa = gsc + slot * sslot + (unit0 + lane_unit) * sb;
    const uint8_t* sbp = usc + slot * sslot + (unit0 + lane_unit) * sb;
    const uint8_t* sa2 = super_base<FMT>(gsc + slot * sslot, I, H, rg, lane);
    const uint8_t* sbp2 = super_base<FMT>(usc + slot * sslot, I, H, rg, lane);
    const uint8_t* ha = hi_base<FMT>(gq + slot * qslot, I, H, unit0 + lane);
    const uint8_t* hb = hi_base<FMT>(uq + slot * qslot, I, H, unit0 + lane);
    const uint16_t* xrow[NT];
    const float* xsum[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int t = act_l[j][4 + (i < 4 ? i : 3)];
      xrow[i] = &xs[(t >= 0 ? t : 0) * H];
      xsum[i] = &xsum_l[kquant(FMT) ? (t >= 0 ? t : 0) * (H / 32) * sums_per_block(FMT) : 0];
    }
    constexpr bool kMma = mma_path(FMT, NT);
    float acc[2][NT];
    f32x4 acc4[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      acc4[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NT; ++i) acc[m][i] = 0.f;
    }
    // chunks per wave per batch: fewer with more tokens and with the k-quants' larger
    // chunk records, so that the batch stays in registers
    constexpr int kRU = RU > 0 ? RU
                      : FMT == kQ4_K ? (NT >= 4 ? 3 : NT >= 2 ? 4 : 6)
                      : FMT == kQ5_K || FMT == kQ6_K ? (NT >= 4 ? 2 : NT >= 2 ? 3 : 4)
                      : NT >= 4 ? 6 : kU;
    for (int cbase = 0; cbase < nc; cbase += kGWaves * kRU) {
      Chunk ca[kRU], cbk[kRU];
#pragma unroll
      for (int u = 0; u < kRU; ++u) {
        const int c = cbase + wave + kGWaves * u;
        const int b = c * LM::kBlocksPerChunk + lblk;
        const bool ok = c < nc && b < nb;
        const int cs = ok ? c : 0;
        load_chunk<FMT>(ca[u], qa + (int64_t)cs * 1024, sa + (int64_t)cs * LM::kScaleChunk,
                        sa2 + (int64_t)(cs >> 1) * 64, ha + (int64_t)cs * LM::kHiChunk, ok);
        load_chunk<FMT>(cbk[u], qb + (int64_t)cs * 1024, sbp + (int64_t)cs * LM::kScaleChunk,
                        sbp2 + (int64_t)(cs >> 1) * 64, hb + (int64_t)cs * LM::kHiChunk, ok);
      }
      __builtin_amdgcn_sched_barrier(0);   // the whole batch in flight before any is used
      if constexpr (kMma) {
        const int tm = lane & 15;   // the lane's token row of A
        const uint16_t* xr = xrow[0];
#pragma unroll
        for (int i = 1; i < NT; ++i) xr = tm == i ? xrow[i] : xr;
#pragma unroll
        for (int u = 0; u < kRU; ++u) {
          const int c = cbase + wave + kGWaves * u;
          const int xo = ca[u].ok ? c * LM::kKPerChunk + koff : 0;   // masked: any valid part
          bf16x8 av[4];
          mma_a(xr + xo, tm < NT, av);
          bf16x2 w[LM::kWPairs];
          widen<FMT>(ca[u], w);
          acc4[0] = mma_chunk(w, av, acc4[0]);
          widen<FMT>(cbk[u], w);
          acc4[1] = mma_chunk(w, av, acc4[1]);
        }
        continue;
      }
#pragma unroll
      for (int u = 0; u < kRU; ++u) {
        const int c = cbase + wave + kGWaves * u;
        const int xo = ca[u].ok ? c * LM::kKPerChunk + koff : 0;   // masked: any valid part
        bf16x2 w[LM::kWPairs];
        uint32_t xw[LM::kXWords];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const Chunk& ch = m == 0 ? ca[u] : cbk[u];
          widen<FMT>(ch, w);
#pragma unroll
          for (int i = 0; i < NT; ++i) {
#pragma unroll
            for (int q = 0; q < LM::kXWords / 4; ++q) {
              const u32x4 xq = *(const u32x4*)(xrow[i] + xo + q * 8);
              xw[4 * q + 0] = xq[0];
              xw[4 * q + 1] = xq[1];
              xw[4 * q + 2] = xq[2];
              xw[4 * q + 3] = xq[3];
            }
            const float* sx = xsum[i] + (kquant(FMT) ? xo / 32 * sums_per_block(FMT) : 0);
            acc[m][i] = dot_chunk_s<FMT>(w, xw, ch.ok ? ch.s : 0u, ch.s2, sx, acc[m][i]);
          }
        }
      }
    }
    // 5. lanes that share a row, then the 4 waves in a fixed order; SwiGLU; h in bf16
    if constexpr (kMma) {
      if (lane < 16) {   // D: lane l < 16 holds tokens 0..3 of row l
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int i = 0; i < NT; ++i) red[wave][i][m][lane] = acc4[m][i];
      }
    } else {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          float a = acc[m][i];
          if constexpr (unit16(FMT)) {
            a += wave_xor(a, 16);
            a += wave_xor(a, 32);
          } else {
            a += wave_xor(a, 1);
            a += wave_xor(a, 32);
          }
          acc[m][i] = a;
        }
      const bool writer = unit16(FMT) ? (lane < 16) : (lane < 32 && (lane & 1) == 0);
      if (writer) {
        const int r = LM::row(lane);
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int i = 0; i < NT; ++i) red[wave][i][m][r] = acc[m][i];
      }
    }
    __syncthreads();
    if (tid < NT * 16) {
      const int i = tid / 16, r = tid % 16;
      if (i < np) {
        float g = red[0][i][0][r], u = red[0][i][1][r];
#pragma unroll
        for (int q = 1; q < kGWaves; ++q) {
          g += red[q][i][0][r];
          u += red[q][i][1][r];
        }
        const uint16_t hv = f32_to_bf16_rne(silu_mul(g, u));
        uint16_t* dst = &h_out[(int64_t)(lo + i) * I + r0 + r];
        if constexpr (kFused) __hip_atomic_store(dst, hv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else *dst = hv;
      }
    }
    publish();
    __syncthreads();   // red is rewritten by the next unit
  }
  if constexpr (kFused) {
    // ---- down units v = blockIdx.x, + gridDim.x, ...: row group v % n_rgh of out, active
    //      expert v / n_rgh. The staged activation rows are no longer needed: xs now holds
    //      a batch's K slice of the unit's h rows, [NT][kSliceD].
    constexpr int kSliceD = kGWaves * RUD * LM::kKPerChunk;
    static_assert(NT * kSliceD <= NT * kRouteMaxH, "an h slice fits in the activation rows");
    constexpr int kSlicePieces = NT * (kSliceD / 8);
    constexpr int kPieces = (kSlicePieces + kGThreads - 1) / kGThreads;
    constexpr bool kMmaD = mma_path(FMT, NT);
    const int n_rgh = H / 16;
    const int nbd = I / 32;
    const int ncd = (nbd + LM::kBlocksPerChunk - 1) / LM::kBlocksPerChunk;
    const int n_rgi = I / 16;   // gate/up units of an expert
    uint16_t* hs = xs;
    __syncthreads();   // every wave is past its last read of the activation rows
    for (int v = blockIdx.x;; v += gridDim.x) {
      const int j = v / n_rgh;
      if (j >= na) break;
      const int rg = v % n_rgh;
      const int slot = act_l[j][1];
      const int lo = min(max(act_l[j][2], 0), n);
      const int np = min(max(act_l[j][3] - lo, 0), min(NT, n - lo));
      const int r0 = rg * 16;
      const bool valid = slot >= 0 && slot < n_slots;
      float acc[NT];
      f32x4 acc4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NT; ++i) acc[i] = 0.f;
      if (valid) {
        const int64_t unit0 = (int64_t)rg * nbd * 16;
        const uint8_t* qa = fd.q + slot * fd.q_slot + unit0 * cb + lane * 16;
        const uint8_t* sa = fd.s + slot * fd.s_slot + (unit0 + lane_unit) * sb;
        const uint8_t* sa2 = super_base<FMT>(fd.s + slot * fd.s_slot, H, I, rg, lane);
        const uint8_t* ha = hi_base<FMT>(fd.q + slot * fd.q_slot, H, I, unit0 + lane);
        for (int cbase = 0; cbase < ncd; cbase += kGWaves * RUD) {
          // 1. this wave's weight chunks of the batch (they do not depend on h)
          Chunk ca[RUD];
#pragma unroll
          for (int u = 0; u < RUD; ++u) {
            const int c = cbase + wave + kGWaves * u;
            const int b = c * LM::kBlocksPerChunk + lblk;
            const bool ok = c < ncd && b < nbd;
            const int cs = ok ? c : 0;
            load_chunk<FMT>(ca[u], qa + (int64_t)cs * 1024, sa + (int64_t)cs * LM::kScaleChunk,
                            sa2 + (int64_t)(cs >> 1) * 64, ha + (int64_t)cs * LM::kHiChunk, ok);
          }
          __builtin_amdgcn_sched_barrier(0);
          // 2. first batch: wait until every gate/up unit of expert j has published its h
          if (cbase == 0) {
            if (tid == 0) {
              const int need = min(kHandoffSplit, n_rgi);   // sub-counters with units
              for (int spins = 0;; ++spins) {
                const int got = __hip_atomic_load(&fd.ready[j * kReadyStride], __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
                if (got >= need) break;
                if (spins >= fd.spin_limit) {
                  if (err_flags) atomicOr(err_flags, 2u);
                  break;
                }
                __builtin_amdgcn_s_sleep(kPollSleep);
              }
            }
            __syncthreads();
          }
          // 3. the batch's K slice of the unit's h rows (device-coherent: stored by other
          //    workgroups of this launch), then into LDS
          const int k0 = cbase * LM::kKPerChunk;
          u32x4 xp[kPieces];
          bool xok[kPieces];
#pragma unroll
          for (int it = 0; it < kPieces; ++it) {
            const int idx0 = tid + it * kGThreads;
            const int idx = idx0 < kSlicePieces ? idx0 : 0;
            const int i = idx / (kSliceD / 8), q = idx % (kSliceD / 8);
            const int kk = k0 + q * 8;
            xok[it] = idx0 < kSlicePieces && i < np && kk < I;
            xp[it] = ld16_coherent(h_out + (int64_t)(lo + (xok[it] ? i : 0)) * I + (xok[it] ? kk : 0));
          }
          __syncthreads();   // the previous batch's reads of hs are done
#pragma unroll
          for (int it = 0; it < kPieces; ++it) {
            const int idx = tid + it * kGThreads;
            const int i = idx / (kSliceD / 8), q = idx % (kSliceD / 8);
            if (idx < kSlicePieces) *(u32x4*)&hs[i * kSliceD + q * 8] = xok[it] ? xp[it] : u32x4{0, 0, 0, 0};
          }
          __syncthreads();
          // 4. consume, as k_gemv does
          if constexpr (kMmaD) {
            const int tm = lane & 15;
#pragma unroll
            for (int u = 0; u < RUD; ++u) {
              const int c = cbase + wave + kGWaves * u;
              const int xo = (c - cbase) * LM::kKPerChunk + koff;
              bf16x8 av[4];
              mma_a(&hs[(tm < NT ? tm : 0) * kSliceD + xo], tm < NT, av);
              bf16x2 w[LM::kWPairs];
              widen<FMT>(ca[u], w);
              acc4 = mma_chunk(w, av, acc4);
            }
          } else {
#pragma unroll
            for (int u = 0; u < RUD; ++u) {
              const int c = cbase + wave + kGWaves * u;
              const int xo = (c - cbase) * LM::kKPerChunk + koff;
              bf16x2 w[LM::kWPairs];
              uint32_t xw[LM::kXWords];
              widen<FMT>(ca[u], w);
#pragma unroll
              for (int i = 0; i < NT; ++i) {
#pragma unroll
                for (int q = 0; q < LM::kXWords / 4; ++q) {
                  const u32x4 hq = *(const u32x4*)&hs[i * kSliceD + xo + q * 8];
                  xw[4 * q + 0] = hq[0];
                  xw[4 * q + 1] = hq[1];
                  xw[4 * q + 2] = hq[2];
                  xw[4 * q + 3] = hq[3];
                }
                acc[i] = dot_chunk<FMT>(w, xw, ca[u].ok ? ca[u].s : 0u, ca[u].s2, acc[i]);
              }
            }
          }
        }
      } else if (tid == 0 && err_flags && slot != kSlotMiss) {
        atomicOr(err_flags, 1u);
      }
      // 5. lanes that share a row, then the 4 waves in a fixed order (as k_gemv)
      if constexpr (kMmaD) {
        if (lane < 16) {
#pragma unroll
          for (int i = 0; i < NT; ++i) red[wave][i][0][lane] = acc4[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          float a = acc[i];
          if constexpr (unit16(FMT)) {
            a += wave_xor(a, 16);
            a += wave_xor(a, 32);
          } else {
            a += wave_xor(a, 1);
            a += wave_xor(a, 32);
          }
          acc[i] = a;
        }
        const bool writer = unit16(FMT) ? (lane < 16) : (lane < 32 && (lane & 1) == 0);
        if (writer) {
          const int r = LM::row(lane);
#pragma unroll
          for (int i = 0; i < NT; ++i) red[wave][i][0][r] = acc[i];
        }
      }
      __syncthreads();
      // 6. wave 0: y rows (device-coherent), the row group's ticket, and the combine by the
      //    workgroup that draws the last one
      if (wave == 0) {
        if (lane < NT * 16) {
          const int i = lane / 16, r = lane % 16;
          if (i < np) {
            float sum = 0.f;
            if (valid) {
              sum = red[0][i][0][r];
#pragma unroll
              for (int q = 1; q < kGWaves; ++q) sum += red[q][i][0][r];
            }
            __hip_atomic_store(&fd.y[(int64_t)(lo + i) * H + r0 + r], sum, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        int ticket = 0;
        if (lane == 0)
          ticket = __hip_atomic_fetch_add(&fd.tickets[rg], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ticket = __builtin_amdgcn_readfirstlane(ticket);
        if (ticket == na - 1 && lane < T * 16) {
          const int t = lane >> 4, r = lane & 15;
          float yv[kMaxK], wv[kMaxK];
#pragma unroll
          for (int jj = 0; jj < kMaxK; ++jj) {   // every load issued before the first use
            const int p = t * k + (jj < k ? jj : 0);
            wv[jj] = w_l[p];
            yv[jj] = __hip_atomic_load(&fd.y[(int64_t)inv_l[p] * H + r0 + r], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
          }
          float a = 0.f;
#pragma unroll
          for (int jj = 0; jj < kMaxK; ++jj)
            if (jj < k) a = fmaf(wv[jj], yv[jj], a);
          fd.out[(int64_t)t * H + r0 + r] = a;
        }
      }
      __syncthreads();   // red and hs are rewritten by the next unit
    }
  }
}

int gemv_nt(int fmt, int T) {
  if (T <= 1) return 1;
  if (T <= 2) return 2;
  if (T <= 4 || unit16(fmt)) return 4;
  return 8;
}

template <int FMT, bool GATED, int SRC>
hipError_t launch_gemv_t(const PoolView& a, const PoolView& b, const int32_t* slot_map,
                         int n_slots, int E, const int32_t* offsets, const int32_t* perm,
                         int T, int k, const uint16_t* src, int K, int rows, uint16_t* h,
                         float* y, uint32_t* err, const int32_t* act, hipStream_t stream) {
  const int n_act = min(E, T * k);
  dim3 grid(rows / 16, n_act);
#define MOE_GEMV_CASE(N, R)                                                                     \
  hipLaunchKernelGGL((k_gemv<FMT, GATED, SRC, N, R>), grid, dim3(kGThreads), 0, stream, a.q,    \
                     a.s, a.q_slot, a.s_slot, b.q, b.s, slot_map, n_slots, E, offsets, perm, k, \
                     src, K, rows, h, y, err, act, DownTail{})
  // 2 or 4 tokens of a 16-byte-unit format: a batch of 6 chunks per wave when the row
  // needs no more (4 waves share a row), e.g. K = 2880: 23 chunks
  const int need = ((K / 32 + LaneMap<FMT>::kBlocksPerChunk - 1) / LaneMap<FMT>::kBlocksPerChunk +
                    kGWaves - 1) / kGWaves;
  const bool six = unit16(FMT) && need <= 6;
  switch (gemv_nt(FMT, T)) {
    case 1: MOE_GEMV_CASE(1, kU); break;
    case 2:
      if constexpr (unit16(FMT)) {
        if (six) { MOE_GEMV_CASE(2, 6); break; }
      }
      MOE_GEMV_CASE(2, kU);
      break;
    case 4:
      if constexpr (unit16(FMT)) {
        if (six) { MOE_GEMV_CASE(4, 6); break; }
      }
      MOE_GEMV_CASE(4, kU);
      break;
    default:
      if constexpr (FMT == kQ8_0) MOE_GEMV_CASE(8, kU);
      break;
  }
#undef MOE_GEMV_CASE
  return hipGetLastError();
}

// Calls f(std::integral_constant<int, FMT>{}) for the runtime format.
template <class F>
hipError_t with_fmt(int fmt, F&& f) {
  switch (fmt) {
    case kMXFP4: return f(std::integral_constant<int, kMXFP4>{});
    case kQ8_0: return f(std::integral_constant<int, kQ8_0>{});
    case kQ4_K: return f(std::integral_constant<int, kQ4_K>{});
    case kQ5_K: return f(std::integral_constant<int, kQ5_K>{});
    case kQ6_K: return f(std::integral_constant<int, kQ6_K>{});
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gate_up_gemv(int fmt, const PoolView& gate, const PoolView& up,
                               const int32_t* slot_map, int n_slots, int E, const uint16_t* x,
                               int T, int k, int H, int I, const int32_t* offsets,
                               const int32_t* perm, uint16_t* h, uint32_t* err,
                               const int32_t* act, hipStream_t stream) {
  return with_fmt(fmt, [&](auto F) {
    if (act != nullptr)
      return launch_gemv_t<F(), true, kSrcAct>(gate, up, slot_map, n_slots, E, offsets, perm, T,
                                               k, x, H, I, h, nullptr, err, act, stream);
    return launch_gemv_t<F(), true, kSrcOffsets>(gate, up, slot_map, n_slots, E, offsets, perm,
                                                 T, k, x, H, I, h, nullptr, err, nullptr, stream);
  });
}


hipError_t coresident_wgs(const void* kern, hipStream_t stream, int* out);

hipError_t launch_gate_up_route(int fmt, const PoolView& gate, const PoolView& up,
                                const int32_t* slot_map, int n_slots, int E, const uint16_t* x,
                                int T, int k, int H, int I, const RouteIn& rin, uint16_t* h,
                                uint32_t* err, hipStream_t stream) {
  if (!route_fused_ok(T, H, E) || rin.T != T || rin.ns != route_fused_split(H) ||
      gate.q_slot != up.q_slot || gate.s_slot != up.s_slot)
    return hipErrorInvalidValue;
  const int n_units = (I / 16) * min(E, T * k);
  const int nt = gemv_nt(fmt, T);
  return with_fmt(fmt, [&](auto F) {
    // at most kRoutedMaxWG workgroups, and no more than fit on the device at once: a
    // workgroup that waited for a slot would pay the routing late and lengthen the tail
#define MOE_ROUTED_CASE(N, R)                                                                 \
  do {                                                                                        \
    const void* kern = (const void*)k_gate_up_routed<F(), N, R>;                              \
    int fit = kRoutedMaxWG;                                                                   \
    if (coresident_wgs(kern, stream, &fit) != hipSuccess || fit < 1) fit = kRoutedMaxWG;      \
    const dim3 grid(min(n_units, min(fit, kRoutedMaxWG)));                                     \
    hipLaunchKernelGGL((k_gate_up_routed<F(), N, R>), grid, dim3(kGThreads), 0, stream,       \
                       gate.q, gate.s, up.q, up.s, gate.q_slot, gate.s_slot, slot_map,        \
                       n_slots, E, k, x, H, I, h, err, rin, FusedDown{});                     \
  } while (0)
    // one token: a batch of chunks per wave (4 waves share a row) that wastes fewer slots
    // on masked chunks than the format's default (8 chunks; Q4_K 6; Q5_K, Q6_K 4)
    const int bpc = LaneMap<F()>::kBlocksPerChunk;
    const int need = ((H / 32 + bpc - 1) / bpc + kGWaves - 1) / kGWaves;
    const int dflt = F() == kQ4_K ? 6 : (F() == kQ5_K || F() == kQ6_K) ? 4 : kU;
    // the batch (4, 6 or the default) that leaves the fewest masked slots, larger on ties
    auto slots = [&](int ru) { return (need + ru - 1) / ru * ru; };
    int ru = dflt;
    if (6 < dflt && slots(6) < slots(ru)) ru = 6;
    if (4 < dflt && slots(4) < slots(ru)) ru = 4;
    constexpr int kDflt = F() == kQ4_K ? 6 : (F() == kQ5_K || F() == kQ6_K) ? 4 : kU;
    bool done = false;
    if constexpr (kDflt > 4)
      if (nt == 1 && ru == 4) {
        MOE_ROUTED_CASE(1, 4);
        done = true;
      }
    if constexpr (kDflt > 6)
      if (!done && nt == 1 && ru == 6) {
        MOE_ROUTED_CASE(1, 6);
        done = true;
      }
    if (done) {
    } else if (nt == 1) MOE_ROUTED_CASE(1, 0);
    else if (nt == 2) MOE_ROUTED_CASE(2, 0);
    else MOE_ROUTED_CASE(4, 0);
#undef MOE_ROUTED_CASE
    return hipGetLastError();
  });
}

// Workgroups of `kern` (256 threads) that fit on the stream's device at once.
hipError_t coresident_wgs(const void* kern, hipStream_t stream, int* out) {
  int dev = 0;
  hipError_t e;
  if (stream != nullptr) {
    hipDevice_t d = 0;
    e = hipStreamGetDevice(stream, &d);
    dev = (int)d;
  } else {
    e = hipGetDevice(&dev);
  }
  if (e != hipSuccess) return e;
  int ncu = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kGThreads, 0);
  if (e != hipSuccess) return e;
  *out = ncu * per_cu;
  return hipSuccess;
}

template <int FMT, int NT, int RU, int RUD>
hipError_t launch_fused_t(const PoolView& gate, const PoolView& up, const PoolView& down,
                          const int32_t* slot_map, int n_slots, int E, const uint16_t* x, int T,
                          int k, int H, int I, const RouteIn& rin, uint16_t* h,
                          const FusedDown& fd, uint32_t* err, hipStream_t stream) {
  const void* kern = reinterpret_cast<const void*>(&k_gate_up_routed<FMT, NT, RU, RUD>);
  int cap = 0;
  hipError_t e = coresident_wgs(kern, stream, &cap);
  if (e != hipSuccess) return e;
  const int n_act = min(E, T * k);
  const int units = max(I / 16, H / 16) * n_act;
  const int grid = min(units, cap);
  if (grid < 1) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((k_gate_up_routed<FMT, NT, RU, RUD>), dim3(grid), dim3(kGThreads), 0, stream,
                     gate.q, gate.s, up.q, up.s, gate.q_slot, gate.s_slot, slot_map, n_slots, E,
                     k, x, H, I, h, err, rin, fd);
  return hipGetLastError();
}

// One token: its k experts (all distinct) share the 8 waves, kDCWaves / k of them per
// expert, so each wave streams ceil(chunks / (kDCWaves / k)) chunks of the row; a batch of
// kDCUShort covers that when it is short (e.g. I = 768 with 8 experts: 6 chunks a wave).
constexpr int kDCUShort = 6;
inline bool down_short_batch(int fmt, int T, int k, int I) {
  if (T != 1 || k < 1 || k > kDCWaves) return false;
  const int bpc = unit16(fmt) ? 4 : 2;   // blocks per 1 KiB chunk (LaneMap)
  const int nc = (I / 32 + bpc - 1) / bpc;
  const int per = kDCWaves / k;
  return (nc + per - 1) / per <= kDCUShort;
}

// The small-batch down kernel's bound on pairs per expert for T tokens: 1, 2, 4 or 8.
template <typename Fn>
void with_pairs_per_expert(int T, Fn&& fn) {
  if (T <= 1) fn(std::integral_constant<int, 1>{});
  else if (T <= 2) fn(std::integral_constant<int, 2>{});
  else if (T <= 4) fn(std::integral_constant<int, 4>{});
  else fn(std::integral_constant<int, kDCMaxPairs>{});
}

hipError_t launch_down_gemv(int fmt, const PoolView& down, const int32_t* slot_map, int n_slots,
                            int E, int T, int k, int H, int I, const int32_t* offsets,
                            const uint16_t* h, float* y, uint32_t* err, hipStream_t stream) {
  // the kernel the fused layer would use for this shape (down_small_preferred), without
  // the combine, so that the stage calls reproduce the layer bit for bit
  return with_fmt(fmt, [&](auto F) {
    if (down_small_preferred(F(), T, k, E, I)) {
      const bool short_batch = down_short_batch(F(), T, k, I);
      with_pairs_per_expert(T, [&](auto NP) {
        if constexpr (NP() == 1) {
          if (short_batch) {
            hipLaunchKernelGGL((k_down_small<F(), false, 1, kDCUShort>), dim3(H / 16),
                               dim3(kDCWaves * kWave), 0, stream, down.q, down.s, down.q_slot,
                               down.s_slot, n_slots, E, nullptr, offsets, slot_map, h, T, k, H,
                               I, nullptr, nullptr, y, nullptr, err);
            return;
          }
        }
        hipLaunchKernelGGL((k_down_small<F(), false, NP()>), dim3(H / 16),
                           dim3(kDCWaves * kWave), 0, stream, down.q, down.s, down.q_slot,
                           down.s_slot, n_slots, E, nullptr, offsets, slot_map, h, T, k, H, I,
                           nullptr, nullptr, y, nullptr, err);
      });
      return hipGetLastError();
    }
    return launch_gemv_t<F(), false, kSrcOffsets>(down, down, slot_map, n_slots, E, offsets,
                                                  nullptr, T, k, h, I, H, nullptr, y, err,
                                                  nullptr, stream);
  });
}

bool decode_fused_ok(int T, int H, int E) { return route_fused_ok(T, H, E); }

hipError_t launch_decode_fused(int fmt, const PoolView& gate, const PoolView& up,
                               const PoolView& down, const int32_t* slot_map, int n_slots, int E,
                               const uint16_t* x, int T, int k, int H, int I, const RouteIn& rin,
                               uint16_t* h, float* y, float* out, int32_t* sync, uint32_t* err,
                               hipStream_t stream) {
  if (!decode_fused_ok(T, H, E) || rin.T != T || rin.ns != route_fused_split(H) ||
      gate.q_slot != up.q_slot || gate.s_slot != up.s_slot || sync == nullptr)
    return hipErrorInvalidValue;
  RouteIn r = rin;
  r.tickets = nullptr;   // the sync words were zeroed by the router kernel
  r.n_tickets = 0;
  int32_t* counters = sync + H / 16;
  const FusedDown fd{down.q, down.s, down.q_slot, down.s_slot, y, out, counters,
                     counters + kFuseMaxPairs * kHandoffSplit, sync, kSpinLimit};
  const int nt = gemv_nt(fmt, T);
  return with_fmt(fmt, [&](auto F) -> hipError_t {
    constexpr int FMT = F();
    // gate/up batch: as launch_gate_up_route chooses it
    const int bpc = LaneMap<FMT>::kBlocksPerChunk;
    const int need = ((H / 32 + bpc - 1) / bpc + kGWaves - 1) / kGWaves;
    const int dflt = FMT == kQ4_K ? 6 : (FMT == kQ5_K || FMT == kQ6_K) ? 4 : kU;
    auto slots = [](int nd, int ru) { return (nd + ru - 1) / ru * ru; };
    int ru = dflt;
    if (6 < dflt && slots(need, 6) < slots(need, ru)) ru = 6;
    if (4 < dflt && slots(need, 4) < slots(need, ru)) ru = 4;
    // down batch: 2, 6 or 8 (k-quants: 2, 6 / 2, 4), the fewest masked slots
    const int needd = ((I / 32 + bpc - 1) / bpc + kGWaves - 1) / kGWaves;
    const int rud_max = FMT == kQ4_K ? 6 : (FMT == kQ5_K || FMT == kQ6_K) ? 4 : 8;
    int rud = rud_max;
    if (6 < rud_max && slots(needd, 6) < slots(needd, rud)) rud = 6;
    if (slots(needd, 2) < slots(needd, rud)) rud = 2;
    auto go = [&](auto NTc, auto RUc) -> hipError_t {
      constexpr int NT = decltype(NTc)::value, RU = decltype(RUc)::value;
      if (rud == 2)
        return launch_fused_t<FMT, NT, RU, 2>(gate, up, down, slot_map, n_slots, E, x, T, k, H, I,
                                              r, h, fd, err, stream);
      if constexpr (FMT == kQ5_K || FMT == kQ6_K) {
        return launch_fused_t<FMT, NT, RU, 4>(gate, up, down, slot_map, n_slots, E, x, T, k, H, I,
                                              r, h, fd, err, stream);
      } else {
        if (rud == 6 || FMT == kQ4_K)
          return launch_fused_t<FMT, NT, RU, 6>(gate, up, down, slot_map, n_slots, E, x, T, k, H,
                                                I, r, h, fd, err, stream);
        if constexpr (FMT != kQ4_K)
          return launch_fused_t<FMT, NT, RU, 8>(gate, up, down, slot_map, n_slots, E, x, T, k, H,
                                                I, r, h, fd, err, stream);
        return hipErrorInvalidValue;
      }
    };
    using I1 = std::integral_constant<int, 1>;
    constexpr int kDflt = FMT == kQ4_K ? 6 : (FMT == kQ5_K || FMT == kQ6_K) ? 4 : kU;
    if (nt == 1) {   // only the batches that can differ from the default are instantiated
      if constexpr (kDflt > 4)
        if (ru == 4) return go(I1{}, std::integral_constant<int, 4>{});
      if constexpr (kDflt > 6)
        if (ru == 6) return go(I1{}, std::integral_constant<int, 6>{});
      return go(I1{}, std::integral_constant<int, 0>{});
    }
    if (nt == 2) return go(std::integral_constant<int, 2>{}, std::integral_constant<int, 0>{});
    return go(std::integral_constant<int, 4>{}, std::integral_constant<int, 0>{});
  });
}

bool down_ticket_ok(int T, int k, int E) {
  return T >= 1 && T <= kFuseMaxT && k >= 1 && k <= kMaxK && E >= 1;
}

hipError_t launch_down_ticket(int fmt, const PoolView& down, int n_slots, int E, int T, int k,
                              int H, int I, const int32_t* act, const uint16_t* h,
                              const int32_t* inv_perm, const float* topk_w, float* y,
                              float* out, int32_t* tickets, uint32_t* err, hipStream_t stream) {
  if (!down_ticket_ok(T, k, E) || tickets == nullptr) return hipErrorInvalidValue;
  const DownTail tail{inv_perm, topk_w, out, tickets, T};
  // one workgroup per (16-row group of out, active expert): at most min(E, T k) experts
  dim3 grid(H / 16, min(E, T * k));
  return with_fmt(fmt, [&](auto F) {
    constexpr int FMT = F();
    // chunks per wave per batch: of the sizes the format's registers allow, the one that
    // leaves the fewest masked slots in the row's batches (the larger on a tie)
    // (MXFP4 and Q8_0 also 14 or 16 for long rows: a wave's batches are sequential round
    // trips, so fewer, larger batches keep more bytes in flight)
    const int bpc = LaneMap<FMT>::kBlocksPerChunk;
    const int need = ((I / 32 + bpc - 1) / bpc + kGWaves - 1) / kGWaves;
    constexpr bool kLong = FMT == kMXFP4 || FMT == kQ8_0;
    const int ru_max = FMT == kQ4_K ? 6 : (FMT == kQ5_K || FMT == kQ6_K) ? 4 : kLong && need > 8 ? 16 : 8;
    auto slots = [&](int ru) { return (need + ru - 1) / ru * ru; };
    int ru = ru_max;
    for (int c = ru_max - 2; c >= 2; c -= 2)
      if ((c <= 8 || c == 14) && slots(c) < slots(ru)) ru = c;
#define MOE_DT_CASE(N, R)                                                                     \
  hipLaunchKernelGGL((k_gemv<FMT, false, kSrcAct, N, R, true>), grid, dim3(kGThreads), 0,     \
                     stream, down.q, down.s, down.q_slot, down.s_slot, nullptr, nullptr,      \
                     nullptr, n_slots, E, nullptr, nullptr, k, h, I, H, nullptr, y, err, act, \
                     tail)
    auto go = [&](auto NTc) {
      constexpr int NT = decltype(NTc)::value;
      if (ru == 2) MOE_DT_CASE(NT, 2);
      else if (ru == 4) MOE_DT_CASE(NT, 4);
      else if constexpr (FMT != kQ5_K && FMT != kQ6_K) {
        if (ru == 6) MOE_DT_CASE(NT, 6);
        else if constexpr (FMT != kQ4_K) {
          if (ru == 8) MOE_DT_CASE(NT, 8);
          else if (ru == 14) MOE_DT_CASE(NT, 14);
          else MOE_DT_CASE(NT, 16);
        }
      }
    };
    if (T <= 1) go(std::integral_constant<int, 1>{});
    else if (T <= 2) go(std::integral_constant<int, 2>{});
    else go(std::integral_constant<int, 4>{});
#undef MOE_DT_CASE
    return hipGetLastError();
  });
}

bool down_combine_small_ok(int T, int k, int E, int I) {
  const int np = T * k;
  return np >= 1 && np <= kDCMaxPairs && (int64_t)np * I <= kDCMaxH && min(E, np) <= kDCWaves;
}

// The small-batch down kernel gives each workgroup a 16-row group of every active expert;
// where that is at most kDCPreferBytes of weights it beats one workgroup per (row group,
// expert) with the ticket combine, whose tail of device-scope round trips (y stores, the
// ticket, y loads) outweighs its finer split: measured, Qwen-A3B-shaped (52 KB per
// workgroup) 53.7 K against 48.7 K tokens/s; GPT-OSS-shaped (98 KB) even; Mixtral-shaped
// Q8_0 (487 KB) 13.5 K against 14.1 K, Q4_K (258 KB) 18.1 K against 19.2 K.
constexpr int64_t kDCPreferBytes = 128 << 10;
bool down_small_preferred(int fmt, int T, int k, int E, int I) {
  if (!down_combine_small_ok(T, k, E, I)) return false;
  const int64_t per_block = code_bytes_per_block(fmt) + scale_bytes_per_block(fmt) +
                            hi_bytes_per_block(fmt);
  const int64_t bytes = (int64_t)16 * min(E, T * k) * (I / 32) * per_block;
  return bytes <= kDCPreferBytes;
}

hipError_t launch_down_combine_small(int fmt, const PoolView& down, int n_slots, int E, int T,
                                     int k, int H, int I, const int32_t* act, const uint16_t* h,
                                     const int32_t* inv_perm, const float* topk_w, float* y,
                                     float* out, uint32_t* err, hipStream_t stream) {
  if (!down_combine_small_ok(T, k, E, I)) return hipErrorInvalidValue;
  return with_fmt(fmt, [&](auto F) {
    const bool short_batch = down_short_batch(F(), T, k, I);
    with_pairs_per_expert(T, [&](auto NP) {
      if constexpr (NP() == 1) {
        if (short_batch) {
          hipLaunchKernelGGL((k_down_small<F(), true, 1, kDCUShort>), dim3(H / 16),
                             dim3(kDCWaves * kWave), 0, stream, down.q, down.s, down.q_slot,
                             down.s_slot, n_slots, E, act, nullptr, nullptr, h, T, k, H, I,
                             inv_perm, topk_w, y, out, err);
          return;
        }
      }
      hipLaunchKernelGGL((k_down_small<F(), true, NP()>), dim3(H / 16), dim3(kDCWaves * kWave), 0,
                         stream, down.q, down.s, down.q_slot, down.s_slot, n_slots, E, act,
                         nullptr, nullptr, h, T, k, H, I, inv_perm, topk_w, y, out, err);
    });
    return hipGetLastError();
  });
}

}  // namespace moe
