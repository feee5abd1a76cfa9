// Expert FFN for many tokens (prefill): grouped GEMM on bf16 MFMA over the experts' blocks.
//
// Once tokens are grouped by expert (tinyserve README, "How it works" item 6) each expert's
// work is a dense contraction [n_e x K] x [K x N]; the llama.cpp discussion's follow-up
// ("Formal gate results") runs it as a grouped quantized matmul after the mapping rewrite.
// Here one launch covers every expert:
//   * the workgroup grid is sized for the worst case, sum_e ceil(n_e / BM) <= T*k/BM + E
//     row tiles, times the column tiles; each workgroup finds its (expert, row tile) from
//     the bucket offsets and exits if it has none, so the host never reads the counts;
//   * A rows are gathered through perm on load (gate/up: x[perm[pos] / k]; down: h[pos]);
//   * B comes straight from the tiled pool, whose 16-byte units hold one 32-element block
//     of one weight row, 16 rows side by side;
//   * the weights enter the MFMAs as exact bf16 values: MXFP4 codes widened with the
//     power-of-two scale folded in, Q6_K as two exact bf16 parts of each sc * (q - 32) with
//     d applied per K step, Q8_0 and Q4_K / Q5_K as their integer codes with the fp32 block
//     scales (and mins) applied to each block's MFMA result;
//   * gate and up tiles of the same columns live in the same wave, so SwiGLU is applied in
//     registers and h is written once, rounded to bf16; the down projection writes fp32 y
//     with nontemporal stores (y is read once, by the combine, and is far larger than the
//     caches: the stores then do not evict the A and B tiles other workgroups still read).
// Two kernels: k_ggemm_mx (MXFP4, Q6_K) loads its tiles straight into LDS; k_ggemm (Q8_0,
// Q4_K, Q5_K) stages them through registers one K step ahead.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kTThreads = 256;
constexpr int kBK = 128;          // K per pipeline step
constexpr int kLdsStride = kBK * 2 + 16;   // bytes per A row in LDS (padded)

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *(const u32x4*)p; }

// Which (expert, first position) a row tile index maps to; returns false if none.
__device__ bool map_row_tile(const int32_t* __restrict__ offsets, int E, int bm, int mt,
                             int* e_out, int* m0_out, int* tmp4, int* sh) {
  const int e = threadIdx.x;
  int lo = 0, n = 0;
  if (e < E) {
    lo = offsets[e];
    n = offsets[e + 1] - lo;
  }
  const int nt = (n + bm - 1) / bm;
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
    sh[1] = lo + (mt - cum) * bm;
  }
  __syncthreads();
  *e_out = sh[0];
  *m0_out = sh[1];
  return sh[0] >= 0;
}

// B of one K step (4 blocks = 128 K) for the workgroup's NG row groups (16 NG weight rows):
// in the tiled pool layout each row group's step is one contiguous run of 64 units
// (4 blocks x 16 rows), so the step is copied verbatim into LDS and a lane's MFMA operand
// is unit `lane` (MXFP4) or units 16 j + lane % 16 (Q8_0) of its row group's run.
template <int FMT, int NG>   // NG: weight row groups (16 rows each) per tile
struct BStage {
  static constexpr int kRunQ = 64 * code_bytes_per_block(FMT);   // code bytes per row group
  static constexpr int kRunS = 64 * scale_bytes_per_block(FMT);  // scale bytes per row group
  static constexpr int kQPieces = NG * kRunQ / 16 / kTThreads;   // 16-byte code pieces/thread
  // Q4_K: the 16 rows' (d, dmin) records of the step's super-block, per row group
  static constexpr int kRunS2 = kquant(FMT) ? kRowGroup * (int)kSuperBytes : 4;
  // Q5_K: the high-bit dwords of the run's 64 units
  static constexpr int kRunH = hi_bytes_per_block(FMT) ? 64 * (int)hi_bytes_per_block(FMT) : 4;
  static constexpr int kHDwords = NG * kRunH / 4 / kTThreads;  // high-part dwords per thread
};

// Q8_0, Q4_K and Q5_K: tiles of 128 bucket rows x 128 weight rows (waves 2 x 2). Each wave
// computes a 64 x 64 block of the tile (gate/up: 32 gate + the same 32 up columns, twice).
template <int FMT, bool GATED>
__global__ __launch_bounds__(kTThreads, 2) void k_ggemm(
    const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as, int64_t qslot,
    int64_t sslot, const uint8_t* __restrict__ bq, const uint8_t* __restrict__ bs,
    const int32_t* __restrict__ slot_map, int n_slots, int E,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm, int k,
    const uint16_t* __restrict__ src, int K, int N, int n_mtiles, int n_ntiles,
    uint16_t* __restrict__ h_out, float* __restrict__ y_out, uint32_t* __restrict__ err_flags) {
  constexpr int BM = 128;                     // bucket rows per tile
  constexpr int WM = BM / 64, WN = 4 / WM;   // waves along rows / columns
  constexpr int NG = 4 * WN;                  // weight row groups per tile
  constexpr int RPT = BM / 16;                // A rows staged per thread
  static_assert(FMT != kMXFP4 && FMT != kQ6_K, "MXFP4 and Q6_K run k_ggemm_mx");
  using BS = BStage<FMT, NG>;
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[BM * kLdsStride];
  // Q8_0 codes are staged already widened to bf16 (2 bytes per code): both waves that
  // read a B fragment would otherwise widen it each
  constexpr int kBqWiden = FMT == kQ8_0 ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint8_t lds_bq[NG * BS::kRunQ * kBqWiden];
  __shared__ __attribute__((aligned(16))) uint8_t lds_bs[NG * BS::kRunS];
  __shared__ __attribute__((aligned(16))) uint8_t lds_bs2[NG * BS::kRunS2];
  __shared__ __attribute__((aligned(16))) uint8_t lds_bh[NG * BS::kRunH];
  __shared__ int tmp4[4];
  __shared__ int sh[2];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int wm = wave / WN, wn = wave % WN;
  // XCD-aware 2-D order: workgroups are dealt to the 8 XCDs in turn (XCD x runs
  // workgroups x, x + 8, ...). Tile i of a list that walks super-tiles of 8 row tiles x 8
  // column tiles (row-major inside each) goes to the XCD of the 64-tile run it lies in, so
  // an XCD's L2 serves A rows to 8 column tiles and B slices to 8 row tiles.
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int64_t i = (int64_t)(local >> 6) * 512 + xcd * 64 + (local & 63);
  if (i >= (int64_t)n_mtiles * n_ntiles) return;   // padding of the grid
  const int sr = (int)(i / (8LL * n_ntiles));       // super-row: row tiles 8 sr ..
  const int h = min(8, n_mtiles - 8 * sr);          // its row tiles
  const int jj = (int)(i - 8LL * n_ntiles * sr);
  const int gcol = jj / (8 * h);                    // column group: column tiles 8 gcol ..
  const int w = min(8, n_ntiles - 8 * gcol);        // its column tiles
  const int kk = jj - 8 * h * gcol;
  const int mt = 8 * sr + kk / w;
  const int nt = 8 * gcol + kk % w;
  int e, m0;
  if (!map_row_tile(offsets, E, BM, mt, &e, &m0, tmp4, sh)) return;
  const int mend = offsets[e + 1];
  const int slot = slot_map[e];
  // columns of this workgroup: GATED -> 32 WN gate + the same 32 WN up columns; else 64 WN
  const int n0 = GATED ? nt * 32 * WN : nt * 64 * WN;
  if (slot < 0 || slot >= n_slots) {
    const int ncols = GATED ? 32 * WN : 64 * WN;
    for (int i = threadIdx.x; i < BM * ncols; i += kTThreads) {
      const int pos = m0 + i / ncols, n = n0 + i % ncols;
      if (pos < mend && n < N) {
        if (GATED) h_out[(int64_t)pos * N + n] = 0;
        else y_out[(int64_t)pos * N + n] = 0.f;
      }
    }
    if (threadIdx.x == 0 && err_flags && slot != kSlotMiss) atomicOr(err_flags, 1u);
    return;
  }
  const int nb = K / 32;
  const int nsteps = (K + kBK - 1) / kBK;

  // ---- A staging: thread handles 16-byte piece (tid % 16) of rows tid/16 + 16 j. Rows
  // past the tile's end repeat its last row: their results are never stored. Only the
  // last K step (past K) is masked to zeros, so that nothing but zeros meets the masked B.
  // The thread's pieces are addressed as 16-byte units of src: a 32-bit unit index reaches
  // 2^35 elements (64 GiB of bf16), the limit the host checks for x and h, where an
  // element offset would wrap at 2^32 and costs a second register per row as 64 bits.
  const int piece = threadIdx.x & 15;
  const int rbase = threadIdx.x >> 4;
  const u32x4* src16 = (const u32x4*)src;
  const uint32_t kp = (uint32_t)K / 8;   // 16-byte units per row
  uint32_t arow[RPT];   // unit index of the thread's piece in each of its rows
  {
    int prow[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j)   // all perm loads first
      prow[j] = GATED ? perm[min(m0 + rbase + 16 * j, mend - 1)] : min(m0 + rbase + 16 * j, mend - 1);
#pragma unroll
    for (int j = 0; j < RPT; ++j)
      arow[j] = (uint32_t)(GATED ? prow[j] / k : prow[j]) * kp + (uint32_t)piece;
  }
  u32x4 areg[RPT];
  auto load_a = [&](int c) {
    const int kk = c * kBK;
    if (kk + kBK <= K) {
#pragma unroll
      for (int j = 0; j < RPT; ++j) areg[j] = src16[arow[j] + (uint32_t)(kk / 8)];
    } else {
      const bool ok = kk + piece * 8 < K;
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const u32x4 v = src16[arow[j] + (uint32_t)(ok ? kk / 8 : 0)];
        areg[j] = ok ? v : u32x4{0, 0, 0, 0};
      }
    }
  };

  // ---- B staging: local row group g (0 .. NG-1) of the tile. GATED: g < NG/2 -> gate rows
  // n0/16 + g, g >= NG/2 -> up rows n0/16 + g - NG/2; else rows n0/16 + g. A row group past
  // N reads group 0 (its columns are never stored). Thread t copies code pieces
  // t + 256 p of the NG runs and, for t < NG * kRunS / 4, one dword of scales.
  const uint8_t* q0 = aq + (int64_t)slot * qslot;
  const uint8_t* s0 = as + (int64_t)slot * sslot;
  const uint8_t* q1 = GATED ? bq + (int64_t)slot * qslot : q0;
  const uint8_t* s1 = GATED ? bs + (int64_t)slot * sslot : s0;
  auto group_base = [&](int g, const uint8_t** qb, const uint8_t** sb) {
    const int rg = GATED ? n0 / 16 + g % (NG / 2) : n0 / 16 + g;
    const int rgc = rg * 16 < N ? rg : 0;
    const int64_t u0 = (int64_t)rgc * nb * 16;   // first unit of the row group
    *qb = (GATED && g >= NG / 2 ? q1 : q0) + u0 * code_bytes_per_block(FMT);
    *sb = (GATED && g >= NG / 2 ? s1 : s0) + u0 * scale_bytes_per_block(FMT);
  };
  const uint8_t* bqp[BS::kQPieces];
  int bq_blk[BS::kQPieces];   // block of the step that the piece lies in
#pragma unroll
  for (int p = 0; p < BS::kQPieces; ++p) {
    const int off = (threadIdx.x + kTThreads * p) * 16;   // byte in the 8 runs
    const int g = off / BS::kRunQ;
    const uint8_t* qb;
    const uint8_t* sb;
    group_base(g, &qb, &sb);
    bqp[p] = qb + (off % BS::kRunQ);
    bq_blk[p] = (off % BS::kRunQ) / (16 * code_bytes_per_block(FMT));
  }
  constexpr int kSDwords = NG * BS::kRunS / 4;
  static_assert(kSDwords <= kTThreads, "one scale dword per thread at most");
  const bool s_thread = threadIdx.x < kSDwords;
  const uint8_t* bsp;
  int bs_blk;
  {
    const int off = (s_thread ? threadIdx.x : 0) * 4;
    const int g = off / BS::kRunS;
    const uint8_t* qb;
    const uint8_t* sb;
    group_base(g, &qb, &sb);
    bsp = sb + (off % BS::kRunS);
    bs_blk = (off % BS::kRunS) / (16 * scale_bytes_per_block(FMT));
  }
  // Q4_K super-block records: thread t < 128 copies row t % 16 of local row group t / 16
  static_assert(!kquant(FMT) || NG * kRowGroup <= kTThreads, "one record per thread");
  const bool s2_thread = kquant(FMT) && threadIdx.x < NG * kRowGroup;
  const uint8_t* bs2p = nullptr;
  if constexpr (kquant(FMT)) {
    const int g = (s2_thread ? threadIdx.x : 0) / kRowGroup;
    const int rg = GATED ? n0 / 16 + g % (NG / 2) : n0 / 16 + g;
    const int rgc = rg * 16 < N ? rg : 0;
    const int nsb = nb / kSuperBlocks;
    bs2p = (GATED && g >= NG / 2 ? s1 : s0) + super_region(N, K) +
           ((int64_t)rgc * nsb * kRowGroup + (threadIdx.x & 15)) * kSuperBytes;
  }
  // Q5_K / Q6_K high-part dwords: thread t copies dwords t + 256 h of the 8 runs
  // (kRunH / 4 per run)
  constexpr int kHD = BS::kHDwords > 0 ? BS::kHDwords : 1;
  const uint8_t* bhp[kHD];
  uint32_t hreg[kHD];
#pragma unroll
  for (int h = 0; h < kHD; ++h) {
    bhp[h] = nullptr;
    hreg[h] = 0u;
  }
  if constexpr (hi_bytes_per_block(FMT) > 0) {
#pragma unroll
    for (int h = 0; h < kHD; ++h) {
      const int dw = threadIdx.x + kTThreads * h;
      const int g = dw / (BS::kRunH / 4);
      const int rg = GATED ? n0 / 16 + g % (NG / 2) : n0 / 16 + g;
      const int rgc = rg * 16 < N ? rg : 0;
      bhp[h] = (GATED && g >= NG / 2 ? q1 : q0) + hi_region(N, K) +
               (int64_t)rgc * nb * 16 * hi_bytes_per_block(FMT) + (dw % (BS::kRunH / 4)) * 4;
    }
  }
  u32x4 breg[BS::kQPieces];
  uint32_t sreg = 0, s2reg = 0;
  auto load_b = [&](int c) {
    // a step's run starts 4 blocks (64 units) after the previous one's; pieces of blocks
    // past the end of the row re-read step 0 (masked when consumed)
#pragma unroll
    for (int p = 0; p < BS::kQPieces; ++p) {
      const int cs = 4 * c + bq_blk[p] < nb ? c : 0;
      breg[p] = ldg16(bqp[p] + (int64_t)cs * BS::kRunQ);
    }
    if (s_thread) {
      const int cs = 4 * c + bs_blk < nb ? c : 0;
      sreg = *(const uint32_t*)(bsp + (int64_t)cs * BS::kRunS);
    }
    if constexpr (kquant(FMT)) {
      // step c's blocks 4c .. 4c+3 lie in super-block c / 2 (K is a multiple of 256)
      if (s2_thread) s2reg = *(const uint32_t*)(bs2p + (int64_t)(c >> 1) * BS::kRunS2);
    }
    if constexpr (hi_bytes_per_block(FMT) > 0) {
#pragma unroll
      for (int h = 0; h < kHD; ++h) hreg[h] = *(const uint32_t*)(bhp[h] + (int64_t)c * BS::kRunH);
    }
  };

  // ---- this wave's 4 n-fragments: local row group and column validity
  int fg[4];
  bool fcol[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    int col0;
    if (GATED) {
      col0 = n0 + 32 * wn + 16 * (f & 1);
      fg[f] = (f < 2 ? 0 : NG / 2) + 2 * wn + (f & 1);
    } else {
      col0 = n0 + 64 * wn + 16 * f;
      fg[f] = 4 * wn + f;
    }
    fcol[f] = col0 < N;
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Q8_0, Q4_K, Q5_K: the fp32 products of one 16-row fragment are scaled into the
  // accumulators while the next fragment's MFMAs run; pend_* carry them one fragment,
  // across blocks and steps (zero scales: a no-op before the first block)
  constexpr bool kPend = FMT == kQ8_0 || FMT == kQ4_K || FMT == kQ5_K;
  f32x4 pend_t[4], pend_s = f32x4{0.f, 0.f, 0.f, 0.f};
  float pend_a[4], pend_c[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    pend_t[f] = f32x4{0.f, 0.f, 0.f, 0.f};
    pend_a[f] = 0.f;
    pend_c[f] = 0.f;
  }
  // acc[mf] += the pending products (a P - c S for the k-quants, d P for Q8_0)
  auto apply_pending = [&](f32x4* accf) {
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float r = fmaf(pend_a[f], pend_t[f][v], accf[f][v]);
        accf[f][v] = FMT == kQ8_0 ? r : fmaf(-pend_c[f], pend_s[v], r);
      }
  };
  constexpr int kPrev[4] = {3, 0, 1, 2};   // the fragment before mf (3: previous block)

  // 16-row fragments of this wave's half of the tile that hold at least one bucket row
  // (wave-uniform; the tile's last rows repeat its last pair and are never stored)
  const int nmf = min(4, max(0, (mend - (m0 + 64 * wm) + 15) >> 4));
  load_a(0);
  load_b(0);
  const int g4 = lane >> 4;
  const int mrow = lane & 15;
  for (int c = 0; c < nsteps; ++c) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < RPT; ++j)
      *(u32x4*)(lds_a + (rbase + 16 * j) * kLdsStride + piece * 16) = areg[j];
    if constexpr (FMT == kQ8_0) {   // 16 int8 codes -> 16 bf16 (exact), 32 bytes
#pragma unroll
      for (int p = 0; p < BS::kQPieces; ++p) {
        uint8_t* dst = lds_bq + (threadIdx.x + kTThreads * p) * 32;
        *(bf16x8*)dst = i8x8_to_bf16x8(breg[p][0], breg[p][1]);
        *(bf16x8*)(dst + 16) = i8x8_to_bf16x8(breg[p][2], breg[p][3]);
      }
    } else {
#pragma unroll
      for (int p = 0; p < BS::kQPieces; ++p)
        *(u32x4*)(lds_bq + (threadIdx.x + kTThreads * p) * 16) = breg[p];
    }
    if (s_thread) *(uint32_t*)(lds_bs + threadIdx.x * 4) = sreg;
    if constexpr (kquant(FMT))
      if (s2_thread) *(uint32_t*)(lds_bs2 + threadIdx.x * 4) = s2reg;
    if constexpr (hi_bytes_per_block(FMT) > 0) {
#pragma unroll
      for (int h = 0; h < kHD; ++h) *(uint32_t*)(lds_bh + (threadIdx.x + kTThreads * h) * 4) = hreg[h];
    }
    __syncthreads();
    if (c + 1 < nsteps) {
      load_a(c + 1);
      load_b(c + 1);
    }
    if constexpr (kquant(FMT)) {
      // one MFMA per 32-wide block, as for Q8_0: lane supplies K = 32 j + 8 g .. + 7 of block
      // j, i.e. bytes 4 g .. 4 g + 3 of unit 16 j + lane%16, widened to bf16 q (exact). A
      // fifth MFMA against ones gives each row's block sum S, and the block adds a P - c S
      // with a = d sc, c = dmin m of the lane's column (one fragment later, as for Q8_0).
      const bf16x8 ones = __builtin_bit_cast(
          bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll 1
      for (int j = 0; j < 4; ++j) {
        bf16x8 bv[4], bvh[4];
        float sa[4], sbias[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int unit = 16 * j + mrow;
          const uint32_t q = *(const uint32_t*)(lds_bq + fg[f] * BS::kRunQ + unit * 16 + 4 * g4);
          bv[f] = u4x8_split_to_bf16x8(q);
          if constexpr (FMT == kQ5_K) {
            // 16 x the high bits of the same 8 elements (bytes 0/1 -> E4M3 0 / 2^-9, x 2^13)
            const uint32_t hw = *(const uint32_t*)(lds_bh + fg[f] * BS::kRunH + unit * 4);
            const uint32_t lo = (hw >> (2 * g4)) & 0x01010101u, hi = (hw >> (2 * g4 + 1)) & 0x01010101u;
            const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 8192.0f, false);
            const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 8192.0f, true);
            const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 8192.0f, false);
            const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 8192.0f, true);
            bvh[f] = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
          }
          const uint32_t keep = (fcol[f] && 4 * c + j < nb) ? 0xffffu : 0u;
          const uint32_t rec = *(const uint16_t*)(lds_bs + fg[f] * BS::kRunS + unit * 2) & keep;
          const uint32_t dd = *(const uint32_t*)(lds_bs2 + fg[f] * BS::kRunS2 + mrow * 4);
          const float a = fp16_to_f32((uint16_t)dd) * (float)(rec & 0xFFu);
          const float cm = fp16_to_f32((uint16_t)(dd >> 16)) * (float)(rec >> 8);
          sa[f] = a;
          sbias[f] = cm;
        }
#pragma unroll
        for (int mf = 0; mf < 4; ++mf) {
          const int row = 64 * wm + 16 * mf + mrow;
          const bf16x8 av =
              __builtin_bit_cast(bf16x8, *(const u32x4*)(lds_a + row * kLdsStride + (32 * j + 8 * g4) * 2));
          const f32x4 sx =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, ones, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          f32x4 t[4];
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            t[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[f], f32x4{0.f, 0.f, 0.f, 0.f}, 0,
                                                           0, 0);
            if constexpr (FMT == kQ5_K)
              t[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bvh[f], t[f], 0, 0, 0);
          }
          apply_pending(acc[kPrev[mf]]);
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            pend_t[f] = t[f];
            pend_a[f] = sa[f];
            pend_c[f] = sbias[f];
          }
          pend_s = sx;
          __builtin_amdgcn_sched_barrier(0);   // keep at most 10 products live
        }
      }
    } else {
      // one MFMA per 32-wide block; lane supplies K = 32 j + 8 g .. + 7 of block j, i.e.
      // codes 8 g .. of unit 16 j + lane%16 of its row group's run (staged as bf16); the
      // block scale d multiplies the fp32 products one fragment later.
#pragma unroll 1
      for (int j = 0; j < 4; ++j) {
        bf16x8 bv[4];
        float ds[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int unit = 16 * j + mrow;
          bv[f] = *(const bf16x8*)(lds_bq + (fg[f] * BS::kRunQ + unit * 32 + 8 * g4) * 2);
          const uint32_t db = *(const uint16_t*)(lds_bs + fg[f] * BS::kRunS + unit * 2);
          const uint32_t keep = (fcol[f] && 4 * c + j < nb) ? 0xffffu : 0u;
          ds[f] = fp16_to_f32((uint16_t)(db & keep));   // fp16 +0 when masked
        }
#pragma unroll
        for (int mf = 0; mf < 4; ++mf) {
          const int row = 64 * wm + 16 * mf + mrow;
          const bf16x8 av =
              __builtin_bit_cast(bf16x8, *(const u32x4*)(lds_a + row * kLdsStride + (32 * j + 8 * g4) * 2));
          f32x4 t[4];
#pragma unroll
          for (int f = 0; f < 4; ++f)
            t[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[f], f32x4{0.f, 0.f, 0.f, 0.f}, 0,
                                                           0, 0);
          apply_pending(acc[kPrev[mf]]);
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            pend_t[f] = t[f];
            pend_a[f] = ds[f];
          }
          __builtin_amdgcn_sched_barrier(0);   // keep at most 8 products live
        }
      }
    }
  }
  if constexpr (kPend) apply_pending(acc[3]);   // the last fragment's products

  // ---- epilogue: lane holds D[row 4*(lane/16) + v][col lane%16] of each 16x16 tile
  const int g = g4;
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
          if (n < N) __builtin_nontemporal_store(acc[mf][f][v], &y_out[(int64_t)pos * N + n]);
        }
      }
    }
  }
}

// Q6_K: the two exact bf16 operands of 8 weights' integer parts v = sc * (q - 32), sc the
// half block's int8 scale (|v| <= 4096, at most 14 bits). With w = v - 128:
//   hi = w with its low 7 bits cleared: a multiple of 128 within [-4224, 3968], at most 6
//        significant bits, and
//   lo = the bf16 of exponent 7 and mantissa w & 127, i.e. 128 + (w & 127),
// so hi + lo = v exactly and two MFMAs against the same A give sum x v. qd: one code dword
// (low nibbles of elements 0..3 in its bytes, high nibbles elements 4..7); hw >> sh and
// hw >> (sh + 2): the elements' 2-bit high parts as bytes (the pool's high-part layout).
__device__ __forceinline__ void q6k_parts(uint32_t qd, uint32_t hw, int sh, int sc, bf16x8& bhi,
                                          bf16x8& blo) {
  const uint32_t qa = (qd & 0x0F0F0F0Fu) | (((hw >> sh) & 0x03030303u) << 4);
  const uint32_t qb = ((qd >> 4) & 0x0F0F0F0Fu) | (((hw >> (sh + 2)) & 0x03030303u) << 4);
  const uint32_t scp = ((uint32_t)sc & 0xFFFFu) * 0x00010001u;
  const uint32_t cp = ((uint32_t)(-32 * sc - 128) & 0xFFFFu) * 0x00010001u;
  u32x4 hi, lo;
#pragma unroll
  for (int pr = 0; pr < 4; ++pr) {
    // elements 2 pr, 2 pr + 1 as two 16-bit lanes, then w = sc q - 32 sc - 128 per lane
    const uint32_t qq = __builtin_amdgcn_perm(0u, pr < 2 ? qa : qb, (pr & 1) ? 0x0c030c02u : 0x0c010c00u);
    const i16x2 wv = __builtin_bit_cast(i16x2, qq) * __builtin_bit_cast(i16x2, scp) +
                     __builtin_bit_cast(i16x2, cp);
    const uint32_t w = __builtin_bit_cast(uint32_t, wv);
    lo[pr] = (w & 0x007F007Fu) | 0x43004300u;
    const i16x2 h = __builtin_bit_cast(i16x2, w & 0xFF80FF80u);
    const float f0 = (float)h[0], f1 = (float)h[1];
    hi[pr] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  }
  bhi = __builtin_bit_cast(bf16x8, hi);
  blo = __builtin_bit_cast(bf16x8, lo);
}

// XOR mask for the 16-byte pieces of LDS row m (0..15) of a 256-byte-row tile. Measured on
// gfx950: a 64-lane ds_read_b128 is served in four passes of 16 lanes, two per half-wave,
// split by the parity of lane bits 2, 3 and 4; a pass is conflict-free when its lanes touch
// 16 different 16-byte bank groups (address / 16 mod 16) or the same address. An MFMA operand
// read takes piece 4 g + i of row m in lane 16 g + m; with this mask (bits 0, 1 of m, then
// bit 3, then bit 2 ^ bit 3) every pass sees 16 different positions, for every i.
__device__ __forceinline__ int lds_row_swizzle(int m) {
  return (m & 3) | (((m >> 3) & 1) << 2) | ((((m >> 2) ^ (m >> 3)) & 1) << 3);
}

// Zeros that the direct-LDS kernel's loads read for A pieces past K.
__device__ __attribute__((aligned(16))) uint32_t g_zero16[4];

// Grouped GEMM (MXFP4, Q6_K) with its tiles loaded straight into LDS (gfx950
// global_load_lds_dwordx4: 64 lanes x 16 bytes land contiguously at an LDS address the wave
// names), so no register holds a staged operand; each workgroup waits for its own step's
// loads while the other workgroups on the CU run their MFMAs (three fit for MXFP4, two for
// Q6_K, whose operand building needs more registers). MXFP4: BM = 64 bucket rows x 256
// weight rows (waves 1 x 4, each a 64 x 64 block, NF = 4 n-fragments), 128 K per step: 4-bit
// B is the smallest operand per weight, so a wide tile cuts the A (activation) bytes each
// CU pulls in per flop. Q6_K: BM = 128 x 128 (each wave 128 x 32, NF = 2), so each pair of
// exact operands it builds (about 40 VALU per fragment and slice) feeds 16 MFMAs.
//   A: row r of the tile at r * 256 bytes, its 16-byte piece c (8 K) at position
//      c ^ lds_row_swizzle(r % 16), which keeps every 128-bit operand read free of bank
//      conflicts. A lane's load picks the global piece whose position is its lane slot;
//      pieces past K read zeros.
//   B: the step's run of each of the 4 NF row groups (64 units of 16 bytes, 1 KiB) verbatim,
//      and likewise the runs' scales (MXFP4: one byte a unit), or their 2-bit high parts,
//      scale records and d records (Q6_K). A lane reads its whole unit at once (consecutive
//      16-byte reads: no bank conflicts); MXFP4 widens one 32-K slice at a time, Q6_K builds
//      the slice's two exact operands (q6k_parts).
template <int FMT, bool GATED, int BM, int NF>
__global__ __launch_bounds__(kTThreads, FMT == kQ6_K ? 2 : 3) void k_ggemm_mx(
    const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as, int64_t qslot,
    int64_t sslot, const uint8_t* __restrict__ bq, const uint8_t* __restrict__ bs,
    const int32_t* __restrict__ slot_map, int n_slots, int E,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm, int k,
    const uint16_t* __restrict__ src, int K, int N, int n_mtiles, int n_ntiles,
    uint16_t* __restrict__ h_out, float* __restrict__ y_out, uint32_t* __restrict__ err_flags) {
  static_assert(FMT == kMXFP4 || FMT == kQ6_K, "MXFP4 or Q6_K");
  static_assert(BM == 64 || BM == 128, "64 or 128 bucket rows");
  static_assert(NF == 4 || (NF == 2 && FMT == kQ6_K), "n-fragments per wave");
  constexpr bool kQ6 = FMT == kQ6_K;
  constexpr int NG = 4 * NF;       // B row groups per tile: each wave loads NF of them
  constexpr int TN = GATED ? NG / 2 * 16 : NG * 16;   // tile columns (gate/up: of each matrix)
  constexpr int MF = BM / 16;      // row fragments per wave (every wave covers all BM rows)
  constexpr int RW = BM / 4;       // tile rows each wave loads, 4 per load
  constexpr int NA = RW / 4;       // A loads per wave per step
  typedef __attribute__((address_space(3))) void* lds_ptr;
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[BM * 256];
  __shared__ __attribute__((aligned(16))) uint8_t lds_bq[NG * 1024];
  // per run: MXFP4's 64 E8M0 bytes; Q6_K's 64 records of two int8 half-block scales
  __shared__ __attribute__((aligned(16))) uint8_t lds_bs[NG * (kQ6 ? 128 : 64)];
  // Q6_K: the runs' 2-bit high parts (8 bytes per unit), and each group's 16 rows' d records
  // of the step's super-block (a 256-byte region per loading wave, NF groups of 64 bytes used)
  __shared__ __attribute__((aligned(16))) uint8_t lds_bh[kQ6 ? NG * 512 : 16];
  __shared__ __attribute__((aligned(16))) uint8_t lds_bd[kQ6 ? 4 * 256 : 16];
  __shared__ int tmp4[4];
  __shared__ int sh[2];
  const int lane = threadIdx.x & (kWave - 1);
  const int wn = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // waves along the columns
  // XCD-aware 2-D tile order, as k_ggemm
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int64_t i = (int64_t)(local >> 6) * 512 + xcd * 64 + (local & 63);
  if (i >= (int64_t)n_mtiles * n_ntiles) return;
  const int sr = (int)(i / (8LL * n_ntiles));
  const int hh = min(8, n_mtiles - 8 * sr);
  const int jj = (int)(i - 8LL * n_ntiles * sr);
  const int gcol = jj / (8 * hh);
  const int w = min(8, n_ntiles - 8 * gcol);
  const int kk0 = jj - 8 * hh * gcol;
  const int mt = 8 * sr + kk0 / w;
  const int nt = 8 * gcol + kk0 % w;
  int e, m0;
  if (!map_row_tile(offsets, E, BM, mt, &e, &m0, tmp4, sh)) return;
  const int mend = offsets[e + 1];
  const int slot = slot_map[e];
  const int n0 = nt * TN;
  if (slot < 0 || slot >= n_slots) {
    const int ncols = TN;
    for (int t = threadIdx.x; t < BM * ncols; t += kTThreads) {
      const int pos = m0 + t / ncols, n = n0 + t % ncols;
      if (pos < mend && n < N) {
        if (GATED) h_out[(int64_t)pos * N + n] = 0;
        else y_out[(int64_t)pos * N + n] = 0.f;
      }
    }
    if (threadIdx.x == 0 && err_flags && slot != kSlotMiss) atomicOr(err_flags, 1u);
    return;
  }
  const int nb = K / 32;
  const int nsteps = (K + kBK - 1) / kBK;

  // ---- A: wave wn loads rows RW wn + 4 j + lane / 16 (j < NA), position lane % 16
  const u32x4* src16 = (const u32x4*)src;
  const uint32_t kp = (uint32_t)K / 8;     // 16-byte units per row
  const int apos = lane & 15;
  uint32_t arow[NA];                       // unit index of each row's start
  int aswz[NA];                            // the global piece that lands at position apos
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int r = RW * wn + 4 * j + (lane >> 4);
    const int pos = min(m0 + r, mend - 1);   // rows past the tile's end repeat its last row
    const int row = GATED ? perm[pos] / k : pos;
    arow[j] = (uint32_t)row * kp;
    aswz[j] = apos ^ lds_row_swizzle(r & 15);
  }
  // ---- B: wave wn copies the runs of local row groups NF wn .. NF wn + NF - 1. GATED:
  // groups g < NG/2 are gate rows n0/16 + g, g >= NG/2 up rows n0/16 + g - NG/2; a group
  // past N reads group 0 (never stored).
  constexpr int NGH = NG / 2;
  const uint8_t* q0 = aq + (int64_t)slot * qslot;
  const uint8_t* s0 = as + (int64_t)slot * sslot;
  const uint8_t* q1 = GATED ? bq + (int64_t)slot * qslot : q0;
  const uint8_t* s1 = GATED ? bs + (int64_t)slot * sslot : s0;
  auto group_rgc = [&](int g) {
    const int rg = GATED ? n0 / 16 + g % NGH : n0 / 16 + g;
    return rg * 16 < N ? rg : 0;
  };
  // fixed-size arrays: when load_step captured arrays sized by NF, hipcc's host pass
  // silently dropped the kernel's launch stub
  const uint8_t* brun[4];   // the first NF are used
  const uint8_t* srun;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int g = NF * wn + (j < NF ? j : 0);
    brun[j] = (GATED && g >= NGH ? q1 : q0) + (int64_t)group_rgc(g) * nb * 16 * 16;
  }
  const uint8_t* hrun[2] = {nullptr, nullptr};   // Q6_K: high parts and scale records (the
  const uint8_t* rrun[2] = {nullptr, nullptr};   // first NF / 2 are used)
  const uint8_t* drun = nullptr;   // Q6_K: d records
  if constexpr (!kQ6) {
    // scales: lane l copies dword l % 16 of run NF wn + l / 16 (NF = 4)
    const int g = NF * wn + (lane >> 4);
    srun = (GATED && g >= NGH ? s1 : s0) + (int64_t)group_rgc(g) * nb * 16 + (lane & 15) * 4;
  } else {
    srun = nullptr;
    // high parts: load h copies the runs of groups NF wn + 2 h (lanes 0..31) and
    // NF wn + 2 h + 1 (lanes 32..63), 16 bytes a lane; scale records likewise, 4 bytes a
    // lane; d records: lane l copies row l % 16 of group NF wn + min(l / 16, NF - 1) into
    // the wave's 256-byte region (lanes past the wave's groups fill its spare bytes)
#pragma unroll
    for (int h = 0; h < NF / 2; ++h) {
      const int g = NF * wn + 2 * h + (lane >> 5);
      const int64_t u0 = (int64_t)group_rgc(g) * nb * 16;   // first unit of the group
      hrun[h] = (GATED && g >= NGH ? q1 : q0) + hi_region(N, K) + u0 * 8 + (lane & 31) * 16;
      rrun[h] = (GATED && g >= NGH ? s1 : s0) + u0 * 2 + (lane & 31) * 4;
    }
    const int g = NF * wn + min(lane >> 4, NF - 1);
    const int nsb = nb / kSuperBlocks;
    drun = (GATED && g >= NGH ? s1 : s0) + super_region(N, K) +
           ((int64_t)group_rgc(g) * nsb * kRowGroup + (lane & 15)) * kSuperBytes;
  }
  const int ublk = lane >> 4;   // block (of the step's 4) of the lane's B unit
  auto load_step = [&](int c) {
    const int kk = c * kBK;
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const bool ok = kk + aswz[j] * 8 < K;
      const void* gp = ok ? (const void*)(src16 + arow[j] + (uint32_t)(kk / 8 + aswz[j]))
                          : (const void*)g_zero16;
      __builtin_amdgcn_global_load_lds(gp, (lds_ptr)(lds_a + (RW * wn + 4 * j) * 256), 16, 0, 0);
    }
    // B: blocks past the row re-read step 0 (their scales are masked when consumed)
    const int cs = 4 * c + ublk < nb ? c : 0;
#pragma unroll
    for (int j = 0; j < NF; ++j)
      __builtin_amdgcn_global_load_lds(brun[j] + (int64_t)cs * 1024 + lane * 16,
                                       (lds_ptr)(lds_bq + (NF * wn + j) * 1024), 16, 0, 0);
    if constexpr (!kQ6) {
      const int css = 4 * c + (lane & 15) / 4 < nb ? c : 0;
      __builtin_amdgcn_global_load_lds(srun + (int64_t)css * 64, (lds_ptr)(lds_bs + 256 * wn), 4, 0, 0);
    } else {
      // K is a whole number of 256-element super-blocks: every step is in range
#pragma unroll
      for (int h = 0; h < NF / 2; ++h) {
        __builtin_amdgcn_global_load_lds(hrun[h] + (int64_t)c * 512,
                                         (lds_ptr)(lds_bh + (NF * wn + 2 * h) * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(rrun[h] + (int64_t)c * 128,
                                         (lds_ptr)(lds_bs + (NF * wn + 2 * h) * 128), 4, 0, 0);
      }
      __builtin_amdgcn_global_load_lds(drun + (int64_t)(c >> 1) * kRowGroup * kSuperBytes,
                                       (lds_ptr)(lds_bd + 256 * wn), 4, 0, 0);
    }
  };

  // ---- this wave's NF n-fragments: local row group and column validity. GATED: fragments
  // f < NF/2 are gate columns n0 + 16 (NF/2) wn + 16 f, f >= NF/2 the same up columns.
  // Every wave reads the whole A tile from LDS, so its 64-column share sets the LDS bytes
  // per flop; a lane reads its B unit whole (no bank conflicts) and widens it per slice.
  constexpr int NH = NF / 2;
  int fg[NF];
  bool fcol[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    int col0;
    if (GATED) {
      col0 = n0 + 16 * NH * wn + 16 * (f % NH);
      fg[f] = (f < NH ? 0 : NG / 2) + NH * wn + f % NH;
    } else {
      col0 = n0 + 16 * NF * wn + 16 * f;
      fg[f] = NF * wn + f;
    }
    fcol[f] = col0 < N;
  }
  f32x4 acc[MF][NF];
#pragma unroll
  for (int a = 0; a < MF; ++a)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[a][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int g4 = lane >> 4;
  const int mrow = lane & 15;
  const int rswz = lds_row_swizzle(mrow);   // rows 16 mf + mrow all have r % 16 == mrow
  for (int c = 0; c < nsteps; ++c) {
    __syncthreads();   // every wave is done reading the previous step
    load_step(c);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();   // every wave's loads have landed
    // all MF row fragments run: rows past the expert's last pair repeat it and are never stored
    auto read_a = [&](int mf, int ii) {
      const int row = 16 * mf + mrow;
      return __builtin_bit_cast(bf16x8, *(const u32x4*)(lds_a + row * 256 + ((4 * g4 + ii) ^ rswz) * 16));
    };
    if constexpr (!kQ6) {
      u32x4 bq4[NF];
      float bsc[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        bq4[f] = *(const u32x4*)(lds_bq + fg[f] * 1024 + lane * 16);
        const uint32_t sb = lds_bs[fg[f] * 64 + lane];
        const uint32_t keep = (fcol[f] && 4 * c + g4 < nb) ? 0xffffffffu : 0u;
        bsc[f] = __uint_as_float((sb << 23) & keep);   // E8M0 -> 2^(b-127), or +0
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        // one 32-K slice: the wave's MF A fragments are read once; each B fragment is
        // widened just before its MF MFMAs, so a single widened fragment is live at a time
        bf16x8 av[MF];
#pragma unroll
        for (int mf = 0; mf < MF; ++mf) {
          const int row = 16 * mf + mrow;
          const int piece = (4 * g4 + ii) ^ rswz;
          av[mf] = __builtin_bit_cast(bf16x8, *(const u32x4*)(lds_a + row * 256 + piece * 16));
        }
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const bf16x8 bv = fp4x8_to_bf16x8(bq4[f][ii], bsc[f]);
#pragma unroll
          for (int mf = 0; mf < MF; ++mf)
            acc[mf][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mf], bv, acc[mf][f], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the next slice's reads after these MFMAs
      }
    } else {
      // lane's unit: block 4 c + lane / 16 of row lane % 16; slice ii is its code dword ii
      // (elements 8 ii .. 8 ii + 7, half ii / 2). Per fragment the step's 4 slices go into one
      // accumulator, two MFMAs each, and the step adds d t (d is the super-block's).
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const u32x4 q4 = *(const u32x4*)(lds_bq + fg[f] * 1024 + lane * 16);
        const u32x2 h2 = *(const u32x2*)(lds_bh + fg[f] * 512 + lane * 8);
        const uint32_t rec = *(const uint16_t*)(lds_bs + fg[f] * 128 + lane * 2);
        const uint8_t* drec = lds_bd + (fg[f] / NF) * 256 + (fg[f] % NF) * 64 + mrow * 4;
        const float d = fcol[f] ? fp16_to_f32(*(const uint16_t*)drec) : 0.f;
        f32x4 t[MF];
#pragma unroll
        for (int mf = 0; mf < MF; ++mf) t[mf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          // per group of 4 row fragments: the A reads first (the first group's latency hides
          // behind building the operands), then their hi MFMAs and their lo ones, so no MFMA
          // waits on the one before and only 4 A fragments are live
          bf16x8 bhi, blo;
#pragma unroll
          for (int mg = 0; mg < MF; mg += 4) {
            bf16x8 av[4];
#pragma unroll
            for (int mf = 0; mf < 4; ++mf) av[mf] = read_a(mg + mf, ii);
            if (mg == 0)
              q6k_parts(q4[ii], h2[ii >> 1], 4 * (ii & 1), (int)(int8_t)(rec >> (8 * (ii >> 1))),
                        bhi, blo);
#pragma unroll
            for (int mf = 0; mf < 4; ++mf)
              t[mg + mf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mf], bhi, t[mg + mf], 0, 0, 0);
#pragma unroll
            for (int mf = 0; mf < 4; ++mf)
              t[mg + mf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mf], blo, t[mg + mf], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);   // one slice's operands live at a time
        }
#pragma unroll
        for (int mf = 0; mf < MF; ++mf)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[mf][f][v] = fmaf(d, t[mf][v], acc[mf][f][v]);
      }
    }
  }
  // ---- epilogue: lane holds D[row 4*(lane/16) + v][col lane%16] of each 16x16 tile
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int pos = m0 + 16 * mf + 4 * g4 + v;
      if (pos >= mend) continue;
      if constexpr (GATED) {
#pragma unroll
        for (int f = 0; f < NH; ++f) {
          const int n = n0 + 16 * NH * wn + 16 * f + mrow;
          if (n < N)
            h_out[(int64_t)pos * N + n] = f32_to_bf16_rne(silu_mul(acc[mf][f][v], acc[mf][f + NH][v]));
        }
      } else {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int n = n0 + 16 * NF * wn + 16 * f + mrow;
          if (n < N) __builtin_nontemporal_store(acc[mf][f][v], &y_out[(int64_t)pos * N + n]);
        }
      }
    }
  }
}

// MXFP4: 64 rows x 256 weight rows; Q6_K: 128 x 128, so each operand it builds feeds
// twice the MFMAs
constexpr int mx_rows(int fmt) { return fmt == kQ6_K ? 128 : 64; }
constexpr int mx_nfrag(int fmt) { return fmt == kQ6_K ? 2 : 4; }

template <int FMT, bool GATED>
hipError_t launch_ggemm_mx(const PoolView& a, const PoolView& b, const int32_t* slot_map,
                           int n_slots, int E, const int32_t* offsets, const int32_t* perm,
                           int T, int k, const uint16_t* src, int K, int N, uint16_t* h,
                           float* y, uint32_t* err, hipStream_t stream) {
  constexpr int BM = mx_rows(FMT);
  constexpr int TN = GATED ? 2 * mx_nfrag(FMT) * 16 : 4 * mx_nfrag(FMT) * 16;   // tile columns
  const int pairs = T * k;
  const int max_mtiles = (pairs + BM - 1) / BM + min(E, pairs);
  const int n_ntiles = (N + TN - 1) / TN;
  const int64_t grid = ((int64_t)max_mtiles * n_ntiles + 511) / 512 * 512;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  if constexpr (FMT == kQ6_K)
    hipLaunchKernelGGL((k_ggemm_mx<FMT, GATED, 128, 2>), dim3((unsigned)grid), dim3(kTThreads), 0,
                       stream,
                       a.q, a.s, a.q_slot, a.s_slot, b.q, b.s, slot_map, n_slots, E, offsets, perm,
                       k, src, K, N, max_mtiles, n_ntiles, h, y, err);
  else
    hipLaunchKernelGGL((k_ggemm_mx<FMT, GATED, 64, 4>), dim3((unsigned)grid), dim3(kTThreads), 0,
                       stream,
                       a.q, a.s, a.q_slot, a.s_slot, b.q, b.s, slot_map, n_slots, E, offsets, perm,
                       k, src, K, N, max_mtiles, n_ntiles, h, y, err);
  return hipGetLastError();
}

template <int FMT, bool GATED>
hipError_t launch_ggemm_t(const PoolView& a, const PoolView& b, const int32_t* slot_map,
                          int n_slots, int E, const int32_t* offsets, const int32_t* perm,
                          int T, int k, const uint16_t* src, int K, int N, uint16_t* h,
                          float* y, uint32_t* err, hipStream_t stream) {
  constexpr int BM = 128;
  const int pairs = T * k;
  const int max_mtiles = (pairs + BM - 1) / BM + min(E, pairs);
  constexpr int kCols = GATED ? 64 : 128;   // columns per tile (gate/up: of each matrix)
  const int n_ntiles = (N + kCols - 1) / kCols;
  const int64_t grid = ((int64_t)max_mtiles * n_ntiles + 511) / 512 * 512;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_ggemm<FMT, GATED>), dim3((unsigned)grid), dim3(kTThreads), 0, stream,
                     a.q, a.s, a.q_slot, a.s_slot, b.q, b.s, slot_map, n_slots, E, offsets, perm,
                     k, src, K, N, max_mtiles, n_ntiles, h, y, err);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_grouped(int fmt, const PoolView& gate, const PoolView& up,
                                  const int32_t* slot_map, int n_slots, int E, const uint16_t* x,
                                  int T, int k, int H, int I, const int32_t* offsets,
                                  const int32_t* perm, uint16_t* h, uint32_t* err,
                                  hipStream_t stream) {
  switch (fmt) {
    case kMXFP4:
      return launch_ggemm_mx<kMXFP4, true>(gate, up, slot_map, n_slots, E, offsets, perm, T, k, x, H, I,
                                   h, nullptr, err, stream);
    case kQ8_0:
      return launch_ggemm_t<kQ8_0, true>(gate, up, slot_map, n_slots, E, offsets, perm, T, k, x,
                                         H, I, h, nullptr, err, stream);
    case kQ4_K:
      return launch_ggemm_t<kQ4_K, true>(gate, up, slot_map, n_slots, E, offsets, perm, T, k, x,
                                         H, I, h, nullptr, err, stream);
    case kQ5_K:
      return launch_ggemm_t<kQ5_K, true>(gate, up, slot_map, n_slots, E, offsets, perm, T, k, x,
                                         H, I, h, nullptr, err, stream);
    case kQ6_K:
      return launch_ggemm_mx<kQ6_K, true>(gate, up, slot_map, n_slots, E, offsets, perm, T, k, x,
                                          H, I, h, nullptr, err, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_down_grouped(int fmt, const PoolView& down, const int32_t* slot_map,
                               int n_slots, int E, int T, int k, int H, int I,
                               const int32_t* offsets, const uint16_t* h, float* y,
                               uint32_t* err, hipStream_t stream) {
  switch (fmt) {
    case kMXFP4:
      return launch_ggemm_mx<kMXFP4, false>(down, down, slot_map, n_slots, E, offsets, nullptr, T, k, h,
                                    I, H, nullptr, y, err, stream);
    case kQ8_0:
      return launch_ggemm_t<kQ8_0, false>(down, down, slot_map, n_slots, E, offsets, nullptr, T,
                                          k, h, I, H, nullptr, y, err, stream);
    case kQ4_K:
      return launch_ggemm_t<kQ4_K, false>(down, down, slot_map, n_slots, E, offsets, nullptr, T,
                                          k, h, I, H, nullptr, y, err, stream);
    case kQ5_K:
      return launch_ggemm_t<kQ5_K, false>(down, down, slot_map, n_slots, E, offsets, nullptr, T,
                                          k, h, I, H, nullptr, y, err, stream);
    case kQ6_K:
      return launch_ggemm_mx<kQ6_K, false>(down, down, slot_map, n_slots, E, offsets, nullptr, T,
                                           k, h, I, H, nullptr, y, err, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
