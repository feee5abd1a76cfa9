// Device helpers shared by the layer's kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));
typedef int16_t i16x2 __attribute__((__vector_size__(2 * sizeof(int16_t))));

constexpr int kWave = 64;
constexpr int kBlock = 32;      // elements per quantization block (MXFP4 and Q8_0)
constexpr int kRowGroup = 16;   // rows interleaved per tile in the pool layout
constexpr int kMaxK = 8;        // largest supported top-k
constexpr int kMaxE = 256;      // largest supported expert count
constexpr int kMaxGridY = 65535;   // largest grid.y a launch takes

enum Fmt : int { kMXFP4 = 1, kQ8_0 = 2, kQ4_K = 3, kQ5_K = 4, kQ6_K = 5 };

// Formats whose 32-element block is a 16-byte unit of 4-bit codes (MXFP4, Q4_K, and Q5_K's
// low nibbles): a lane of a 64-lane 16-byte load holds one whole block of one row.
__host__ __device__ constexpr bool unit16(int fmt) { return fmt != kQ8_0; }
// k-quants: per-unit scale records of two bytes and one 4-byte record per (row,
// 256-element super-block). Q4_K and Q5_K: 6-bit scale and min per block, fp16 d and dmin
// per super-block. Q6_K: a signed 8-bit scale per 16-element half block, fp16 d per
// super-block (the record's high half unused).
__host__ __device__ constexpr bool kquant(int fmt) { return fmt == kQ4_K || fmt == kQ5_K || fmt == kQ6_K; }
// Block sums the k-quant kernels need per 32-element block: Q6_K's two halves have their
// own scales.
__host__ __device__ constexpr int sums_per_block(int fmt) { return fmt == kQ6_K ? 2 : 1; }

// ---------------------------------------------------------------- scalar conversions

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// fp16 bits -> fp32 (exact).
__device__ __forceinline__ float fp16_to_f32(uint16_t v) {
  return (float)__builtin_bit_cast(_Float16, v);
}

// E8M0 scale byte -> fp32 2^(b-127), exact for b in [1, 254].
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) { return __uint_as_float(b << 23); }

// Two E2M1 codes in byte `sel` of `src` -> two bf16 values times `scale` (a power of two):
// element 0 from the low nibble, element 1 from the high nibble. One gfx950 instruction.
template <int sel>
__device__ __forceinline__ bf16x2 fp4x2_to_bf16x2(uint32_t src, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, scale, sel);
}

// 8 E2M1 codes (one dword, element 0 in the low nibble of byte 0) -> 8 bf16, scaled.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t v, float scale) {
  bf16x2 a = fp4x2_to_bf16x2<0>(v, scale);
  bf16x2 b = fp4x2_to_bf16x2<1>(v, scale);
  bf16x2 c = fp4x2_to_bf16x2<2>(v, scale);
  bf16x2 d = fp4x2_to_bf16x2<3>(v, scale);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 4 int8 codes (one dword) -> 4 fp32 (exact).
__device__ __forceinline__ void i8x4_to_f32(uint32_t v, float* o) {
  o[0] = float(int32_t(v << 24) >> 24);
  o[1] = float(int32_t(v << 16) >> 24);
  o[2] = float(int32_t(v << 8) >> 24);
  o[3] = float(int32_t(v) >> 24);
}

// 2 fp32 holding bf16-exact values -> packed bf16x2 (truncation is exact here).
__device__ __forceinline__ uint32_t pack_bf16x2_exact(float lo, float hi) {
  // one v_perm_b32: bytes 2, 3 of lo, then bytes 2, 3 of hi
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// 8 unsigned 4-bit codes in the pool's split order (byte j holds element j in its low
// nibble and element j + 4 in its high nibble) -> 4 bf16 pairs (q0,q1) (q2,q3) (q4,q5)
// (q6,q7), exact. A byte holding q in 0..15 is the FP8 E4M3 code of q * 2^-9 (subnormal for
// q < 8, exponent field 1 for q >= 8), so the gfx950 scaled FP8 -> bf16 conversion with
// scale 2^9 gives q; one conversion per pair.
__device__ __forceinline__ void u4x8_split_to_bf16(uint32_t v, bf16x2* w) {
  const uint32_t lo = v & 0x0F0F0F0Fu, hi = (v >> 4) & 0x0F0F0F0Fu;
  w[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, false);
  w[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, true);
  w[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, false);
  w[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, true);
}
__device__ __forceinline__ bf16x8 u4x8_split_to_bf16x8(uint32_t v) {
  bf16x2 w[4];
  u4x8_split_to_bf16(v, w);
  return bf16x8{w[0][0], w[0][1], w[1][0], w[1][1], w[2][0], w[2][1], w[3][0], w[3][1]};
}

// 8 int8 codes (two dwords) -> 8 bf16 (exact: |q| <= 128 has at most 8 significant bits).
__device__ __forceinline__ bf16x8 i8x8_to_bf16x8(uint32_t v0, uint32_t v1) {
  float f[8];
  i8x4_to_f32(v0, f);
  i8x4_to_f32(v1, f + 4);
  u32x4 p = {pack_bf16x2_exact(f[0], f[1]), pack_bf16x2_exact(f[2], f[3]),
             pack_bf16x2_exact(f[4], f[5]), pack_bf16x2_exact(f[6], f[7])};
  return __builtin_bit_cast(bf16x8, p);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), acc, false);
}
__device__ __forceinline__ float dot2_bf16(bf16x2 a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2, b), acc, false);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

// ------------------------------------------------------------------ wave reductions

__device__ __forceinline__ float wave_xor(float v, int mask) { return __shfl_xor(v, mask, kWave); }

// ------------------------------------------------------------------ pool layout

// Index of the 16-byte (MXFP4) / 32-byte (Q8_0) unit of row r, block b, in a matrix
// with nb blocks per row (see the tiled layout in include/moe.h).
__device__ __forceinline__ int64_t pool_unit(int r, int b, int nb) {
  return (int64_t(r >> 4) * nb + b) * kRowGroup + (r & 15);
}

__host__ __device__ constexpr int64_t code_bytes_per_block(int fmt) { return unit16(fmt) ? 16 : 32; }
// Scale bytes per unit (MXFP4: E8M0 byte; Q8_0: fp16 d; Q4_K: the block's 6-bit scale and
// min in two bytes, sc | m << 8).
__host__ __device__ constexpr int64_t scale_bytes_per_block(int fmt) { return fmt == kMXFP4 ? 1 : 2; }

// Q4_K also has per-super-block scales: after the per-unit records of a matrix (rows * nb *
// 2 bytes) come 4-byte records d | dmin << 16 (fp16 bits), one per (row, 256-element
// super-block), tiled like the units: record (r, s) at index ((r/16) * nsb + s) * 16 + r%16.
constexpr int kSuperBlocks = 8;      // 32-element blocks per Q4_K super-block
constexpr int64_t kSuperBytes = 4;   // bytes of one (d, dmin) record
__host__ __device__ constexpr int64_t scale_plane_bytes(int fmt, int64_t rows, int64_t K) {
  return rows * (K / 32) * scale_bytes_per_block(fmt) +
         (kquant(fmt) ? rows * (K / (32 * kSuperBlocks)) * kSuperBytes : 0);
}
// Q5_K's fifth code bit: after the 16-byte units of a matrix's code plane (rows * nb * 16
// bytes) comes one dword per unit, at unit index * 4. Bit 8j + s of the dword is the high
// bit of element 8 (s / 2) + j + 4 (s % 2) of the block, so that (dword >> s) & 0x01010101
// gives, as bytes, the high bits of the four elements whose low nibbles form a nibble plane
// of dword s / 2 of the unit (the low plane for even s, the high plane for odd s).
// Q6_K's 2-bit high parts: two dwords per unit at unit index * 8; dword g covers the unit's
// code dwords 2g and 2g + 1, its bits 8j + s, 8j + s + 1 holding the high part of element
// 8 (2g + s / 4) + j + 4 ((s / 2) % 2) (s even), so that (dword >> s) & 0x03030303 gives one
// nibble plane's high parts as bytes.
__host__ __device__ constexpr int64_t hi_bytes_per_block(int fmt) {
  return fmt == kQ5_K ? 4 : fmt == kQ6_K ? 8 : 0;
}
__host__ __device__ constexpr int64_t code_plane_bytes(int fmt, int64_t rows, int64_t K) {
  return rows * (K / 32) * (code_bytes_per_block(fmt) + hi_bytes_per_block(fmt));
}
__host__ __device__ constexpr int64_t hi_region(int64_t rows, int64_t K) { return rows * (K / 32) * 16; }
// Byte offset, within a matrix's scale plane, of the super-block records (Q4_K).
__host__ __device__ constexpr int64_t super_region(int64_t rows, int64_t K) {
  return rows * (K / 32) * 2;
}

// Active-expert list written by the small-batch router (see route.hip): act[0] = count,
// then kActStride int32 per active expert.
constexpr int kActStride = 8;

// slot_map value of an expert that is not in the pool (MOE_SLOT_MISS): its pairs get
// zero output and raise no error flag.
constexpr int kSlotMiss = -1;

// A split router's partial logits handed to the kernel that finishes the routing (the
// decode gate/up kernel), and where that kernel stores the routing it computes.
//   partial [ns][T][E] fp32; ids, w [T][k]; counts [E]; offsets [E+1]; perm, inv_perm [T*k];
//   act: the active-expert list (1 + kActStride * E int32).
constexpr int kMaxRouteSplit = 32;   // most splits of the router's reduction dimension
constexpr int kFuseMaxT = 4;         // most tokens a fused routing prologue handles
constexpr int kFuseMaxTE = 256;      // most (token, expert) logits it handles
constexpr int kFuseMaxPairs = kFuseMaxT * kMaxK;
constexpr int kRouteMaxH = 4096;    // largest H whose activation rows it stages whole
struct RouteIn {
  const float* partial;
  int ns;
  const float* bias;
  int T;
  int32_t* ids;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv_perm;
  int32_t* act;
  int32_t* tickets;   // the down kernel's per-row-group tickets, zeroed here (NULL: none)
  int n_tickets;
};
__host__ __device__ constexpr int act_ints(int E) { return 1 + kActStride * E; }

// The fused decode layer's down kernel combines without a separate launch: each of a row
// group's workgroups (one per active expert) stores its y rows with device-coherent
// stores, waits for them to complete and takes a ticket; the one that draws the last
// ticket reads the group's y rows back (device-coherent loads) and writes out.
struct DownTail {
  const int32_t* inv_perm;   // [T*k]
  const float* w;            // [T*k]
  float* out;                // [T][H]
  int32_t* tickets;          // [H/16], zero on entry
  int T;
};

// The fused decode layer (one persistent kernel for the routing, gate/up, down and
// combine; see gemv.hip) hands each expert's h from its gate/up workgroups to its down
// workgroups in two levels: the gate/up unit of row group rg of active expert j, once its h
// rows are stored device-coherently, adds one to counters[j][rg % kHandoffSplit]; the unit
// that completes a sub-counter (handoff_units of them) adds one to ready[j]; a down unit of
// expert j waits until ready[j] counts every sub-counter that has units. The sub-counters
// keep an expert's I/16 atomics from queueing on one address, and the waiting workgroups
// poll one word per expert, each on a cache line of its own, with a pause between polls:
// hundreds of workgroups polling every sub-counter back to back slowed the whole launch
// several times over. Every wait is bounded: after spin_limit polls it gives up and sets
// bit 1 of err_flags.
constexpr int kHandoffSplit = 8;
constexpr int kReadyStride = 32;     // int32 between two experts' ready words (128 bytes)
constexpr int kSpinLimit = 1 << 15;
constexpr int kPollSleep = 20;       // s_sleep between two polls (x 64 clocks)
struct FusedDown {
  const uint8_t* q;     // down code plane, slot 0
  const uint8_t* s;     // down scale plane, slot 0
  int64_t q_slot, s_slot;
  float* y;             // [T*k][H]
  float* out;           // [T][H]
  int32_t* counters;    // [kFuseMaxPairs][kHandoffSplit], zero on entry
  int32_t* ready;       // [kFuseMaxPairs][kReadyStride] (word 0 used), zero on entry
  int32_t* tickets;     // [H/16], zero on entry
  int spin_limit;
};
// Gate/up units of an expert counted by sub-counter q: the row groups rg < n_rg with
// rg % kHandoffSplit == q.
__host__ __device__ constexpr int handoff_units(int n_rg, int q) {
  return q < n_rg ? (n_rg - q + kHandoffSplit - 1) / kHandoffSplit : 0;
}
// int32 words of the fused layer's synchronisation region: the tickets, the sub-counters,
// then the ready words
__host__ __device__ constexpr int sync_ints(int H) {
  return H / 16 + kFuseMaxPairs * kHandoffSplit + kFuseMaxPairs * kReadyStride;
}

// s_waitcnt with only vmcnt(0): every vector memory access the wave issued has completed
// (expcnt and lgkmcnt fields at their no-wait maxima).
constexpr int kWaitVmcnt0 = 0x0F70;

struct PoolView {
  const uint8_t* q;   // code plane, slot 0
  const uint8_t* s;   // scale plane, slot 0
  int64_t q_slot;     // bytes per slot in the code plane
  int64_t s_slot;     // bytes per slot in the scale plane
};

}  // namespace moe
