// Canonical row-major block planes -> the pool's tiled layout (16 rows interleaved block
// by block). This is the per-slot "mapping" a loader runs when an expert lands in the
// resident pool (tinyserve README, "How it works" item 3; llama.cpp discussion, "Formal
// gate results": mapping rewrite before the grouped matmul). Pure data movement.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

template <int FMT>
__global__ __launch_bounds__(256) void k_pack(int64_t n_units, int rows, int nb,
                                              const uint8_t* __restrict__ sq,
                                              const uint8_t* __restrict__ ss,
                                              uint8_t* __restrict__ dq, uint8_t* __restrict__ ds) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // canonical (mat, row, block)
  if (i >= n_units) return;
  const int64_t per_mat = (int64_t)rows * nb;
  const int64_t mat = i / per_mat;
  const int64_t rem = i % per_mat;
  const int r = (int)(rem / nb), b = (int)(rem % nb);
  const int64_t u = mat * per_mat + pool_unit(r, b, nb);
  if constexpr (FMT == kMXFP4) {
    *(u32x4*)(dq + u * 16) = *(const u32x4*)(sq + i * 16);
    ds[u] = ss[i];
  } else if constexpr (kquant(FMT)) {
    // codes: canonical element 2j / 2j+1 in byte j's low / high nibble -> the pool's split
    // order, in each dword (8 elements) byte j holding element j (low) and j + 4 (high)
    const int64_t K = 32 * (int64_t)nb;
    const int64_t crow = (int64_t)nb * (16 + hi_bytes_per_block(FMT));   // canonical row bytes
    const uint8_t* scrow = sq + (mat * rows + r) * crow;
    uint8_t* dqmat = dq + mat * code_plane_bytes(FMT, rows, K);
    const int64_t um = pool_unit(r, b, nb);                               // unit in the matrix
    const u32x4 cw = *(const u32x4*)(scrow + 16 * (int64_t)b);
    u32x4 pw;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t e[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) e[t] = (cw[d] >> (4 * t)) & 0xFu;   // element t of the dword
      uint32_t o = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) o |= (e[j] | (e[j + 4] << 4)) << (8 * j);
      pw[d] = o;
    }
    *(u32x4*)(dqmat + um * 16) = pw;
    if constexpr (FMT == kQ5_K) {
      // canonical high bits of the block (bit e = element e) -> the pool's dword, whose bit
      // 8j + s is element 8 (s / 2) + j + 4 (s % 2)
      const uint8_t* hb = scrow + 16 * (int64_t)nb + 4 * (int64_t)b;
      const uint32_t h32 = (uint32_t)hb[0] | ((uint32_t)hb[1] << 8) | ((uint32_t)hb[2] << 16) |
                           ((uint32_t)hb[3] << 24);
      uint32_t g = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int sh = 0; sh < 8; ++sh)
          g |= ((h32 >> (8 * (sh >> 1) + j + 4 * (sh & 1))) & 1u) << (8 * j + sh);
      *(uint32_t*)(dqmat + hi_region(rows, K) + um * 4) = g;
    }
    if constexpr (FMT == kQ6_K) {
      // canonical 2-bit high parts of the block (bits 2e, 2e+1 = element e) -> the pool's
      // two dwords: dword g, bits 8j + s + t (s even) = bit t of element
      // 8 (2g + s / 4) + j + 4 ((s / 2) % 2)
      const uint8_t* hb = scrow + 16 * (int64_t)nb + 8 * (int64_t)b;
      uint64_t h64 = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) h64 |= (uint64_t)hb[j] << (8 * j);
      uint32_t g2[2] = {0u, 0u};
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int sh = 0; sh < 8; sh += 2) {
            const int e = 8 * (2 * g + sh / 4) + j + 4 * ((sh / 2) % 2);
            g2[g] |= (uint32_t)((h64 >> (2 * e)) & 3u) << (8 * j + sh);
          }
      *(u32x2*)(dqmat + hi_region(rows, K) + um * 8) = u32x2{g2[0], g2[1]};
    }
    // canonical scale row: Q4_K / Q5_K (sc, m) per block, then (d, dmin) fp16 per
    // super-block; Q6_K the two int8 sub-block scales per block, then fp16 d per super-block
    const int nsb = nb / kSuperBlocks;
    const int64_t srow_sup = FMT == kQ6_K ? 2 : kSuperBytes;     // canonical bytes per super-block
    const int64_t row_bytes = 2 * (int64_t)nb + srow_sup * nsb;
    const uint8_t* srow = ss + (mat * rows + r) * row_bytes;
    uint8_t* dmat = ds + mat * scale_plane_bytes(FMT, rows, K);
    dmat[um * 2 + 0] = srow[2 * b + 0];
    dmat[um * 2 + 1] = srow[2 * b + 1];
    if (b % kSuperBlocks == 0) {
      const int sblk = b / kSuperBlocks;
      const int64_t rec = ((int64_t)(r >> 4) * nsb + sblk) * kRowGroup + (r & 15);
      uint8_t* dst = dmat + super_region(rows, K) + rec * kSuperBytes;
      const uint8_t* src = srow + 2 * nb + srow_sup * sblk;
#pragma unroll
      for (int j = 0; j < kSuperBytes; ++j) dst[j] = j < srow_sup ? src[j] : 0;
    }
  } else {
    *(u32x4*)(dq + u * 32) = *(const u32x4*)(sq + i * 32);
    *(u32x4*)(dq + u * 32 + 16) = *(const u32x4*)(sq + i * 32 + 16);
    ((uint16_t*)ds)[u] = ((const uint16_t*)ss)[i];
  }
}

}  // namespace

hipError_t launch_pack(int fmt, int n_mats, int rows, int K, const void* sq, const void* ss,
                       void* dq, void* ds, hipStream_t stream) {
  const int nb = K / 32;
  const int64_t n = (int64_t)n_mats * rows * nb;
  const int64_t blocks = (n + 255) / 256;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (fmt == kMXFP4)
    hipLaunchKernelGGL(k_pack<kMXFP4>, dim3((unsigned)blocks), dim3(256), 0, stream, n, rows, nb,
                       (const uint8_t*)sq, (const uint8_t*)ss, (uint8_t*)dq, (uint8_t*)ds);
  else if (fmt == kQ4_K || fmt == kQ5_K || fmt == kQ6_K) {
    if (nb % kSuperBlocks) return hipErrorInvalidValue;
    if (fmt == kQ4_K)
      hipLaunchKernelGGL(k_pack<kQ4_K>, dim3((unsigned)blocks), dim3(256), 0, stream, n, rows,
                         nb, (const uint8_t*)sq, (const uint8_t*)ss, (uint8_t*)dq, (uint8_t*)ds);
    else if (fmt == kQ6_K)
      hipLaunchKernelGGL(k_pack<kQ6_K>, dim3((unsigned)blocks), dim3(256), 0, stream, n, rows,
                         nb, (const uint8_t*)sq, (const uint8_t*)ss, (uint8_t*)dq, (uint8_t*)ds);
    else
      hipLaunchKernelGGL(k_pack<kQ5_K>, dim3((unsigned)blocks), dim3(256), 0, stream, n, rows,
                         nb, (const uint8_t*)sq, (const uint8_t*)ss, (uint8_t*)dq, (uint8_t*)ds);
  } else
    hipLaunchKernelGGL(k_pack<kQ8_0>, dim3((unsigned)blocks), dim3(256), 0, stream, n, rows, nb,
                       (const uint8_t*)sq, (const uint8_t*)ss, (uint8_t*)dq, (uint8_t*)ds);
  return hipGetLastError();
}

}  // namespace moe
