// Weighted merge of each token's k expert outputs: the "merges the weighted outputs" step
// of the llama.cpp discussion's original post.
//   out[t, :] = sum_{j<k} w[t, j] * y[inv_perm[t*k + j], :]   (fp32, increasing j)
// Pure streaming: each thread owns 4 consecutive columns of one token and reads the k
// source rows with 16-byte loads.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y,
                                                 const int32_t* __restrict__ inv_perm,
                                                 const float* __restrict__ w, int T, int k,
                                                 int H, float* __restrict__ out) {
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= H) return;
  for (int t = blockIdx.y; t < T; t += gridDim.y) {   // grid.y is capped at kMaxGridY
    // every load is issued before the first one is consumed (k <= kMaxK)
    int pos[kMaxK];
    float wj[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      const int jj = j < k ? j : 0;
      pos[j] = inv_perm[(int64_t)t * k + jj];
      wj[j] = w[(int64_t)t * k + jj];
    }
    f32x4 v[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)   // y is read once: nontemporal
      v[j] = __builtin_nontemporal_load((const f32x4*)(y + (int64_t)pos[j] * H + c));
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k) {
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = fmaf(wj[j], v[j][q], acc[q]);
      }
    *(f32x4*)(out + (int64_t)t * H + c) = acc;
  }
}

}  // namespace

hipError_t launch_combine(const float* y, const int32_t* inv_perm, const float* w, int T, int k,
                          int H, float* out, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  dim3 grid((H / 4 + 255) / 256, min(T, kMaxGridY));
  hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, stream, y, inv_perm, w, T, k, H, out);
  return hipGetLastError();
}

}  // namespace moe
