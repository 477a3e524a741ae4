// RMSNorm (one wavefront per row, reduction by cross-lane shuffles), the
// embedding gather and a float copy.
//   RMSNorm: out = w * (x / sqrt(mean(x^2) + eps)) -- abi96062 components.py, RMSNorm;
//            statistics in float32, one rounding to the operand type at the output.
//   Embedding: x[m, :] = E[ids[m], :] -- abi96062 model.py, SmolLM2Model.forward.
#include "common.h"
#include "kernels.h"

namespace smol {

constexpr int NORM_ROWS = 4;  // rows (waves) per workgroup

// VPL = H / 64 values per lane when known at compile time (the row stays in
// registers and all its loads are in flight at once); VPL = 0 is the generic path.
template <typename T, typename O, int VPL>
__global__ void __launch_bounds__(64 * NORM_ROWS)
rmsnorm_kernel(const float *__restrict__ x, const T *__restrict__ w, O *__restrict__ out, int M, int H, float eps) {
  const int lane = threadIdx.x & 63;
  int row;
  if (xcd_rows(M)) {  // XCD x normalises rows of its own range (same L2 as the GEMMs)
    const int rpx = rows_per_xcd(M);
    row = (blockIdx.x % SMOL_XCDS) * rpx + (blockIdx.x / SMOL_XCDS) * NORM_ROWS + (threadIdx.x >> 6);
    if (row >= min(M, (int)(blockIdx.x % SMOL_XCDS + 1) * rpx)) return;
  } else {
    row = blockIdx.x * NORM_ROWS + (threadIdx.x >> 6);
  }
  if (row >= M) return;
  const float *xr = x + (size_t)row * H;
  O *orow = out + (size_t)row * H;
  if constexpr (VPL > 0) {
    float v[VPL], wv[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      v[j] = xr[lane + 64 * j];
      wv[j] = to_f32(w[lane + 64 * j]);
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) ss += v[j] * v[j];
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
    for (int j = 0; j < VPL; ++j) orow[lane + 64 * j] = from_f32<O>(wv[j] * (v[j] * r));
  } else {
    float ss = 0.f;
    for (int i = lane; i < H; i += 64) {
      const float v = xr[i];
      ss += v * v;
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)H + eps);
    for (int i = lane; i < H; i += 64) orow[i] = from_f32<O>(to_f32(w[i]) * (xr[i] * r));
  }
}

template <typename T>
hipError_t rmsnorm(const float *x, const T *w, Act<T> *out, int M, int H, float eps, hipStream_t s) {
  const dim3 grid(xcd_rows(M) ? SMOL_XCDS * rows_per_xcd(M) / NORM_ROWS : (M + NORM_ROWS - 1) / NORM_ROWS);
  const dim3 block(64 * NORM_ROWS);
  switch (H) {
    case 576: hipLaunchKernelGGL((rmsnorm_kernel<T, Act<T>, 9>), grid, block, 0, s, x, w, out, M, H, eps); break;
    case 2048: hipLaunchKernelGGL((rmsnorm_kernel<T, Act<T>, 32>), grid, block, 0, s, x, w, out, M, H, eps); break;
    default: hipLaunchKernelGGL((rmsnorm_kernel<T, Act<T>, 0>), grid, block, 0, s, x, w, out, M, H, eps); break;
  }
  return hipGetLastError();
}

template <typename T>
__global__ void __launch_bounds__(256)
embed_kernel(const int32_t *__restrict__ ids, const T *__restrict__ E, float *__restrict__ x, int M, int H, int V) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const int id = ids[row];
  float *xr = x + (size_t)row * H;
  if (id < 0 || id >= V) {
    for (int i = lane; i < H; i += 64) xr[i] = __builtin_nanf("");
    return;
  }
  const T *er = E + (size_t)id * H;
#pragma unroll 8
  for (int i = lane; i < H; i += 64) xr[i] = to_f32(er[i]);
}

template <typename T>
hipError_t embed_rows(const int32_t *ids, const T *E, float *x, int M, int H, int V, hipStream_t s) {
  hipLaunchKernelGGL((embed_kernel<T>), dim3((M + 3) / 4), dim3(256), 0, s, ids, E, x, M, H, V);
  return hipGetLastError();
}

__global__ void copy_f32_kernel(const float *__restrict__ src, float *__restrict__ dst, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) dst[i] = src[i];
}

hipError_t copy_f32(const float *src, float *dst, size_t n, hipStream_t s) {
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

template hipError_t rmsnorm<float>(const float *, const float *, float *, int, int, float, hipStream_t);
template hipError_t rmsnorm<bf16>(const float *, const bf16 *, f16 *, int, int, float, hipStream_t);
template hipError_t embed_rows<float>(const int32_t *, const float *, float *, int, int, int, hipStream_t);
template hipError_t embed_rows<bf16>(const int32_t *, const bf16 *, float *, int, int, int, hipStream_t);

}  // namespace smol
