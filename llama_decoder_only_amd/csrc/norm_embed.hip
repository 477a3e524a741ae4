// Entry of the residual stream: the embedding gather (x[m, :] = E[ids[m], :],
// abi96062 model.py, SmolLM2Model.forward) or a copy of the caller's hidden states,
// together with what the first block's deferred RMSNorm reads (w * (x / sqrt(mean(x^2)
// + eps)), abi96062 components.py, RMSNorm; statistics in float32, one rounding to the
// operand type).
#include "common.h"
#include "kernels.h"

namespace smol {

// One wavefront per row: x[row] = E[ids[row]] (ids != nullptr) or x[row] = src[row];
// the row's sums of squares per 64 columns into ss_new and ss_old ([H/64, M]); and,
// when w != nullptr, xs[row] = w * x * r * 2^-8 with the row's r -- the input of the
// first deferred RMSNorm (stored at SMOL_XS_SCALE, as every xs); and the row's RoPE (cos, sin) table (RopeIn). An id outside
// [0, V) makes the row (and its sums) NaN.
template <typename T>
__global__ void __launch_bounds__(256)
rows_ss_kernel(const int32_t *__restrict__ ids, const T *__restrict__ E, const float *src, float *x,
               float *__restrict__ ss_new, float *__restrict__ ss_old, const T *__restrict__ w,
               Act<T> *__restrict__ xs, float eps, int M, int H, int V, const RopeIn rope) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  // the loads that depend on nothing go out together: the row's id, its position and
  // the norm weights of the operand pass (the embedding row waits only for the id)
  const int id = ids ? ids[row] : 0;
  const int pos = (rope.cs && rope.cache_len) ? rope.cache_len[row] : rope.pos0 + row % max(rope.seq, 1);
  constexpr int R = 16;
  const int nj = H / 64;
  float wv[R];
  if (w && nj <= R) {
#pragma unroll
    for (int e = 0; e < R; ++e) wv[e] = to_f32(w[min(e, nj - 1) * 64 + lane]);
  }
  if (rope.cs && lane < rope.half) {
    // RoPE angle i of this row (abi96062 components.py, RotaryEmbedding: pos * omega_i)
    rope.cs[(size_t)row * rope.half + lane] = rope_cos_sin(pos, rope.inv_freq[lane]);
  }
  float *xr = x + (size_t)row * H;
  const bool bad = ids && (id < 0 || id >= V);
  const T *er = E + (size_t)(bad ? 0 : id) * H;
  const float *sr = src + (size_t)row * H;
  // The row in rounds of 16 columns per lane, every load of a round issued before any
  // is used (one memory round trip per round instead of one per 64 columns); rows up
  // to 1024 wide stay in registers for the operand pass.
  float keep[R];
  float tot = 0.f;
  for (int j0 = 0; j0 < nj; j0 += R) {
    float v[R];
#pragma unroll
    for (int e = 0; e < R; ++e) {
      const int i = min(j0 + e, nj - 1) * 64 + lane;
      v[e] = bad ? __builtin_nanf("") : ids ? to_f32(er[i]) : sr[i];
    }
#pragma unroll
    for (int e = 0; e < R; ++e) {
      if (j0 + e >= nj) break;
      const int i = (j0 + e) * 64 + lane;
      if (ids || src != x) xr[i] = v[e];
      const float q = wave_sum(v[e] * v[e]);
      tot += q;
      if (lane == 0) {
        ss_new[(size_t)(j0 + e) * M + row] = q;
        ss_old[(size_t)(j0 + e) * M + row] = q;
      }
      keep[e] = v[e];
    }
  }
  if (!w) return;
  const float r = 1.0f / sqrtf(tot / (float)H + eps) * SMOL_XS_SCALE;  // xs is stored times 2^-8
  Act<T> *ur = xs + (size_t)row * H;
  if (nj <= R) {
#pragma unroll
    for (int e = 0; e < R; ++e)
      if (e < nj) ur[e * 64 + lane] = from_f32<Act<T>>(wv[e] * (keep[e] * r));
  } else {
    for (int i = lane; i < H; i += 64) ur[i] = from_f32<Act<T>>(to_f32(w[i]) * (xr[i] * r));
  }
}

template <typename T>
hipError_t rows_ss(const int32_t *ids, const T *E, const float *src, float *x, float *ss_new, float *ss_old,
                   const T *w, Act<T> *xs, float eps, int M, int H, int V, const RopeIn &rope, hipStream_t s) {
  if (H % 64 != 0 || rope.half > 64 || (rope.cs && !rope.cache_len && rope.seq <= 0)) return hipErrorInvalidValue;
  if (M == 0) return hipSuccess;
  return launch(rows_ss_kernel<T>, dim3((M + 3) / 4), dim3(256), s, ids, E, src, x, ss_new, ss_old, w, xs, eps, M, H,
                V, rope);
}

// Generation helpers. The prompt length of sequence b is lens[b] clamped to
// [1, T] (T when lens is nullptr): right-padded prompts of different lengths.
__device__ __forceinline__ int prompt_len_of(const int32_t *lens, int b, int T) {
  return lens ? min(max(lens[b], 1), T) : T;
}

// gather_last: row b of xs_out and of the two sums-of-squares buffers ([H/64, B])
// takes row b*T + len_b - 1 of the prefill's ([H/64, B*T]), so that the head runs
// on each sequence's last prompt position only.
template <typename A>
__global__ void __launch_bounds__(256)
gather_last_kernel(const A *xs, const float *ssp, const float *ssq, int B, int T, int H, const int32_t *lens,
                   A *xs_out, float *ssp_out, float *ssq_out) {
  const int b = blockIdx.x;
  const size_t row = (size_t)b * T + prompt_len_of(lens, b, T) - 1, M = (size_t)B * T;
  for (int i = threadIdx.x; i < H; i += 256) xs_out[(size_t)b * H + i] = xs[row * H + i];
  for (int j = threadIdx.x; j < H / 64; j += 256) {
    ssp_out[(size_t)j * B + b] = ssp[j * M + row];
    ssq_out[(size_t)j * B + b] = ssq[j * M + row];
  }
}

template <typename T>
hipError_t gather_last(const Act<T> *xs, const float *ssp, const float *ssq, int B, int T_, int H, const int32_t *lens,
                       Act<T> *xs_out, float *ssp_out, float *ssq_out, hipStream_t s) {
  if (H % 64 != 0 || B < 1 || T_ < 1) return hipErrorInvalidValue;
  return launch(gather_last_kernel<Act<T>>, dim3(B), dim3(256), s, xs, ssp, ssq, B, T_, H, lens, xs_out, ssp_out,
                ssq_out);
}

// pos[j * B + b] = len_b + j for j < n: the cache length of every decode step.
__global__ void __launch_bounds__(256) fill_positions_kernel(int32_t *pos, int B, int n, int T, const int32_t *lens) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < B * n) pos[i] = prompt_len_of(lens, i % B, T) + i / B;
}

hipError_t fill_positions(int32_t *pos, int B, int n, int T, const int32_t *lens, hipStream_t s) {
  if (B * n == 0) return hipSuccess;
  return launch(fill_positions_kernel, dim3((B * n + 255) / 256), dim3(256), s, pos, B, n, T, lens);
}

template hipError_t gather_last<float>(const float *, const float *, const float *, int, int, int, const int32_t *,
                                       float *, float *, float *, hipStream_t);
template hipError_t gather_last<bf16>(const f16 *, const float *, const float *, int, int, int, const int32_t *, f16 *,
                                      float *, float *, hipStream_t);

template hipError_t rows_ss<float>(const int32_t *, const float *, const float *, float *, float *, float *,
                                   const float *, float *, float, int, int, int, const RopeIn &, hipStream_t);
template hipError_t rows_ss<bf16>(const int32_t *, const bf16 *, const float *, float *, float *, float *, const bf16 *,
                                  f16 *, float, int, int, int, const RopeIn &, hipStream_t);

}  // namespace smol
