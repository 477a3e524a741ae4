// Entry of the residual stream: the embedding gather (x[m, :] = E[ids[m], :],
// abi96062 model.py, SmolLM2Model.forward) or a copy of the caller's hidden states,
// together with what the first block's deferred RMSNorm reads (w * (x / sqrt(mean(x^2)
// + eps)), abi96062 components.py, RMSNorm; statistics in float32, one rounding to the
// operand type).
#include "common.h"
#include "kernels.h"

namespace smol {

// Four consecutive elements of a row as float (bf16 widens exactly), and back.
__device__ __forceinline__ void load4(const float *p, float v[4]) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
}
__device__ __forceinline__ void load4(const bf16 *p, float v[4]) {
  const uint2 a = *reinterpret_cast<const uint2 *>(p);
  v[0] = __uint_as_float(a.x << 16); v[1] = __uint_as_float(a.x & 0xffff0000u);
  v[2] = __uint_as_float(a.y << 16); v[3] = __uint_as_float(a.y & 0xffff0000u);
}
__device__ __forceinline__ void store4(float *p, const float v[4]) {
  *reinterpret_cast<f32x4 *>(p) = (f32x4){v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ void store4(f16 *p, const float v[4]) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<h4 *>(p) = (h4){(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3]};
}

// Sum over each row of 16 lanes, in every lane of the row: neighbours, pairs, then
// the mirrored half-rows and the mirrored row (DPP moves, no LDS round trip). Every
// lane adds the same two operands at each step, so all 16 hold the same bits.
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row_mirror
  return v;
}

// One wavefront per row: x[row] = E[ids[row]] (ids != nullptr) or x[row] = src[row];
// the row's sums of squares per 64 columns into ss_new and ss_old ([H/64, M]); and,
// when w != nullptr, xs[row] = w * x * r * 2^-8 with the row's r -- the input of the
// first deferred RMSNorm (stored at SMOL_XS_SCALE, as every xs); and the row's RoPE
// (cos, sin) table (RopeIn). An id outside [0, V) makes the row (and its sums) NaN.
// A lane handles 4-column units: unit u (columns 4u .. 4u + 3) is lane u % 64 in round
// u / 64, so each 64-column group is one DPP row of 16 lanes, summed without LDS.
template <typename T>
__global__ void __launch_bounds__(256)
rows_ss_kernel(const int32_t *__restrict__ ids, const T *__restrict__ E, const float *src, float *x,
               float *__restrict__ ss_new, float *__restrict__ ss_old, const T *__restrict__ w,
               Act<T> *__restrict__ xs, float eps, int M, int H, int V, const RopeIn rope) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  constexpr int R = 8;            // rounds kept in registers: rows up to 2048 wide
  const int nu = H / 4, nr = (nu + 63) / 64;
  // the loads that depend on nothing go out together: the row's id, its position and
  // the norm weights of the operand pass (the embedding row waits only for the id)
  const int id = ids ? ids[row] : 0;
  const int pos = (rope.cs && rope.cache_len) ? rope.cache_len[row] : rope.pos0 + row % max(rope.seq, 1);
  float wv[R][4];
  if (w && nr <= R) {
#pragma unroll
    for (int t = 0; t < R; ++t)
      if (t < nr) load4(w + 4 * min(lane + 64 * t, nu - 1), wv[t]);
  }
  if (rope.cs && lane < rope.half) {
    // RoPE angle i of this row (abi96062 components.py, RotaryEmbedding: pos * omega_i)
    rope.cs[(size_t)row * rope.half + lane] = rope_cos_sin(pos, rope.inv_freq[lane]);
  }
  float *xr = x + (size_t)row * H;
  const bool bad = ids && (id < 0 || id >= V);
  const T *er = E + (size_t)(bad ? 0 : id) * H;
  const float *sr = src + (size_t)row * H;
  auto load_unit = [&](int u, float v[4]) {
    if (bad) {
      v[0] = v[1] = v[2] = v[3] = __builtin_nanf("");
    } else if (ids) {
      load4(er + 4 * u, v);
    } else {
      load4(sr + 4 * u, v);
    }
  };
  float keep[R][4];
  float tot = 0.f;  // lanes 0, 16, 32, 48: the sums of their groups, in round order
  for (int t0 = 0; t0 < nr; t0 += R) {
    float v[R][4];
#pragma unroll
    for (int t = 0; t < R; ++t)
      if (t0 + t < nr) load_unit(min(lane + 64 * (t0 + t), nu - 1), v[t]);
#pragma unroll
    for (int t = 0; t < R; ++t) {
      if (t0 + t >= nr) break;
      const int u = lane + 64 * (t0 + t);
      const bool ok = u < nu;  // a whole 16-lane group is in or out (nu % 16 == 0)
      if (ok && (ids || src != x)) store4(xr + 4 * u, v[t]);
      float q = v[t][0] * v[t][0];
      q = fmaf(v[t][1], v[t][1], q);
      q = fmaf(v[t][2], v[t][2], q);
      q = fmaf(v[t][3], v[t][3], q);
      q = row16_sum(ok ? q : 0.f);
      if (ok && (lane & 15) == 0) {
        const int g = u >> 4;
        ss_new[(size_t)g * M + row] = q;
        ss_old[(size_t)g * M + row] = q;
        tot += q;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) keep[t][e] = v[t][e];
    }
  }
  if (!w) return;
  auto lane_val = [&](int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tot), l)); };
  const float sum = (lane_val(0) + lane_val(16)) + (lane_val(32) + lane_val(48));
  const float r = 1.0f / sqrtf(sum / (float)H + eps) * SMOL_XS_SCALE;  // xs is stored times 2^-8
  Act<T> *ur = xs + (size_t)row * H;
  if (nr <= R) {
#pragma unroll
    for (int t = 0; t < R; ++t) {
      const int u = lane + 64 * t;
      if (t >= nr || u >= nu) continue;
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = wv[t][e] * (keep[t][e] * r);
      store4(ur + 4 * u, o);
    }
  } else {
    // wider rows: the source again (read-only here; x itself only when src == x,
    // which this kernel then leaves unwritten)
    for (int u = lane; u < nu; u += 64) {
      float v[4], wu[4], o[4];
      load_unit(u, v);
      load4(w + 4 * u, wu);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = wu[e] * (v[e] * r);
      store4(ur + 4 * u, o);
    }
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
