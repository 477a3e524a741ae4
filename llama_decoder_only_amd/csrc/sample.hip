// Next-token choice from one row of logits per sequence: greedy, or temperature /
// top-k / top-p filtered sampling with a uniform number supplied by the caller.
//
// What is computed (Sualeh77 model.py, "7. Top-level SmolLM2-135M Model
// Architecture", generate; abi96062 model.py, SmolLM2Model.generate):
//   temperature == 0: the index of the largest logit (the lowest such index on ties);
//   otherwise, with z = logit / temperature:
//     top-k (0 < k < V): drop every token whose logit is below the k-th largest
//       logit (tokens equal to it stay);
//     top-p (p < 1): order the remaining tokens by logit, descending (equal logits by
//       ascending index), take their softmax probabilities and drop each token after
//       the first whose preceding tokens already hold more than p of the mass;
//     sample from the softmax of the kept z: the first index j, in vocabulary order,
//       whose cumulative probability exceeds u (inverse CDF with the caller's u).
// A row holding a NaN gives -1; so does a sampled row whose largest logit is not
// finite (its softmax is undefined).
//
// One workgroup of 1024 threads per row. The row stays in L2 and is read once per
// pass: the maximum; for top-k a radix select of the k-th largest logit over
// order-preserving 32-bit keys (8-bit digits, exact integer counts); for top-p a
// radix select by probability mass (4-bit digits; every float sum is taken in a
// fixed order, so the result does not depend on scheduling); then an ordered scan
// (each wave owns a contiguous range of the vocabulary) for the inverse CDF.
#include "common.h"
#include "kernels.h"

namespace smol {

namespace {

constexpr int NT = 1024, NWV = NT / 64;

// Order-preserving key: a > b (as floats, -0 == +0) <=> key(a) > key(b).
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(__fadd_rn(f, 0.0f));  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <typename T>
__device__ __forceinline__ float ld(const T *row, int i) {
  return to_f32(row[i]);
}

// Sum over the block, taken in a fixed order (a shuffle tree per wave, then the wave
// sums in wave order); every thread gets the same value.
__device__ float block_sum(float v, float *red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_down(v, o, 64);
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NWV; ++i) s += red[i];
  __syncthreads();
  return s;
}

__device__ int block_sum_int(int v, int *red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_down(v, o, 64);
  if (lane == 0) red[w] = v;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int i = 0; i < NWV; ++i) s += red[i];
  __syncthreads();
  return s;
}

// Inclusive scan over the 64 lanes of a wave (fixed order).
template <typename V>
__device__ __forceinline__ V wave_incl_scan(V v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const V t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

struct SampleShared {
  uint32_t hist[256];
  float fbin[NWV][16];
  float fred[NWV];
  int ired[NWV];
  uint32_t kred[NWV];
  int xred[NWV];
  float wave_total[NWV];
  int wave_ties[NWV];
  uint32_t sel_key;
  int sel_want;
  int answer;
};

}  // namespace

template <typename T>
__global__ void __launch_bounds__(NT) sample_kernel(const T *logits, long row_stride, int V, float temperature,
                                                    int top_k, float top_p, const float *uniforms, int32_t *next_ids) {
  __shared__ SampleShared sh;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const T *row = logits + (size_t)blockIdx.x * row_stride;

  // ---- pass 1: maximum (lowest index on ties), NaN check
  uint32_t kmax = 0;
  int imax = 0x7fffffff, nan = 0;
  for (int i = tid; i < V; i += NT) {
    const float f = ld(row, i);
    nan |= f != f;
    const uint32_t k = fkey(f);
    if (k > kmax || (k == kmax && i < imax)) kmax = k, imax = i;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t k2 = __shfl_xor(kmax, o, 64);
    const int i2 = __shfl_xor(imax, o, 64);
    if (k2 > kmax || (k2 == kmax && i2 < imax)) kmax = k2, imax = i2;
  }
  if (lane == 0) sh.kred[w] = kmax, sh.xred[w] = imax;
  nan = block_sum_int(nan, sh.ired);  // also orders the writes above
  kmax = sh.kred[0];
  imax = sh.xred[0];
  for (int i = 1; i < NWV; ++i)
    if (sh.kred[i] > kmax || (sh.kred[i] == kmax && sh.xred[i] < imax)) kmax = sh.kred[i], imax = sh.xred[i];
  const float lmax = ld(row, imax);
  if (nan || (temperature > 0.f && !isfinite(lmax))) {
    if (tid == 0) next_ids[blockIdx.x] = -1;
    return;
  }
  if (!(temperature > 0.f)) {
    if (tid == 0) next_ids[blockIdx.x] = imax;
    return;
  }
  const float inv_t = 1.0f / temperature;
  auto weight = [&](float f) { return expf((f - lmax) * inv_t); };

  // ---- top-k: key of the k-th largest logit (radix select, 8-bit digits, MSB first)
  uint32_t kth = 0;  // keep keys >= kth
  if (top_k > 0 && top_k < V) {
    uint32_t prefix = 0, mask = 0;
    int want = top_k;  // rank still wanted within the current prefix
    for (int d = 24; d >= 0; d -= 8) {
      for (int i = tid; i < 256; i += NT) sh.hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < V; i += NT) {
        const uint32_t k = fkey(ld(row, i));
        if ((k & mask) == prefix) atomicAdd(&sh.hist[(k >> d) & 255], 1u);
      }
      __syncthreads();
      if (w == 0) {  // lane j owns bins 4j .. 4j+3; find the bin holding rank `want`, from the top
        uint32_t c[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) c[e] = sh.hist[4 * lane + e];
        const uint32_t s = c[0] + c[1] + c[2] + c[3];
        // incl: count in this lane's bins and every higher lane's (a suffix scan)
        uint32_t incl = s;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t t = __shfl_down(incl, o, 64);
          if (lane + o < 64) incl += t;
        }
        uint32_t above = incl - s;
        if (above < (uint32_t)want && (uint32_t)want <= incl) {
          for (int e = 3; e >= 0; --e) {
            if ((uint32_t)want <= above + c[e]) {
              sh.sel_key = (uint32_t)(4 * lane + e);
              sh.sel_want = want - (int)above;
              break;
            }
            above += c[e];
          }
        }
      }
      __syncthreads();
      prefix |= sh.sel_key << d;
      mask |= 255u << d;
      want = sh.sel_want;
      __syncthreads();
    }
    kth = prefix;
  }

  // ---- top-p: the token at which the descending cumulative mass first exceeds p
  // (radix select by mass, 4-bit digits). Tokens above key kp stay, and the first
  // n_tie tokens (by index) whose key equals kp.
  uint32_t kp = 0;
  int n_tie = 0x7fffffff;
  if (top_p < 1.0f) {
    float z = 0.f;
    for (int i = tid; i < V; i += NT) {
      const float f = ld(row, i);
      if (fkey(f) >= kth) z += weight(f);
    }
    const float P = top_p * block_sum(z, sh.fred);
    uint32_t prefix = 0, mask = 0;
    float above = 0.f;  // mass of the kept tokens with keys above the current range
    bool crossed = true;
    for (int d = 28; d >= 0; d -= 4) {
      float bin[16];
#pragma unroll
      for (int b = 0; b < 16; ++b) bin[b] = 0.f;
      for (int i = tid; i < V; i += NT) {
        const float f = ld(row, i);
        const uint32_t k = fkey(f);
        if (k >= kth && (k & mask) == prefix) {
          const uint32_t dg = (k >> d) & 15;
          const float e = weight(f);
#pragma unroll
          for (int b = 0; b < 16; ++b) bin[b] += dg == (uint32_t)b ? e : 0.f;
        }
      }
#pragma unroll
      for (int b = 0; b < 16; ++b) {
        float v = bin[b];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_down(v, o, 64);
        if (lane == 0) sh.fbin[w][b] = v;
      }
      __syncthreads();
      if (tid == 0) {
        float tot[16];
        for (int b = 0; b < 16; ++b) {
          tot[b] = 0.f;
          for (int i = 0; i < NWV; ++i) tot[b] += sh.fbin[i][b];
        }
        int sel = -1;
        for (int b = 15; b >= 0; --b) {
          if (tot[b] > 0.f && above + tot[b] > P) {
            sel = b;
            break;
          }
          above += tot[b];
        }
        if (sel < 0) {  // the mass never exceeds P (rounding): keep everything
          sh.sel_want = -1;
        } else {
          sh.sel_key = (uint32_t)sel;
          sh.sel_want = 0;
          sh.fred[0] = above;
        }
      }
      __syncthreads();
      if (sh.sel_want < 0) {
        crossed = false;
        __syncthreads();
        break;
      }
      prefix |= sh.sel_key << d;
      mask |= 15u << d;
      above = sh.fred[0];
      __syncthreads();
    }
    if (crossed) {
      kp = prefix;
      // every token with key kp has the same weight q: keep the first c of them,
      // c the smallest count with above + c * q > P
      float fk = 0.f;
      {
        // the float whose key is kp
        const uint32_t u = (kp & 0x80000000u) ? (kp & 0x7fffffffu) : ~kp;
        fk = __uint_as_float(u);
      }
      const float q = weight(fk);
      float c = floorf((P - above) / q) + 1.f;
      n_tie = c < 1.f ? 1 : (c > 2.0e9f ? 0x7fffffff : (int)c);
    } else {
      kp = kth;
      n_tie = 0x7fffffff;
    }
  }
  const uint32_t klo = top_p < 1.0f ? kp : kth;  // keys > klo stay; keys == klo: the first n_tie
                                                  // (kp >= kth, so top-k holds for them too)

  // ---- inverse CDF in vocabulary order. Wave w owns [w * R, (w + 1) * R); it walks
  // its range in 64-element steps (lane l: element base + l) with a running sum.
  const int R = (V + NWV - 1) / NWV;
  const int lo = min(V, w * R), hi = min(V, lo + R);
  // ties of key klo before this wave's range (rank of a tie = its order by index)
  int nt = 0;
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    if (i < hi && fkey(ld(row, i)) == klo) ++nt;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) nt += __shfl_down(nt, o, 64);
  if (lane == 0) sh.wave_ties[w] = nt;
  __syncthreads();
  int tie0 = 0;
  for (int i = 0; i < w; ++i) tie0 += sh.wave_ties[i];
  // weights of the kept tokens, summed per wave in index order
  auto kept_weight = [&](int tie_rank, bool is_tie, float f) {
    const bool keep = fkey(f) > klo || (is_tie && tie_rank < n_tie);
    return keep ? weight(f) : 0.f;
  };
  float run = 0.f;
  int ties = tie0;
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    const float f = i < hi ? ld(row, i) : -INFINITY;
    const bool is_tie = i < hi && fkey(f) == klo;
    const int ti = wave_incl_scan<int>(is_tie ? 1 : 0);
    const float e = i < hi ? kept_weight(ties + ti - (is_tie ? 1 : 0), is_tie, f) : 0.f;
    const float incl = wave_incl_scan<float>(e);
    run += __shfl(incl, 63, 64);
    ties += __shfl(ti, 63, 64);
  }
  if (lane == 0) sh.wave_total[w] = run;
  if (tid == 0) sh.answer = -1;
  __syncthreads();
  float total = 0.f;
  for (int i = 0; i < NWV; ++i) total += sh.wave_total[i];
  const float target = uniforms[blockIdx.x] * total;
  // owner: the first wave whose range ends above the target; else the last with mass
  int owner = -1;
  float pre = 0.f, owner_pre = 0.f;
  for (int i = 0; i < NWV; ++i) {
    if (sh.wave_total[i] > 0.f) {
      if (pre + sh.wave_total[i] > target) {
        owner = i;
        owner_pre = pre;
        break;
      }
      owner = i;
      owner_pre = pre;
    }
    pre += sh.wave_total[i];
  }
  if (w == owner) {
    float r = owner_pre;
    int t = tie0;
    int found = -1, last = -1;
    for (int base = lo; base < hi && found < 0; base += 64) {
      const int i = base + lane;
      const float f = i < hi ? ld(row, i) : -INFINITY;
      const bool is_tie = i < hi && fkey(f) == klo;
      const int ti = wave_incl_scan<int>(is_tie ? 1 : 0);
      const float e = i < hi ? kept_weight(t + ti - (is_tie ? 1 : 0), is_tie, f) : 0.f;
      const float incl = wave_incl_scan<float>(e);
      const unsigned long long hit = __ballot(e > 0.f && r + incl > target);
      const unsigned long long any = __ballot(e > 0.f);
      if (hit) found = base + __ffsll((long long)hit) - 1;
      if (any) last = base + 63 - __clzll((long long)any);
      r += __shfl(incl, 63, 64);
      t += __shfl(ti, 63, 64);
    }
    if (lane == 0) sh.answer = found >= 0 ? found : last;
  }
  __syncthreads();
  if (tid == 0) next_ids[blockIdx.x] = sh.answer;
}

template <typename T>
hipError_t sample_next(const T *logits, long row_stride, int B, int V, float temperature, int top_k, float top_p,
                       const float *uniforms, int32_t *next_ids, hipStream_t s) {
  return launch(sample_kernel<T>, dim3(B), dim3(NT), s, logits, row_stride, V, temperature, top_k, top_p, uniforms,
                next_ids);
}

template hipError_t sample_next<float>(const float *, long, int, int, float, int, float, const float *, int32_t *,
                                       hipStream_t);
template hipError_t sample_next<bf16>(const bf16 *, long, int, int, float, int, float, const float *, int32_t *,
                                      hipStream_t);

}  // namespace smol
