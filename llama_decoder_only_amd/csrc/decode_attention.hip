// Decode attention: one new query per (sequence, head) against the KV cache,
// split along the keys so that the whole cache streams through every CU.
//
// The new token of sequence b sits at position P = cache_len[b] and sees keys
// 0 .. P (Sualeh77 model.py, "4. Attention": with a cache the single new token
// attends to all past keys and itself), minus those an optional key mask removes
// (the pages' additive padding mask) and, on a windowed block, those at or before
// P - window. This step is bound by HBM: every cached key and value is read once.
//
// Kernel 1, grid (splits, n_kv, B), 256 threads: a workgroup takes `chunk`
// consecutive keys of kv head g and serves all G query heads of the group.
// D/EPC lanes cooperate on one key row (16-byte loads, fully coalesced rows);
// phase 1 writes scaled scores to LDS, phase 2 takes the chunk's max and exp-sum
// per head, phase 3 accumulates p * v. The partial (max, sum, o[D]) goes to ws.
// Kernel 2, grid (B * n_heads), D threads: merges the partials of one head
// (rescaling by exp(m_s - m)) and writes the attention output.
#include "common.h"
#include "kernels.h"

namespace smol {

constexpr int DEC_THREADS = 256;

// Keys per workgroup: 512 for a 2-byte cache at head_dim 64, else 256. At the batch-64
// step over 2048 keys, 512-key chunks (4 splits, 150 registers, 3 waves per SIMD)
// leave half the partials to merge: the step went from 1.853 to 1.791 ms although the
// kernel itself went from 22.5 to 23.2 us (384 keys: 1.917 ms, 1024: 2.456 ms at one
// wave per SIMD). Other instances would need about 250 registers at 512.
__host__ __device__ constexpr int dec_chunk(int head_dim, int esz) { return head_dim == 64 && esz == 2 ? 512 : 256; }

int decode_splits(int cap, int head_dim, int esz, int *chunk) {
  *chunk = dec_chunk(head_dim, esz);
  return (cap + *chunk - 1) / *chunk;
}

__device__ __forceinline__ bool decode_pos_ok(int P, int cap, int max_pos) { return P >= 0 && P < cap && P < max_pos; }

template <typename T, int D, int G>
__global__ void __launch_bounds__(DEC_THREADS)
decode_attn_kernel(const DecodeAttnArgs a) {
  using A = Act<T>;  // q arrives in the operand type; the cache is in the storage type T
  constexpr int EPC = 16 / sizeof(T);
  constexpr int LPK = D / EPC;             // lanes per key row
  constexpr int KPP = DEC_THREADS / LPK;   // keys per pass
  constexpr int CHUNK = dec_chunk(D, sizeof(T));
  static_assert(64 % LPK == 0, "a key row must stay inside one wavefront");

  __shared__ float S[G][CHUNK];
  __shared__ float red[KPP][G][D];
  __shared__ float stat[G][2];

  const int sp = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int kk = tid / LPK, dl = tid % LPK, d0 = dl * EPC;
  const int P = a.cache_len[b];
  float *part = a.part + (((size_t)b * a.n_heads + g * G) * a.splits + sp) * (D + 2);
  const size_t head_stride = (size_t)a.splits * (D + 2);

  const int k_begin = sp * CHUNK;
  const int k_end = decode_pos_ok(P, a.cap, a.max_pos) ? min(k_begin + CHUNK, P + 1) : 0;
  const int k_lo = a.window > 0 ? P - a.window + 1 : 0;  // first key inside the window
  const int n = k_end <= k_lo ? 0 : k_end - k_begin;     // a chunk wholly before it is empty
  if (n <= 0) {  // empty split: neutral partial
    if (tid < G) {
      part[tid * head_stride + 0] = -INFINITY;
      part[tid * head_stride + 1] = 0.f;
    }
    return;
  }

  float q[G][EPC];
  const A *qp = (const A *)a.q + (size_t)b * a.n_heads * D + g * G * D + d0;
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const Chunk16 c = ld16(qp + hh * D);
#pragma unroll
    for (int j = 0; j < EPC; ++j) q[hh][j] = to_f32(chunk_elem<A>(c, j));
  }

  const T *kb = (const T *)a.k + ((size_t)(b * a.n_kv + g) * a.cap + k_begin) * D + d0;
  const T *vb = (const T *)a.v + ((size_t)(b * a.n_kv + g) * a.cap + k_begin) * D + d0;
  const float c_log2 = 1.4426950408889634f / sqrtf((float)D);

  // phase 1: scores
  constexpr int PASSES = CHUNK / KPP;
  {
    Chunk16 kc[PASSES];
    bool keep[PASSES];
#pragma unroll
    for (int it = 0; it < PASSES; ++it) {
      const int j = min(kk + it * KPP, n - 1);  // rows past the chunk re-read its last key
      kc[it] = ld16(kb + (size_t)j * D);
      keep[it] = (!a.key_mask || a.key_mask[(size_t)b * a.mask_ld + k_begin + j] != 0) && k_begin + j >= k_lo;
    }
#pragma unroll
    for (int it = 0; it < PASSES; ++it) {
      const int j = kk + it * KPP;
      float dot[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float acc = 0.f;
#pragma unroll
        for (int x = 0; x < EPC; ++x) acc += q[hh][x] * to_f32(chunk_elem<T>(kc[it], x));
        dot[hh] = acc;
      }
#pragma unroll
      for (int o = LPK / 2; o > 0; o >>= 1)
#pragma unroll
        for (int hh = 0; hh < G; ++hh) dot[hh] += __shfl_xor(dot[hh], o, 64);
      if (dl == 0 && j < n)
#pragma unroll
        for (int hh = 0; hh < G; ++hh) S[hh][j] = keep[it] ? dot[hh] * c_log2 : -INFINITY;
    }
  }
  __syncthreads();

  // phase 2: per-head max and exp-sum over the chunk (wave w serves head w)
  const int w = tid >> 6, lane = tid & 63;
  for (int hh = w; hh < G; hh += DEC_THREADS / 64) {
    float m = -INFINITY;
    for (int j = lane; j < n; j += 64) m = fmaxf(m, S[hh][j]);
    m = wave_max(m);
    const float mu = m == -INFINITY ? 0.f : m;  // every key of the chunk masked: p = 0
    float l = 0.f;
    for (int j = lane; j < n; j += 64) {
      const float p = exp2f(S[hh][j] - mu);
      S[hh][j] = p;
      l += p;
    }
    l = wave_sum(l);
    if (lane == 0) {
      stat[hh][0] = m;
      stat[hh][1] = l;
    }
  }
  __syncthreads();

  // phase 3: o = sum_j p_j v_j
  {
    float acc[G][EPC];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int x = 0; x < EPC; ++x) acc[hh][x] = 0.f;
    Chunk16 vc[PASSES];
#pragma unroll
    for (int it = 0; it < PASSES; ++it) {
      const int j = min(kk + it * KPP, n - 1);
      vc[it] = ld16(vb + (size_t)j * D);
    }
#pragma unroll
    for (int it = 0; it < PASSES; ++it) {
      const int j = kk + it * KPP;
      if (j < n) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float p = S[hh][j];
#pragma unroll
          for (int x = 0; x < EPC; ++x) acc[hh][x] += p * to_f32(chunk_elem<T>(vc[it], x));
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int x = 0; x < EPC; ++x) red[kk][hh][d0 + x] = acc[hh][x];
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += DEC_THREADS) {
    const int hh = i / D, d = i % D;
    float s = 0.f;
#pragma unroll 8
    for (int r = 0; r < KPP; ++r) s += red[r][hh][d];
    part[hh * head_stride + 2 + d] = s;
  }
  if (tid < G) {
    part[tid * head_stride + 0] = stat[tid][0];
    part[tid * head_stride + 1] = stat[tid][1];
  }
}

template <typename T, int D>
__global__ void __launch_bounds__(D)
decode_combine_kernel(const DecodeAttnArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.n_heads, h = bh % a.n_heads;
  const int d = threadIdx.x;
  const int P = a.cache_len[b];
  using A = Act<T>;
  A *out = (A *)a.o + (size_t)b * a.n_heads * D + h * D + d;
  if (!decode_pos_ok(P, a.cap, a.max_pos)) {
    *out = from_f32<A>(__builtin_nanf(""));
    return;
  }
  const float *part = a.part + ((size_t)b * a.n_heads + h) * a.splits * (D + 2);
  const int used = (P + a.chunk) / a.chunk;  // splits that hold keys 0 .. P
  // Online merge in rounds of R splits, every load of a round in flight at once
  // (indices clamped in bounds, surplus entries masked out).
  constexpr int R = 8;
  float m = -INFINITY, l = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < used; s0 += R) {
    float ms[R], ls[R], os[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float *ps = part + (size_t)min(s0 + i, used - 1) * (D + 2);
      ms[i] = ps[0];
      ls[i] = ps[1];
      os[i] = ps[2 + d];
    }
    float mr = m;
#pragma unroll
    for (int i = 0; i < R; ++i)
      if (s0 + i < used) mr = fmaxf(mr, ms[i]);
    const float f = m == -INFINITY ? 0.f : exp2f(m - mr);  // a split with no key weighs 0
    l *= f;
    acc *= f;
#pragma unroll
    for (int i = 0; i < R; ++i)
      if (s0 + i < used) {
        const float fi = ms[i] == -INFINITY ? 0.f : exp2f(ms[i] - mr);
        l += fi * ls[i];
        acc += fi * os[i];
      }
    m = mr;
  }
  *out = from_f32<A>(acc / l);
}

template <typename T, int D, int G>
static hipError_t launch_dec(const DecodeAttnArgs &a, hipStream_t s) {
  timing_before(8, s);
  hipError_t e = launch(decode_attn_kernel<T, D, G>, dim3(a.splits, a.n_kv, a.B), dim3(DEC_THREADS), s, a);
  timing_after(8, s);
  if (e != hipSuccess) return e;
  timing_before(9, s);
  e = launch(decode_combine_kernel<T, D>, dim3(a.B * a.n_heads), dim3(D), s, a);
  timing_after(9, s);
  return e;
}

template <typename T, int D>
static hipError_t launch_dec_d(const DecodeAttnArgs &a, hipStream_t s) {
  switch (a.n_heads / a.n_kv) {
    case 1: return launch_dec<T, D, 1>(a, s);
    case 2: return launch_dec<T, D, 2>(a, s);
    case 3: return launch_dec<T, D, 3>(a, s);
    case 4: return launch_dec<T, D, 4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t attention_decode(const DecodeAttnArgs &a, hipStream_t s) {
  if (a.head_dim == 64) return launch_dec_d<T, 64>(a, s);
  if (a.head_dim == 128) return launch_dec_d<T, 128>(a, s);
  return hipErrorInvalidValue;
}

template hipError_t attention_decode<float>(const DecodeAttnArgs &, hipStream_t);
template hipError_t attention_decode<bf16>(const DecodeAttnArgs &, hipStream_t);

}  // namespace smol
