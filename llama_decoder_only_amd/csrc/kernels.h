// Internal launcher declarations (host side). Every launcher enqueues on the given
// stream and returns hipGetLastError() of its launch.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace smol {

enum { EPI_STORE = 0, EPI_RESIDUAL = 1, EPI_SWIGLU = 2, EPI_QKV_ROPE = 3,
       EPI_SPLIT = 16 };  // flag: a K split's partial sums instead of the epilogue

// Where the QKV projection writes: q [M, nq_cols]; k, v into [B, n_kv, cap, d] at
// index pos - kv_off (prefill: pos = pos0 + t) or cache_len[b] (decode, M == B).
struct QkvOut {
  int M, hidden, nq_cols, nkv_cols, head_dim;
  void *q, *k, *v;
  int seq, cap, n_kv, pos0, kv_off, max_pos;
  const int *cache_len;
  const float2 *rope;     // [M, head_dim / 2] (cos, sin) of each row's angles (RopeIn)
  int rope_on;            // 0: a NoPE block (q and k stay as projected)
};

// The deferred RMSNorm u = w * x * r, r = 1 / sqrt(mean(x^2) + eps) per row of the
// float residual stream x [M, H]. Whoever updates x also leaves, for the next norm,
//   xs [M, H] (operand type) = w * x * r_old, r_old: the row's r before the update;
//   the row sums of squares of the new x as H/64 partials, ss[j * M + row] over
//   columns [64 j, 64 j + 64) (ss_new; ss_old keeps those from before the update).
// A GEMM with xs as its A operand scales output row m by r(ss_new) / r(ss_old).
struct NormIn {
  const float *ss_new, *ss_old;  // ss_new == nullptr: A is used as it is
  float eps;
};
// What a residual GEMM leaves for the next norm: ss_new (nullptr: nothing) and, when
// xs != nullptr, xs with norm weight w and r_old from ss_old.
struct NormOut {
  const float *ss_old;
  float *ss_new;
  const void *w;
  void *xs;
  float eps;
};

// T is the storage type (weights, cache, logits); activations are Act<T>.
// part: float scratch for K-split partial sums, gemm_part_floats(M, N, K, sizeof(T))
// floats (nullptr: never split). Calls on one stream may share it.
template <typename T>
hipError_t gemm_store(const Act<T> *A, const NormIn &nrm, const T *B, int M, int N, int K, void *C, int c_f32,
                      float *part, hipStream_t s);
template <typename T>
hipError_t gemm_residual(const Act<T> *A, const T *B, int M, int N, int K, float *X, const NormOut &nrm, float *part,
                         hipStream_t s);
template <typename T>
hipError_t gemm_swiglu(const Act<T> *A, const NormIn &nrm, const T *Wg, const T *Wu, int M, int I, int K, Act<T> *Y,
                       float *part, hipStream_t s);
template <typename T>
hipError_t gemm_qkv_rope(const Act<T> *A, const NormIn &nrm, const T *Wq, const T *Wk, const T *Wv, const QkvOut &o,
                         float *part, hipStream_t s);
size_t gemm_part_floats(int M, int N, int K, int esz);  // 0: that GEMM does not split

// x[m] = E[ids[m]] (ids != nullptr: the embedding gather) or x[m] = src[m], and what
// the first deferred RMSNorm reads: the row sums of squares into both ss_new and
// ss_old, and xs = w * x * r with the row's own r (w == nullptr: no xs).
// The RoPE angles of every row, computed once per forward: cs[row * half + i] =
// (cos, sin)(pos(row) * inv_freq[i]), pos(row) = cache_len[row] when cache_len != nullptr
// (a decode step) else pos0 + row % seq.
struct RopeIn {
  float2 *cs;  // nullptr: none
  int half, pos0, seq;
  const int *cache_len;
  float inv_freq[64];
};
template <typename T>
hipError_t rows_ss(const int32_t *ids, const T *E, const float *src, float *x, float *ss_new, float *ss_old,
                   const T *w, Act<T> *xs, float eps, int M, int H, int V, const RopeIn &rope, hipStream_t s);

// Generation: the last prompt position of each sequence's prefill state (xs row and
// its two sums-of-squares columns), and the per-step decode positions
// pos[j * B + b] = len_b + j, with len_b = lens[b] clamped to [1, T] (T: no lens).
template <typename T>
hipError_t gather_last(const Act<T> *xs, const float *ssp, const float *ssq, int B, int T_, int H, const int32_t *lens,
                       Act<T> *xs_out, float *ssp_out, float *ssq_out, hipStream_t s);
hipError_t fill_positions(int32_t *pos, int B, int n, int T, const int32_t *lens, hipStream_t s);

// Causal GQA attention over a [B, n_kv, cap, d] key/value store. Query t of
// sequence b sits at key index t + q_key_off; it sees key indices <= that, except
// those whose key_mask byte is 0 (key_mask: [B, mask_ld] uint8 over key indices, or
// nullptr). A query left with no key comes out NaN.
struct AttnArgs {
  const void *q;  // [B*T, n_heads*d] operand type; k, v, o: storage / operand types
  const void *k, *v;
  void *o;        // [B*T, n_heads*d]
  int B, T, n_heads, n_kv, head_dim, cap, q_key_off;
  const uint8_t *key_mask;
  int mask_ld;
  int window;  // > 0: a query at key index i sees only indices > i - window
};
template <typename T>
hipError_t attention_prefill(const AttnArgs &a, hipStream_t s);

// Decode: one query per sequence at key index cache_len[b]; split-K partials in ws.
// key_mask as in AttnArgs ([B, mask_ld], or nullptr).
struct DecodeAttnArgs {
  const void *q;  // [B, n_heads*d]
  const void *k, *v;
  void *o;        // [B, n_heads*d]
  const int *cache_len;
  int B, n_heads, n_kv, head_dim, cap, max_pos, splits, chunk;
  float *part;    // [B, n_heads, splits, head_dim + 2]
  const uint8_t *key_mask;
  int mask_ld;
  int window;     // > 0: the new token sees only key indices > cache_len - window
};
template <typename T>
hipError_t attention_decode(const DecodeAttnArgs &a, hipStream_t s);
int decode_splits(int cap, int *chunk);

// Next-token choice per row of logits (smol_sample in smol.h).
template <typename T>
hipError_t sample_next(const T *logits, long row_stride, int B, int V, float temperature, int top_k, float top_p,
                       const float *uniforms, int32_t *next_ids, hipStream_t s);

// Kernel-class timing (see smol_timing_begin). timing_before arms the next launch()
// of that class with a start/stop event pair, which hipExtLaunchKernelGGL records at
// the dispatch itself: the pair brackets the kernel's own execution, not the queue
// around it. timing_after counts the launch.
void timing_before(int kernel, hipStream_t s);
void timing_after(int kernel, hipStream_t s);
bool timing_take(hipEvent_t *start, hipEvent_t *stop);  // the armed pair, handed out once

// A launch that records start (at the dispatch) and/or stop (at the kernel's end)
// when they are not null.
template <typename... Params, typename... Args>
hipError_t launch_ev(void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t s, hipEvent_t start,
                     hipEvent_t stop, Args... args) {
  if (start || stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, start, stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  return hipGetLastError();
}

// Every single-kernel operation of the library launches here.
template <typename... Params, typename... Args>
hipError_t launch(void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t s, Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  timing_take(&e0, &e1);
  return launch_ev(kernel, grid, block, s, e0, e1, args...);
}

}  // namespace smol
