// Internal launcher declarations (host side). Every launcher enqueues on the given
// stream and returns hipGetLastError() of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace smol {

enum { EPI_STORE = 0, EPI_RESIDUAL = 1, EPI_SWIGLU = 2, EPI_QKV_ROPE = 3 };

// Where the QKV projection writes: q [M, nq_cols]; k, v into [B, n_kv, cap, d] at
// index pos - kv_off (prefill: pos = pos0 + t) or cache_len[b] (decode, M == B).
struct QkvOut {
  int M, hidden, nq_cols, nkv_cols, head_dim;
  void *q, *k, *v;
  int seq, cap, n_kv, pos0, kv_off, max_pos;
  const int *cache_len;
  const float *inv_freq;  // host array, head_dim / 2 entries
};

// T is the storage type (weights, cache, logits); activations are Act<T>.
template <typename T>
hipError_t gemm_store(const Act<T> *A, const T *B, int M, int N, int K, void *C, int c_f32, hipStream_t s);
template <typename T>
hipError_t gemm_residual(const Act<T> *A, const T *B, int M, int N, int K, float *X, hipStream_t s);
template <typename T>
hipError_t gemm_swiglu(const Act<T> *A, const T *Wg, const T *Wu, int M, int I, int K, Act<T> *Y, hipStream_t s);
template <typename T>
hipError_t gemm_qkv_rope(const Act<T> *A, const T *Wq, const T *Wk, const T *Wv, const QkvOut &o, hipStream_t s);

template <typename T>
hipError_t rmsnorm(const float *x, const T *w, Act<T> *out, int M, int H, float eps, hipStream_t s);
template <typename T>
hipError_t embed_rows(const int32_t *ids, const T *E, float *x, int M, int H, int V, hipStream_t s);
hipError_t copy_f32(const float *src, float *dst, size_t n, hipStream_t s);

// Causal GQA attention over a [B, n_kv, cap, d] key/value store. Query t of
// sequence b sits at key index t + q_key_off; it sees key indices <= that.
struct AttnArgs {
  const void *q;  // [B*T, n_heads*d] operand type; k, v, o: storage / operand types
  const void *k, *v;
  void *o;        // [B*T, n_heads*d]
  int B, T, n_heads, n_kv, head_dim, cap, q_key_off;
};
template <typename T>
hipError_t attention_prefill(const AttnArgs &a, hipStream_t s);

// Decode: one query per sequence at key index cache_len[b]; split-K partials in ws.
struct DecodeAttnArgs {
  const void *q;  // [B, n_heads*d]
  const void *k, *v;
  void *o;        // [B, n_heads*d]
  const int *cache_len;
  int B, n_heads, n_kv, head_dim, cap, max_pos, splits, chunk;
  float *part;    // [B, n_heads, splits, head_dim + 2]
};
template <typename T>
hipError_t attention_decode(const DecodeAttnArgs &a, hipStream_t s);
int decode_splits(int cap, int *chunk);

// kernel-class timing hooks (see smol_timing_begin)
void timing_before(int kernel, hipStream_t s);
void timing_after(int kernel, hipStream_t s);

}  // namespace smol
