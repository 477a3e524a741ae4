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
//   xs [M, H] (operand type) = w * x * r_old * 2^-8, r_old: the row's r before the
//   update (2^-8 = SMOL_XS_SCALE, common.h: float16 headroom for large growth);
//   the row sums of squares of the new x as H/64 partials, ss[j * M + row] over
//   columns [64 j, 64 j + 64) (ss_new; ss_old keeps those from before the update).
// A GEMM with xs as its A operand scales output row m by r(ss_new) / r(ss_old) * 2^8.
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
// ss_old, and xs = w * x * r * 2^-8 with the row's own r (w == nullptr: no xs).
// The RoPE angles of every row, computed once per forward: cs[row * half + i] =
// (cos, sin)(pos(row) * inv_freq[i]), pos(row) = cache_len[row] when cache_len != nullptr
// (a decode step) else pos0 + row % seq.
struct RopeIn {
  float2 *cs;  // nullptr: none
  int half, pos0, seq;
  const int *cache_len;
  double inv_freq[64];  // omega_i in double: the angle is formed and reduced in double
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
int decode_splits(int cap, int head_dim, int esz, int *chunk);

// Next-token choice per row of logits (smol_sample in smol.h).
template <typename T>
hipError_t sample_next(const T *logits, long row_stride, int B, int V, float temperature, int top_k, float top_p,
                       const float *uniforms, int32_t *next_ids, hipStream_t s);

// ------------------------------------------------------------------ backward (float32)
// backward.hip: the kernels of smol_block_backward.

// A GEMM operand: up to three row-major matrices stacked along their rows (rows
// [0, seg0) from p0, [seg0, seg1) from p1, the rest from p2), row length ld.
struct BwOperand {
  const float *p0, *p1, *p2;
  int seg0, seg1, ld;
};
// C[M, N] = sum_k A(m, k) B(k, n), float32 MFMA. layout:
//   BW_NT  A [M, K] and B [N, K] (K-contiguous): y = x W^T
//   BW_NN  A [M, K], B [K, N]: dx = dy W
//   BW_TN  A [K, M] and B [K, N] (contraction down the columns): dW = dy^T x
// epi: BW_STORE C = acc; BW_ACCUM C += acc; BW_RESID C = R + acc; BW_SWIGLU, the
// SwiGLU backward: with g = G[m, n], u = G[m, half + n] (the forward's gate and up)
// and acc = dL/d(silu(g) u): C[m, n] = acc u silu'(g), C[m, half + n] = acc silu(g),
// Y[m, n] = silu(g) u.
enum { BW_NT = 0, BW_NN = 1, BW_TN = 2 };
enum { BW_STORE = 0, BW_ACCUM = 1, BW_RESID = 2, BW_SWIGLU = 3 };
// C rows [0, cseg0) go to C, [cseg0, cseg1) to C1, the rest to C2 (e.g. the three
// gradients dW_q | dW_k | dW_v of one fused launch); all with row length ldc.
// ksplit > 1: K is cut into ksplit ranges whose workgroups write unscaled partial
// tiles to part ([ksplit, M, N] floats); a second kernel adds them in split order
// and applies the epilogue (store, add or residual only).
struct BwGemm {
  BwOperand a, b;
  int M, N, K;
  float *C, *C1, *C2;
  int cseg0, cseg1, ldc;
  const float *R;
  int ldr;
  const float *G;
  int ldg, half;
  float *Y;
  int ldy;
  int ksplit;
  float *part;
};
hipError_t bw_gemm(int layout, int epi, const BwGemm &p, hipStream_t s);
// The K split bw_gemm would take for this shape and epilogue (1: none), and the
// partial-sum floats it then needs.
int bw_gemm_ksplit(int M, int N, int K, int epi);
size_t bw_gemm_part_floats(int M, int N, int K, int epi);

struct InvFreq {
  double v[64];
};
// Attention of the block being differentiated: qkv [B*T, ld] holds q | k | v (q and
// k rotated), query head h reads kv head h / G; key_mask [B, T] (token index) or
// nullptr; window > 0: a query at t sees keys t - window < t' <= t.
struct BwAttn {
  const float *qkv;
  int ld;
  int B, T, nq, nkv, G, D;
  const uint8_t *key_mask;
  int window;
  float scale, scale2;  // 1/sqrt(D), log2(e)/sqrt(D)
  float *o;             // [B*T, nq*D]            (forward)
  float *lse;           // [B, nq, T], base 2     (forward; read by dq, dkdv)
  const float *dO;      // [B*T, nq*D]
  const float *dsum;    // [B, nq, T]
  float *dqkv;          // [B*T, ld]: dq written by dq; dk, dv by bw_kv_reduce
  float *part;          // [2, nq, B*T, D]: per-query-head dk, dv partials (dkdv)
  int rope_on;
  const float2 *rope_cs;  // [B*T, D/2] (cos, sin) of each row's angles (bw_rope_table)
};
hipError_t bw_attention(int which, const BwAttn &a, hipStream_t s);  // 0 forward, 1 dq, 2 dk/dv
hipError_t bw_rowdot(const float *dO, const float *O, float *dsum, int M, int T, int nq, int D, hipStream_t s);
hipError_t bw_kv_reduce(const float *part, float *dqkv, int M, int nq, int nkv, int G, int D, int ld, hipStream_t s);
// The RoPE (cos, sin) of every row of the call: cs[m * D/2 + i] at angle
// (pos0 + m % T) * omega_i (rope_cos_sin in common.h).
hipError_t bw_rope_table(float2 *cs, int M, int T, int D, int pos0, const InvFreq &f, hipStream_t s);
hipError_t bw_rope(float *qkv, int M, int ld, int heads, int D, const float2 *cs, hipStream_t s);
hipError_t bw_rms_fwd(const float *x, const float *w, float *u, float *r, int M, int H, float eps, hipStream_t s);
int bw_rms_part_rows(int M);  // rows of the column partials bw_rms_bwd writes
hipError_t bw_rms_bwd(const float *du, const float *x, const float *r, const float *w, const float *resid, float *dx,
                      float *part, int M, int H, hipStream_t s);
hipError_t bw_colsum(const float *part, int nrows, int H, float *dw, int accumulate, hipStream_t s);
hipError_t bw_widen(const bf16 *src, float *dst, size_t n, hipStream_t s);  // dst = (float)src, exact

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
