// MFMA GEMM  C[M, N] = A[M, K] . B[N, K]^T  with fused epilogues, for gfx950.
//
// Both operands are K-contiguous (activations row-major, weights [out, in] as the
// linear layers store them), so every lane reads 8 consecutive K values of one
// row for a 32x32x16 MFMA step. Weight rows arrive in the storage type W and are
// converted to the activations' operand type Act<W> on their way into LDS. A
// workgroup owns a BM x BN tile; its waves each own (32*TM) x (32*TN). K is staged through LDS 128 bytes per row at a time,
// double-buffered: the next stage is fetched into registers while the current
// one feeds the MFMAs.
//
// Epilogues (what the five projections of a block and the head need):
//   EPI_STORE     C = acc                       lm_head logits (float or the storage type)
//   EPI_RESIDUAL  X += acc (float X)            o_proj and down_proj with residual add
//   EPI_SWIGLU    Y = silu(gate) * up           gate/up projection; B rows interleave
//                                               32 gate rows then 32 up rows
//   EPI_QKV_ROPE  q, k rotated at their position, q stored [M, n_heads*d];
//                 k, v stored into the [B, n_kv, cap, d] cache at their index.
// Projection math: abi96062 components.py (GroupedQueryAttention, SwiGLU_FFN);
// RoPE pairs (i, i + d/2): Sualeh77 model.py, "3. RoPE".
#include "common.h"
#include "kernels.h"

namespace smol {

struct GemmParams {
  const void *A;
  int lda;
  const void *B0, *B1, *B2;
  int M, N, K;
  void *C;
  int ldc;
  int c_f32;
  // QKV + RoPE
  int nq_cols, nkv_cols, head_dim;
  void *q_out, *k_out, *v_out;
  int seq, cap, n_kv, pos0, kv_off, max_pos;
  const int *cache_len;
  float inv_freq[64];
};

template <typename W, int EPI>
__device__ __forceinline__ const W *b_row(const GemmParams &p, int n) {
  if (EPI == EPI_SWIGLU) {
    const int c = n & 63;
    const int r = ((n >> 6) << 5) + (c & 31);
    return (c < 32 ? (const W *)p.B0 : (const W *)p.B1) + (size_t)r * p.K;
  } else if (EPI == EPI_QKV_ROPE) {
    if (n < p.nq_cols) return (const W *)p.B0 + (size_t)n * p.K;
    n -= p.nq_cols;
    if (n < p.nkv_cols) return (const W *)p.B1 + (size_t)n * p.K;
    return (const W *)p.B2 + (size_t)(n - p.nkv_cols) * p.K;
  } else {
    return (const W *)p.B0 + (size_t)n * p.K;
  }
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

template <typename W, int TM, int TN, int WAVES_M, int WAVES_N, int EPI>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N)
gemm_kernel(const GemmParams p) {
  using T = Act<W>;  // MFMA operand type; B rows are converted from W while staged
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int BM = 32 * TM * WAVES_M;
  constexpr int BN = 32 * TN * WAVES_N;
  constexpr int EPC = 16 / sizeof(T);           // elements per 16-byte chunk
  constexpr int BK = 128 / sizeof(T);           // K elements per stage (128 bytes per row)
  constexpr int PITCH = BK + EPC;               // padded LDS row (144 bytes)
  constexpr int KSTEPS = BK / 16;
  constexpr int A_CH = BM * 8 / NT;             // 16-byte chunks per thread per stage
  constexpr int B_CH = BN * 8 / NT;
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile/thread mismatch");

  __shared__ __attribute__((aligned(16))) T smem[2][(BM + BN) * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;

  // XCD-aware tile order: consecutive workgroups land on different XCDs, so give
  // neighbouring N tiles (which share the A rows) to the same XCD's L2.
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = p.N / BN;
  const int ntiles = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if (ntiles % 8 == 0) bid = (bid % 8) * (ntiles / 8) + bid / 8;
  const int tm = bid % tiles_m, tn = bid / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;

  // per-thread global source pointers (fixed rows, K advances)
  const T *a_src[A_CH];
  const W *b_src[B_CH];
  int a_dst[A_CH], b_dst[B_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = tid + i * NT;
    const int r = c >> 3, k = (c & 7) * EPC;
    const int gr = min(m0 + r, p.M - 1);
    a_src[i] = (const T *)p.A + (size_t)gr * p.lda + k;
    a_dst[i] = r * PITCH + k;
  }
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = tid + i * NT;
    const int r = c >> 3, k = (c & 7) * EPC;
    b_src[i] = b_row<W, EPI>(p, n0 + r) + k;
    b_dst[i] = (BM + r) * PITCH + k;
  }

  Chunk16 ra[A_CH], rb[B_CH];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) ra[i] = ld16(a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < B_CH; ++i) rb[i] = ld16(b_src[i] + k0);
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) st16(&smem[buf][a_dst[i]], ra[i]);
#pragma unroll
    for (int i = 0; i < B_CH; ++i) st16(&smem[buf][b_dst[i]], to_operand<W>(rb[i]));
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){};

  const int nk = p.K / BK;
  fetch(0);
  stash(0);
  __syncthreads();

  const int frag_row = lane & 31;
  const int frag_k = (lane >> 5) * 8;
  for (int kb = 0; kb < nk; ++kb) {
    const int cur = kb & 1;
    // Prefetch the next stage (the last iteration re-reads the final stage into the
    // idle buffer: a branch-free loop keeps the prefetch registers out of scratch).
    fetch(min(kb + 1, nk - 1) * BK);
    const T *sa = &smem[cur][(wm * 32 * TM + frag_row) * PITCH + frag_k];
    const T *sb = &smem[cur][(BM + wn * 32 * TN + frag_row) * PITCH + frag_k];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      Frag<T> fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) load_frag(fa[i], sa + i * 32 * PITCH + s * 16);
#pragma unroll
      for (int j = 0; j < TN; ++j) load_frag(fb[j], sb + j * 32 * PITCH + s * 16);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mma_32x32x16(acc[i][j], fa[i], fb[j]);
    }
    stash(cur ^ 1);
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogue
  const int col_in_tile = lane & 31;
  const int wrow0 = m0 + wm * 32 * TM;
  const int wcol0 = n0 + wn * 32 * TN;

  if constexpr (EPI == EPI_STORE) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wrow0 + i * 32 + acc_row(r, lane);
        if (row >= p.M) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = wcol0 + j * 32 + col_in_tile;
          if (p.c_f32)
            ((float *)p.C)[(size_t)row * p.ldc + col] = acc[i][j][r];
          else
            ((W *)p.C)[(size_t)row * p.ldc + col] = from_f32<W>(acc[i][j][r]);
        }
      }
  } else if constexpr (EPI == EPI_RESIDUAL) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wrow0 + i * 32 + acc_row(r, lane);
        if (row >= p.M) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          float *x = (float *)p.C + (size_t)row * p.ldc + wcol0 + j * 32 + col_in_tile;
          *x = *x + acc[i][j][r];
        }
      }
  } else if constexpr (EPI == EPI_SWIGLU) {
    static_assert(TN % 2 == 0, "gate/up pairs");
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wrow0 + i * 32 + acc_row(r, lane);
        if (row >= p.M) continue;
#pragma unroll
        for (int j = 0; j < TN; j += 2) {
          const int n = wcol0 + j * 32;             // logical column of the gate tile (multiple of 64)
          const int col = (n >> 1) + col_in_tile;   // output column
          const float g = acc[i][j][r], u = acc[i][j + 1][r];
          ((T *)p.C)[(size_t)row * p.ldc + col] = from_f32<T>(silu(g) * u);
        }
      }
  } else if constexpr (EPI == EPI_QKV_ROPE) {
    // The wave's 32*TN columns are one head (TN*32 == head_dim): column e and e + d/2
    // sit in tiles j and j + TN/2 of the same lane.
    constexpr int HALF = TN / 2;
    const int D = 32 * TN;
    int kind, head;  // 0 = q, 1 = k, 2 = v
    if (wcol0 < p.nq_cols) {
      kind = 0;
      head = wcol0 / D;
    } else if (wcol0 < p.nq_cols + p.nkv_cols) {
      kind = 1;
      head = (wcol0 - p.nq_cols) / D;
    } else {
      kind = 2;
      head = (wcol0 - p.nq_cols - p.nkv_cols) / D;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wrow0 + i * 32 + acc_row(r, lane);
        if (row >= p.M) continue;
        int b, pos, idx;
        bool valid = true;
        if (p.cache_len) {
          b = row;
          pos = p.cache_len[b];
          idx = pos;
          valid = pos >= 0 && pos < p.cap && pos < p.max_pos;
        } else {
          b = row / p.seq;
          pos = p.pos0 + (row - b * p.seq);
          idx = pos - p.kv_off;
        }
        float z[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) z[j] = acc[i][j][r];
        if (kind != 2) {
#pragma unroll
          for (int j = 0; j < HALF; ++j) {
            const int e = j * 32 + col_in_tile;
            float s, c;
            sincosf((float)pos * p.inv_freq[e], &s, &c);
            const float a = z[j], bb = z[j + HALF];
            z[j] = a * c - bb * s;
            z[j + HALF] = bb * c + a * s;
          }
        }
        if (kind == 0) {
          T *q = (T *)p.q_out + (size_t)row * p.nq_cols + head * D + col_in_tile;
#pragma unroll
          for (int j = 0; j < TN; ++j) q[j * 32] = from_f32<T>(z[j]);
        } else if (valid) {
          W *dst = (W *)(kind == 1 ? p.k_out : p.v_out) +
                   (((size_t)b * p.n_kv + head) * p.cap + idx) * D + col_in_tile;
#pragma unroll
          for (int j = 0; j < TN; ++j) dst[j * 32] = from_f32<W>(z[j]);
        }
      }
  }
}

// ---------------------------------------------------------------- launchers

template <typename W, int TM, int TN, int WM, int WN, int EPI>
static hipError_t launch_cfg(const GemmParams &p, hipStream_t s) {
  constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
  if (p.N % BN != 0) return hipErrorInvalidValue;
  const int tiles = ((p.M + BM - 1) / BM) * (p.N / BN);
  hipLaunchKernelGGL((gemm_kernel<W, TM, TN, WM, WN, EPI>), dim3(tiles), dim3(64 * WM * WN), 0, s, p);
  return hipGetLastError();
}

// Tile choice: 128x128 when N allows it and the grid still fills the chip, else
// narrower tiles; the QKV epilogue needs the wave's N extent to equal head_dim.
template <typename T, int EPI>
static hipError_t launch_gemm(const GemmParams &p, hipStream_t s) {
  if constexpr (EPI == EPI_QKV_ROPE) {
    if (p.head_dim == 64) {
      if (p.M <= 64) return launch_cfg<T, 1, 2, 1, 1, EPI>(p, s);
      return launch_cfg<T, 2, 2, 2, 1, EPI>(p, s);
    }
    if (p.M <= 64) return launch_cfg<T, 1, 4, 1, 1, EPI>(p, s);
    return launch_cfg<T, 2, 4, 2, 1, EPI>(p, s);
  } else {
    const long big_tiles = (long)((p.M + 127) / 128) * (p.N / 128);
    if (p.N % 128 == 0 && p.M > 64 && big_tiles >= 256) return launch_cfg<T, 2, 2, 2, 2, EPI>(p, s);
    if (p.M <= 64) return launch_cfg<T, 1, 2, 2, 1, EPI>(p, s);
    return launch_cfg<T, 2, 2, 2, 1, EPI>(p, s);
  }
}

template <typename T>
hipError_t gemm_store(const Act<T> *A, const T *B, int M, int N, int K, void *C, int c_f32, hipStream_t s) {
  GemmParams p{};
  p.A = A; p.lda = K; p.B0 = B; p.M = M; p.N = N; p.K = K; p.C = C; p.ldc = N; p.c_f32 = c_f32;
  return launch_gemm<T, EPI_STORE>(p, s);
}

template <typename T>
hipError_t gemm_residual(const Act<T> *A, const T *B, int M, int N, int K, float *X, hipStream_t s) {
  GemmParams p{};
  p.A = A; p.lda = K; p.B0 = B; p.M = M; p.N = N; p.K = K; p.C = X; p.ldc = N;
  return launch_gemm<T, EPI_RESIDUAL>(p, s);
}

template <typename T>
hipError_t gemm_swiglu(const Act<T> *A, const T *Wg, const T *Wu, int M, int I, int K, Act<T> *Y, hipStream_t s) {
  GemmParams p{};
  p.A = A; p.lda = K; p.B0 = Wg; p.B1 = Wu; p.M = M; p.N = 2 * I; p.K = K; p.C = Y; p.ldc = I;
  return launch_gemm<T, EPI_SWIGLU>(p, s);
}

template <typename T>
hipError_t gemm_qkv_rope(const Act<T> *A, const T *Wq, const T *Wk, const T *Wv, const QkvOut &o, hipStream_t s) {
  GemmParams p{};
  p.A = A; p.lda = o.hidden; p.B0 = Wq; p.B1 = Wk; p.B2 = Wv;
  p.M = o.M; p.N = o.nq_cols + 2 * o.nkv_cols; p.K = o.hidden;
  p.nq_cols = o.nq_cols; p.nkv_cols = o.nkv_cols; p.head_dim = o.head_dim;
  p.q_out = o.q; p.k_out = o.k; p.v_out = o.v;
  p.seq = o.seq; p.cap = o.cap; p.n_kv = o.n_kv; p.pos0 = o.pos0; p.kv_off = o.kv_off; p.max_pos = o.max_pos;
  p.cache_len = o.cache_len;
  for (int i = 0; i < o.head_dim / 2 && i < 64; ++i) p.inv_freq[i] = o.inv_freq[i];
  return launch_gemm<T, EPI_QKV_ROPE>(p, s);
}

#define SMOL_INST(T)                                                                                           \
  template hipError_t gemm_store<T>(const Act<T> *, const T *, int, int, int, void *, int, hipStream_t);        \
  template hipError_t gemm_residual<T>(const Act<T> *, const T *, int, int, int, float *, hipStream_t);          \
  template hipError_t gemm_swiglu<T>(const Act<T> *, const T *, const T *, int, int, int, Act<T> *, hipStream_t); \
  template hipError_t gemm_qkv_rope<T>(const Act<T> *, const T *, const T *, const T *, const QkvOut &, hipStream_t);
SMOL_INST(float)
SMOL_INST(bf16)

}  // namespace smol
