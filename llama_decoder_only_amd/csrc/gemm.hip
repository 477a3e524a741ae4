// MFMA GEMM  C[M, N] = A[M, K] . B[N, K]^T  with fused epilogues, for gfx950.
//
// Both operands are K-contiguous (activations row-major, weights [out, in] as the
// linear layers store them), so every lane reads 8 consecutive K values of one
// row for a 32x32x16 MFMA step. Weight rows arrive in the storage type W and are
// converted to the activations' operand type Act<W> as their fragments leave LDS.
//
// A workgroup of four waves (2 x 2) owns a BM x BN tile; K is staged through an
// S-deep ring of LDS stages, 128 bytes per row each, filled by direct global->LDS
// copies (no register staging) that run S-1 stages ahead of the MFMAs; one barrier
// per stage hands a filled slot to all waves and frees the slot just consumed.
// Weight fragments are converted from W to the operand type as they leave LDS.
// When the K loop ends, the
// float accumulators go to LDS (reusing the staging buffers) and the epilogue
// walks the tile row-major, so every global write is a contiguous 8- or 16-byte
// vector and each epilogue sees whole rows of the tile:
//   EPI_STORE     C = acc                          lm_head logits
//   EPI_RESIDUAL  X += acc (float X)               o_proj / down_proj + residual
//   EPI_SWIGLU    Y = silu(gate) * up              gate/up projection: tile columns
//                                                  [0, BN/2) read gate rows and
//                                                  [BN/2, BN) the matching up rows
//   EPI_QKV_ROPE  q, k rotated at their position, q stored [M, n_heads*d]; k, v
//                 stored into the [B, n_kv, cap, d] cache at their index.
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

// Source row of logical B column n.
template <typename W, int EPI, int BN>
__device__ __forceinline__ const W *b_row(const GemmParams &p, int n) {
  if constexpr (EPI == EPI_SWIGLU) {
    constexpr int HB = BN / 2;
    const int c = n % BN;
    const int r = (n / BN) * HB + (c % HB);
    return (c < HB ? (const W *)p.B0 : (const W *)p.B1) + (size_t)r * p.K;
  } else if constexpr (EPI == EPI_QKV_ROPE) {
    if (n < p.nq_cols) return (const W *)p.B0 + (size_t)n * p.K;
    n -= p.nq_cols;
    if (n < p.nkv_cols) return (const W *)p.B1 + (size_t)n * p.K;
    return (const W *)p.B2 + (size_t)(n - p.nkv_cols) * p.K;
  } else {
    return (const W *)p.B0 + (size_t)n * p.K;
  }
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// 1 = column ownership per XCD, 2 = row ownership, 0 = plain order.
__host__ __device__ inline int xcd_mode(int M, int N, int BN) {
  if (N > M && N / BN >= SMOL_XCDS) return 1;
  if (xcd_rows(M)) return 2;
  return 0;
}

// Store N (4 or 8) consecutive floats as type O.
template <typename O, int N>
__device__ __forceinline__ void store_vec(O *dst, const float *v) {
  if constexpr (sizeof(O) == 2 && N == 8) {
    Chunk16 c;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      c[i] = (uint32_t)__builtin_bit_cast(uint16_t, from_f32<O>(v[2 * i])) |
             ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<O>(v[2 * i + 1])) << 16);
    st16(dst, c);
  } else if constexpr (sizeof(O) == 2 && N == 4) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    u32x2 c;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      c[i] = (uint32_t)__builtin_bit_cast(uint16_t, from_f32<O>(v[2 * i])) |
             ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<O>(v[2 * i + 1])) << 16);
    *reinterpret_cast<u32x2 *>(dst) = c;
  } else {
    static_assert(sizeof(O) == 4, "float output");
#pragma unroll
    for (int i = 0; i < N; i += 4)
      *reinterpret_cast<f32x4 *>((float *)dst + i) = (f32x4){v[i], v[i + 1], v[i + 2], v[i + 3]};
  }
}

// Fragment of 8 consecutive K values of one row from a swizzled LDS stage row:
// 16-byte chunk c of row r sits at slot c ^ (r & 7) (see gemm_kernel).
template <typename T>
__device__ __forceinline__ Chunk16 lds_chunk(const char *row, int c, int sw) {
  return *reinterpret_cast<const Chunk16 *>(row + ((c ^ sw) << 4));
}

template <typename W, int BM, int BN, int EPI, int S>
__global__ void __launch_bounds__(256)
gemm_kernel(const GemmParams p) {
  using T = Act<W>;  // MFMA operand type; weight fragments convert from W as they are read
  static_assert(sizeof(T) == sizeof(W), "storage and operand types have the same width");
  constexpr int NT = 256;
  constexpr int TM = BM / 64, TN = BN / 64;  // 32x32 MFMA tiles per wave (2 x 2 waves)
  constexpr int ROWS = BM + BN;              // LDS rows per stage: A rows, then B rows
  constexpr int STAGE_BYTES = ROWS * 128;    // 128 bytes of K per row per stage
  constexpr int IPW = ROWS / 32;             // DMA instructions per wave per stage (8 rows each)
  constexpr int KE = 128 / sizeof(T);        // K elements per stage
  constexpr int KSTEPS = KE / 16;
  constexpr int CPF = 16 * sizeof(T) / 16 / 2;  // 16-byte chunks per 8-element fragment (1 or 2)
  constexpr int OP = BN + 4;                 // float pitch of the epilogue tile
  // The epilogue walks the tile in row chunks of ER rows that fit the staging LDS.
  constexpr int ER = (BM * OP * 4 <= S * STAGE_BYTES) ? BM : 32 * TM;
  static_assert(ER * OP * 4 <= S * STAGE_BYTES, "epilogue chunk must fit the staging LDS");
  static_assert(S >= 2, "at least double buffering");

  __shared__ __attribute__((aligned(16))) char smem[S * STAGE_BYTES];
  float *tile = reinterpret_cast<float *>(smem);
  const uint32_t smem_base = lds_addr(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // XCD-aware tile order (workgroup i runs on XCD i % 8; each XCD has its own L2
  // and whatever misses it streams at roughly HBM rate). Column ownership when the
  // weights outweigh the activations (N > M): XCD x takes a contiguous slice of N
  // tiles, so every weight byte is fetched by one XCD only. Otherwise row
  // ownership (see xcd_rows): XCD x takes the M tiles of its row range. Within an
  // XCD, M runs fastest so that concurrent workgroups share a weight tile.
  int tm, tn;
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = p.N / BN;
  const int local = blockIdx.x / SMOL_XCDS, xcd = blockIdx.x % SMOL_XCDS;
  switch (xcd_mode(p.M, p.N, BN)) {
    case 1: {  // columns
      const int ntx = (tiles_n + SMOL_XCDS - 1) / SMOL_XCDS;
      tm = local % tiles_m;
      tn = xcd * ntx + local / tiles_m;
      if (tn >= tiles_n) return;  // whole workgroup
      break;
    }
    case 2: {  // rows
      const int mtx = rows_per_xcd(p.M) / BM;
      tm = xcd * mtx + local % mtx;
      tn = local / mtx;
      if (tm >= tiles_m) return;  // whole workgroup
      break;
    }
    default:
      tm = blockIdx.x % tiles_m;
      tn = blockIdx.x / tiles_m;
  }
  const int m0 = tm * BM, n0 = tn * BN;

  // DMA sources. Wave w's instruction j fills rows 8*(w*IPW + j) .. +7 of a stage;
  // lane l writes slot l % 8 of row 8*(..) + l / 8 and so fetches the row's 16-byte
  // chunk (l % 8) ^ (row & 7): an XOR swizzle that keeps fragment reads (32 rows,
  // one chunk each) free of bank conflicts without padding.
  const char *src[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int r = 8 * (wave * IPW + j) + (lane >> 3);
    const int c = (lane & 7) ^ (r & 7);
    if (r < BM)
      src[j] = (const char *)((const T *)p.A + (size_t)min(m0 + r, p.M - 1) * p.lda) + c * 16;
    else
      src[j] = (const char *)b_row<W, EPI, BN>(p, n0 + r - BM) + c * 16;
  }
  auto issue = [&](int stage, int slot) {
#pragma unroll
    for (int j = 0; j < IPW; ++j)
      lds_dma16(src[j] + stage * 128, smem_base + slot * STAGE_BYTES + (8 * (wave * IPW + j)) * 128);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){};

  const int nk = p.K / KE;
#pragma unroll
  for (int st = 0; st < S - 1; ++st)
    if (st < nk) issue(st, st);

  const int sw = lane & 7;  // row & 7 for every fragment row this lane reads
  const int half = lane >> 5;
  for (int kb = 0; kb < nk; ++kb) {
    // stage kb has landed (for this wave) once at most S-2 later stages are pending
    if (kb + S - 2 < nk)
      wait_vmcnt<(S - 2) * IPW>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();  // ... and for every wave; also all reads of stage kb-1 are done
    if (kb + S - 1 < nk) issue(kb + S - 1, (kb + S - 1) % S);  // refill the slot of stage kb-1
    const char *sa = smem + (kb % S) * STAGE_BYTES + (wm * 32 * TM + (lane & 31)) * 128;
    const char *sb = smem + (kb % S) * STAGE_BYTES + (BM + wn * 32 * TN + (lane & 31)) * 128;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      Frag<T> fa[TM], fb[TN];
      const int c0 = (2 * s + half) * CPF;  // first chunk of this lane's 8 K values
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const char *row = sa + i * 32 * 128;
        if constexpr (CPF == 1) {
          const Chunk16 c = lds_chunk<T>(row, c0, sw);
          fa[i].v = __builtin_bit_cast(decltype(fa[i].v), c);
        } else {
          const Chunk16 lo = lds_chunk<T>(row, c0, sw), hi = lds_chunk<T>(row, c0 + 1, sw);
          fa[i].v = (f32x8){__uint_as_float(lo[0]), __uint_as_float(lo[1]), __uint_as_float(lo[2]), __uint_as_float(lo[3]),
                            __uint_as_float(hi[0]), __uint_as_float(hi[1]), __uint_as_float(hi[2]), __uint_as_float(hi[3])};
        }
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const char *row = sb + j * 32 * 128;
        if constexpr (CPF == 1) {
          const Chunk16 c = to_operand<W>(lds_chunk<W>(row, c0, sw));
          fb[j].v = __builtin_bit_cast(decltype(fb[j].v), c);
        } else {
          const Chunk16 lo = lds_chunk<W>(row, c0, sw), hi = lds_chunk<W>(row, c0 + 1, sw);
          fb[j].v = (f32x8){__uint_as_float(lo[0]), __uint_as_float(lo[1]), __uint_as_float(lo[2]), __uint_as_float(lo[3]),
                            __uint_as_float(hi[0]), __uint_as_float(hi[1]), __uint_as_float(hi[2]), __uint_as_float(hi[3])};
        }
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mma_32x32x16(acc[i][j], fa[i], fb[j]);
    }
  }
  __syncthreads();  // every wave is done reading the stages: the epilogue tile reuses them

  // ------------------------------------------------------------ accumulators -> LDS
  // Row chunk ec holds tile rows [ec*ER, ec*ER + ER): the waves whose rows fall in it
  // write their accumulators, then the epilogue walks those rows.
#pragma unroll
  for (int ec = 0; ec < BM / ER; ++ec) {
    const int r_lo = ec * ER;
    if (ER == BM || wm == ec) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            tile[(wm * 32 * TM + i * 32 + acc_row(r, lane) - r_lo) * OP + wn * 32 * TN + j * 32 + (lane & 31)] =
                acc[i][j][r];
    }
    __syncthreads();
    const int em0 = m0 + r_lo;  // first global row of this chunk

    // ------------------------------------------------------------ epilogue (row-major walk)
    if constexpr (EPI == EPI_STORE) {
      if (p.c_f32 || sizeof(W) == 4) {
        constexpr int V = 4;
        for (int it = tid; it < ER * BN / V; it += NT) {
          const int r = it / (BN / V), c = (it % (BN / V)) * V;
          if (em0 + r >= p.M) continue;
          store_vec<float, V>((float *)p.C + (size_t)(em0 + r) * p.ldc + n0 + c, &tile[r * OP + c]);
        }
      } else {
        constexpr int V = 8;
        for (int it = tid; it < ER * BN / V; it += NT) {
          const int r = it / (BN / V), c = (it % (BN / V)) * V;
          if (em0 + r >= p.M) continue;
          if constexpr (sizeof(W) == 2) store_vec<W, V>((W *)p.C + (size_t)(em0 + r) * p.ldc + n0 + c, &tile[r * OP + c]);
        }
      }
    } else if constexpr (EPI == EPI_RESIDUAL) {
      constexpr int V = 4;
      for (int it = tid; it < ER * BN / V; it += NT) {
        const int r = it / (BN / V), c = (it % (BN / V)) * V;
        if (em0 + r >= p.M) continue;
        f32x4 *x = reinterpret_cast<f32x4 *>((float *)p.C + (size_t)(em0 + r) * p.ldc + n0 + c);
        const f32x4 t = *reinterpret_cast<const f32x4 *>(&tile[r * OP + c]);
        *x = *x + t;
      }
    } else if constexpr (EPI == EPI_SWIGLU) {
      constexpr int HB = BN / 2;
      constexpr int V = 16 / sizeof(T);
      static_assert(HB % V == 0, "output row segment");
      for (int it = tid; it < ER * HB / V; it += NT) {
        const int r = it / (HB / V), c = (it % (HB / V)) * V;
        if (em0 + r >= p.M) continue;
        float y[V];
  #pragma unroll
        for (int e = 0; e < V; ++e) y[e] = silu(tile[r * OP + c + e]) * tile[r * OP + HB + c + e];
        store_vec<T, V>((T *)p.C + (size_t)(em0 + r) * p.ldc + n0 / 2 + c, y);
      }
    } else if constexpr (EPI == EPI_QKV_ROPE) {
      // Items: (row, head within the tile, 4 consecutive dims e0.. of the first half);
      // each item rotates the pairs (e, e + d/2) for its 4 dims.
      const int D = p.head_dim, HALF = D / 2;
      const int heads = BN / D;
      const int per_row = heads * (HALF / 4);
      for (int it = tid; it < ER * per_row; it += NT) {
        const int r = it / per_row, rem = it % per_row;
        const int hi = rem / (HALF / 4), e0 = (rem % (HALF / 4)) * 4;
        const int row = em0 + r;
        if (row >= p.M) continue;
        const int ncol = n0 + hi * D;  // first column of this head
        int kind, head;                // 0 = q, 1 = k, 2 = v
        if (ncol < p.nq_cols) {
          kind = 0;
          head = ncol / D;
        } else if (ncol < p.nq_cols + p.nkv_cols) {
          kind = 1;
          head = (ncol - p.nq_cols) / D;
        } else {
          kind = 2;
          head = (ncol - p.nq_cols - p.nkv_cols) / D;
        }
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
        const float *t = &tile[r * OP + hi * D];
        float lo[4], up[4];
  #pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = t[e0 + e];
          up[e] = t[HALF + e0 + e];
        }
        if (kind != 2) {
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            float s, c;
            sincosf((float)pos * p.inv_freq[e0 + e], &s, &c);
            const float a = lo[e], bb = up[e];
            lo[e] = a * c - bb * s;
            up[e] = bb * c + a * s;
          }
        }
        if (kind == 0) {
          T *q = (T *)p.q_out + (size_t)row * p.nq_cols + head * D;
          store_vec<T, 4>(q + e0, lo);
          store_vec<T, 4>(q + HALF + e0, up);
        } else if (valid) {
          W *dst = (W *)(kind == 1 ? p.k_out : p.v_out) + (((size_t)b * p.n_kv + head) * p.cap + idx) * D;
          store_vec<W, 4>(dst + e0, lo);
          store_vec<W, 4>(dst + HALF + e0, up);
        }
      }
    }
    __syncthreads();  // the next chunk overwrites the tile
  }
}

// ---------------------------------------------------------------- launchers

template <typename W, int BM, int BN, int EPI, int S>
static hipError_t launch_cfg(const GemmParams &p, hipStream_t s) {
  if (p.N % BN != 0 || p.K % (128 / (int)sizeof(W)) != 0) return hipErrorInvalidValue;
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = p.N / BN;
  int tiles;
  switch (xcd_mode(p.M, p.N, BN)) {
    case 1: tiles = SMOL_XCDS * ((tiles_n + SMOL_XCDS - 1) / SMOL_XCDS) * tiles_m; break;
    case 2: tiles = SMOL_XCDS * (rows_per_xcd(p.M) / BM) * tiles_n; break;
    default: tiles = tiles_m * tiles_n;
  }
  hipLaunchKernelGGL((gemm_kernel<W, BM, BN, EPI, S>), dim3(tiles), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Tile choice (measured on MI355X over the model's shapes: a 2-stage ring was never
// slower than 3 or 4 stages): 128 x 128 when that still gives >= 2 workgroups per
// CU (lm_head), else 128 x 64 under the same rule (gate/up), else 64 x 64 for
// parallelism on small N (o_proj, down, QKV, every decode GEMM); 64 x 128 when a
// 128-wide head must stay in one tile for RoPE.
template <typename T, int EPI>
static hipError_t launch_gemm(const GemmParams &p, hipStream_t s) {
  const long tm128 = (p.M + 127) / 128;
  const long t128 = (p.N % 128 == 0) ? tm128 * (p.N / 128) : 0;
  if (t128 >= 512) return launch_cfg<T, 128, 128, EPI, 2>(p, s);
  if (EPI == EPI_QKV_ROPE && p.head_dim == 128) return launch_cfg<T, 64, 128, EPI, 2>(p, s);
  if (tm128 * (p.N / 64) >= 512) return launch_cfg<T, 128, 64, EPI, 2>(p, s);
  return launch_cfg<T, 64, 64, EPI, 2>(p, s);
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
