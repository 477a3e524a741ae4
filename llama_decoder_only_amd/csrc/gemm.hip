// MFMA GEMM  C[M, N] = A[M, K] . B[N, K]^T  with fused epilogues, for gfx950.
//
// Both operands are K-contiguous (activations row-major, weights [out, in] as the
// linear layers store them), so every lane reads 8 consecutive K values of one
// row for a 32x32x16 MFMA step. Weight rows arrive in the storage type W and are
// converted to the activations' operand type Act<W> as their fragments leave LDS.
//
// A workgroup owns a BM x BN tile, computed by WM x WN waves, times KW groups of
// waves that split each stage's K steps between them (more waves per SIMD to hide
// the LDS -> convert -> MFMA chain when the grid is small; their partial sums are
// added in a fixed order at the end). K is staged through an S-deep ring of LDS
// stages (128 bytes of weights per row each), filled by direct global->LDS copies
// (no register staging) that run S-1 stages ahead of the MFMAs; one barrier per
// stage hands a filled slot to all waves and frees the slot just consumed.
//
// RMSNorm, deferred (u = w * x * r with r = 1 / sqrt(mean(x^2) + eps) per row,
// abi96062 components.py, RMSNorm). A residual epilogue, which holds the updated
// rows x only one BN-column slice at a time, cannot know r yet; it stores
// xs = w_next * x * r_old * 2^-8, with r_old the row's r before this update (the
// fixed 2^-8 leaves float16 room for a row whose rms grows several thousand times in
// one update; common.h, SMOL_XS_SCALE), plus the row's sums of squares per 64
// columns. The GEMM that reads xs as A then scales each output row by r / r_old * 2^8,
// both taken from those partial sums, which makes its result u B^T up to the one
// rounding of xs.
//
// When the K loop ends, the float accumulators go to LDS (reusing the staging
// buffers) and the epilogue walks the tile row-major, so every global write is a
// contiguous 8- or 16-byte vector and each epilogue sees whole rows of the tile:
//   EPI_STORE     C = acc                          lm_head logits
//   EPI_RESIDUAL  X += acc (float X)               o_proj / down_proj + residual; also
//                                                  xs and the new sums of squares for
//                                                  the next norm
//   EPI_SWIGLU    Y = silu(gate) * up              gate/up projection: tile columns
//                                                  [0, BN/2) read gate rows and
//                                                  [BN/2, BN) the matching up rows
//   EPI_QKV_ROPE  q, k rotated at their position (not on a NoPE block), q stored
//                 [M, n_heads*d]; k, v
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
  const float2 *rope;  // [M, head_dim / 2] (cos, sin) of each row's RoPE angles
  int rope_on;         // 0: a NoPE block, q and k are stored as projected
  // Row sums of squares of the residual stream, H/64 partials per row:
  // ss[j * M + row] over columns [64 j, 64 j + 64).
  //   A GEMM on xs (EPI != EPI_RESIDUAL, ss_new != nullptr): output row scaled by
  //   r(ss_new) / r(ss_old).
  //   EPI_RESIDUAL: writes ss_new of the updated X when ss_new != nullptr, and, when
  //   xs != nullptr, xs = norm_w * X * r(ss_old).
  const float *ss_old;
  float *ss_new;
  const void *norm_w;
  void *xs;
  int ss_cols;  // H
  float eps;
  // K split (EPI_SPLIT): ksplit workgroups per tile, each over K / ksplit; split i
  // writes its unscaled partial sums to part[i * M * N + row * N + col].
  int ksplit;
  float *part;
};

// r = 1 / sqrt(mean(x^2) + eps) of one row from its H/64 partial sums of squares,
// added in part order (16 loads in flight per round; indices clamped in bounds and
// the extras masked out of the sum).
__device__ __forceinline__ float row_r(const float *ss, int M, int row, int H, float eps) {
  const int parts = H / 64;
  float q = 0.f;
  for (int q0 = 0; q0 < parts; q0 += 16) {
    float v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = ss[(size_t)min(q0 + e, parts - 1) * M + row];
#pragma unroll
    for (int e = 0; e < 16; ++e) q += (q0 + e < parts) ? v[e] : 0.f;
  }
  return 1.0f / sqrtf(q / (float)H + eps);
}

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

// Position of GEMM row `row` in the QKV epilogue: cache_len[row] in a decode step
// (one row per sequence), else pos0 + the row's index within its sequence.
__device__ __forceinline__ int qkv_pos(const GemmParams &p, int row) {
  return p.cache_len ? p.cache_len[row] : p.pos0 + row % p.seq;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// 1 = column ownership per XCD, 2 = row ownership, 0 = plain order.
//
// The choice goes by an estimate of the bytes each mode fetches from beyond the
// XCDs' L2 caches (4 MB each; an operand of up to 3 MB is taken to stay resident
// while the XCD walks its tiles). Column ownership: every XCD reads its eighth of
// the weights once and the whole activation A, once if A stays resident, else once
// per column tile of its slice (its resident workgroups walk M fastest). Row
// ownership: every XCD reads the whole weight matrix and its eighth of A, once if
// that stays resident, else once per round of the columns its ~32 resident
// workgroups cover together. At batch 4 x seq 512 the lm_head keeps column ownership
// (A 2.4 MB: 75 MB against 455 MB); at 8192 rows it takes row ownership, as does
// the SmolLM3-3B-shaped gate/up (1.1 GB against 3.0 GB). Measured against column
// ownership for those three: lm_head at batch 1 x seq 8192 656 -> 605 us, the SmolLM3
// shape's gate/up 853 -> 815 us and lm_head 4.77 -> 4.57 ms. Below 1024 rows every
// XCD must get work: column ownership when N > M, else the plain order.
__host__ __device__ inline int xcd_mode(int M, int N, int K, int BM, int BN, int esz) {
  const bool col_ok = N / BN >= SMOL_XCDS;
  if (!xcd_rows(M)) return N > M && col_ok ? 1 : 0;
  if (!col_ok) return 2;
  // integers only: the host sizes the grid and the kernel maps its tiles by this same
  // decision, which must come out alike on both sides
  constexpr long long RESIDENT = 3ll << 20;
  const long long a = (long long)M * K * esz, w = (long long)N * K * esz;
  const long long tiles_n = N / BN, ntx = (tiles_n + SMOL_XCDS - 1) / SMOL_XCDS;
  const long long col = SMOL_XCDS * a * (a <= RESIDENT ? 1 : ntx) + w;
  const long long mtx = rows_per_xcd(M, BM) / BM;
  const long long cols_per_round = mtx >= 32 ? 1 : 32 / mtx;
  const long long row = a * (a / SMOL_XCDS <= RESIDENT ? 1 : (tiles_n + cols_per_round - 1) / cols_per_round) +
                        SMOL_XCDS * w;
  return col < row ? 1 : 2;
}

// A store to global memory through a global-address-space pointer: the compiler
// then emits global_store, never a flat store (the pointers here are loaded from the
// kernel's parameter struct, where it cannot infer the address space itself).
// NTS: a non-temporal store (global_store ... nt), for output that streams out and
// is not read again by the next kernels.
template <bool NTS = false, typename V>
__device__ __forceinline__ void gstore(void *dst, const V &v) {
  auto *g = reinterpret_cast<__attribute__((address_space(1))) V *>(reinterpret_cast<uintptr_t>(dst));
  if constexpr (NTS)
    __builtin_nontemporal_store(v, g);
  else
    *g = v;
}

// Store N (4 or 8) consecutive floats as type O (non-temporal with NTS).
template <typename O, int N, bool NTS = false>
__device__ __forceinline__ void store_vec(O *dst, const float *v) {
  if constexpr (sizeof(O) == 2 && N == 8) {
    Chunk16 c;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      c[i] = (uint32_t)__builtin_bit_cast(uint16_t, from_f32<O>(v[2 * i])) |
             ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<O>(v[2 * i + 1])) << 16);
    gstore<NTS>(dst, c);
  } else if constexpr (sizeof(O) == 2 && N == 4) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    u32x2 c;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      c[i] = (uint32_t)__builtin_bit_cast(uint16_t, from_f32<O>(v[2 * i])) |
             ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<O>(v[2 * i + 1])) << 16);
    gstore<NTS>(dst, c);
  } else {
    static_assert(sizeof(O) == 4, "float output");
#pragma unroll
    for (int i = 0; i < N; i += 4) gstore<NTS>((float *)dst + i, (f32x4){v[i], v[i + 1], v[i + 2], v[i + 3]});
  }
}

// XOR swizzle of a staged row with CPR 16-byte chunks: chunk c of row r sits at slot
// c ^ (r & 7). A fragment read (ds_read_b128) takes one chunk from each of 32
// consecutive rows; measured on gfx950, that pattern then runs at the conflict-free
// rate (about 9 clocks per wave instruction), while unswizzled 128-byte rows take
// four times as long.
template <int CPR>
__host__ __device__ constexpr int lds_swz(int r) {
  static_assert(CPR >= 8, "the swizzle spans 8 chunks");
  return r & 7;
}

// Fragment of 8 consecutive K values of one row from a swizzled LDS stage row:
// 16-byte chunk c of row r sits at slot c ^ lds_swz<CPR>(r) (see gemm_kernel).
template <typename T>
__device__ __forceinline__ Chunk16 lds_chunk(const char *row, int c, int sw) {
  return *reinterpret_cast<const Chunk16 *>(row + ((c ^ sw) << 4));
}

// Epilogue operands that come from memory, loaded by a kernel before its main work
// so that their latency hides under it. Items as in epilogue_rows' walks, item
// tid + k * NT for k < XPI (QPI). Residual: the thread's X values (4 floats an item)
// and, when scaled, the norm weights of those columns. QKV: the RoPE (cos, sin) of
// the item's 4 frequencies and, in a decode step, the row's position.
template <typename W, int BN, int NT, int XPI>
__device__ __forceinline__ void prefetch_residual(const GemmParams &p, int m0, int n0, int tid, bool scaled,
                                                  f32x4 *xpre, float (*wpre)[4]) {
#pragma unroll
  for (int k = 0; k < XPI; ++k) {
    const int it = tid + k * NT;
    const int r = it / (BN / 4), c = (it % (BN / 4)) * 4;
    xpre[k] = *reinterpret_cast<const f32x4 *>((const float *)p.C + (size_t)min(m0 + r, p.M - 1) * p.ldc + n0 + c);
    if (scaled) {
#pragma unroll
      for (int e = 0; e < 4; ++e) wpre[k][e] = to_f32(((const W *)p.norm_w)[n0 + c + e]);
    }
  }
}
template <int BN, int NT, int QPI>
__device__ __forceinline__ void prefetch_qkv(const GemmParams &p, int m0, int tid, f32x4 (*cspre)[2], int *pospre) {
  const int HALF = p.head_dim / 2, per_row = BN / 8;
#pragma unroll
  for (int k = 0; k < QPI; ++k) {
    const int it = tid + k * NT;
    const int r = it / per_row, e0 = ((it % per_row) % (HALF / 4)) * 4;
    const int row = min(m0 + r, p.M - 1);
    const f32x4 *cs = reinterpret_cast<const f32x4 *>(p.rope + (size_t)row * HALF + e0);
    cspre[k][0] = cs[0];
    cspre[k][1] = cs[1];
    pospre[k] = p.cache_len ? p.cache_len[row] : 0;
  }
}

// Deferred-RMSNorm factor of one row: r_old * 2^-8 for a residual epilogue (it
// scales xs, stored at SMOL_XS_SCALE), r(ss_new) / r(ss_old) * 2^8 for a GEMM that
// reads xs.
template <int EPI>
__device__ __forceinline__ float row_factor(const GemmParams &p, int row) {
  const float r_old = row_r(p.ss_old, p.M, row, p.ss_cols, p.eps);
  return EPI == EPI_RESIDUAL ? r_old * SMOL_XS_SCALE
                             : row_r(p.ss_new, p.M, row, p.ss_cols, p.eps) / r_old * SMOL_XS_UNSCALE;
}

// The epilogue of ER rows of a tile, from the float accumulator sums in LDS (tile,
// pitch OP, row r at tile + r * OP): em0 is the global row of tile row 0, n0 the
// tile's first column, srow[r] the row's deferred-RMSNorm factor (read only when
// scaled). XPI > 0 / QPI > 0: the residual / QKV operands from memory were
// prefetched into xpre, wpre / cspre, pospre, XPI / QPI items per thread.
template <typename W, int BN, int EPI, int NT, int ER, int OP, int XPI, int QPI>
__device__ __forceinline__ void epilogue_rows(const GemmParams &p, const float *tile, const float *srow, bool scaled,
                                              int em0, int n0, int tid, const f32x4 *xpre, const float (*wpre)[4],
                                              const f32x4 (*cspre)[2], const int *pospre) {
  using T = Act<W>;
  // deferred-RMSNorm factor of tile row r of this chunk (1 when not scaled)
  auto rowf = [&](int r) { return (EPI != EPI_RESIDUAL && scaled) ? srow[r] : 1.0f; };

  // ------------------------------------------------------------ epilogue (row-major walk)
  if constexpr (EPI == EPI_STORE) {
    // Logits stream out (201 MB at batch 4 x seq 512) and nothing here reads them
    // again: non-temporal stores keep them from displacing the weights in MALL, which
    // the next prefill reads again (measured: prefill step 2.33 -> 2.20 ms).
    if (p.c_f32 || sizeof(W) == 4) {
      constexpr int V = 4;
      for (int it = tid; it < ER * BN / V; it += NT) {
        const int r = it / (BN / V), c = (it % (BN / V)) * V;
        if (em0 + r >= p.M) continue;
        const float f = rowf(r);
        float v[V];
#pragma unroll
        for (int e = 0; e < V; ++e) v[e] = tile[r * OP + c + e] * f;
        store_vec<float, V, true>((float *)p.C + (size_t)(em0 + r) * p.ldc + n0 + c, v);
      }
    } else {
      constexpr int V = 8;
      for (int it = tid; it < ER * BN / V; it += NT) {
        const int r = it / (BN / V), c = (it % (BN / V)) * V;
        if (em0 + r >= p.M) continue;
        const float f = rowf(r);
        float v[V];
#pragma unroll
        for (int e = 0; e < V; ++e) v[e] = tile[r * OP + c + e] * f;
        if constexpr (sizeof(W) == 2) store_vec<W, V, true>((W *)p.C + (size_t)(em0 + r) * p.ldc + n0 + c, v);
      }
    }
  } else if constexpr (EPI == EPI_RESIDUAL) {
    constexpr int V = 4;
    auto item = [&](int it, const f32x4 *pre, const float *wp) {
      const int r = it / (BN / V), c = (it % (BN / V)) * V;
      if (em0 + r >= p.M) return;
      const int row = em0 + r, col = n0 + c;
      f32x4 *x = reinterpret_cast<f32x4 *>((float *)p.C + (size_t)row * p.ldc + col);
      const f32x4 t = *reinterpret_cast<const f32x4 *>(&tile[r * OP + c]);
      const f32x4 xn = (pre ? *pre : *x) + t;
      *x = xn;
      if (p.ss_new) {
        // the 16 consecutive items (lanes) of one 64-column segment of a row
        float q = xn[0] * xn[0] + xn[1] * xn[1] + xn[2] * xn[2] + xn[3] * xn[3];
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) q += __shfl_xor(q, o, 64);
        if ((c & 63) == 0) p.ss_new[(size_t)(col >> 6) * p.M + row] = q;
      }
      if (scaled) {
        const float r_old = srow[r];
        const W *w = (const W *)p.norm_w + col;
        float v[V];
#pragma unroll
        for (int e = 0; e < V; ++e) v[e] = (wp ? wp[e] : to_f32(w[e])) * (xn[e] * r_old);
        store_vec<T, V>((T *)p.xs + (size_t)row * p.ldc + col, v);
      }
    };
    if constexpr (XPI > 0) {
#pragma unroll
      for (int k = 0; k < XPI; ++k) item(tid + k * NT, &xpre[k], wpre[k]);
    } else {
      for (int it = tid; it < ER * BN / V; it += NT) item(it, nullptr, nullptr);
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    constexpr int HB = BN / 2;
    constexpr int V = 16 / sizeof(T);
    static_assert(HB % V == 0, "output row segment");
    for (int it = tid; it < ER * HB / V; it += NT) {
      const int r = it / (HB / V), c = (it % (HB / V)) * V;
      if (em0 + r >= p.M) continue;
      const float f = rowf(r);
      float y[V];
#pragma unroll
      for (int e = 0; e < V; ++e) y[e] = silu(tile[r * OP + c + e] * f) * (tile[r * OP + HB + c + e] * f);
      store_vec<T, V>((T *)p.C + (size_t)(em0 + r) * p.ldc + n0 / 2 + c, y);
    }
  } else if constexpr (EPI == EPI_QKV_ROPE) {
    // Items: (row, head within the tile, 4 consecutive dims e0.. of the first half);
    // each item rotates the pairs (e, e + d/2) for its 4 dims. BN / 8 items a row.
    const int D = p.head_dim, HALF = D / 2;
    const int per_row = BN / 8;
    auto item = [&](int it, const f32x4 *cs_pre, int pos_pre) {
      const int r = it / per_row, rem = it % per_row;
      const int hi = rem / (HALF / 4), e0 = (rem % (HALF / 4)) * 4;
      const int row = em0 + r;
      if (row >= p.M) return;
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
      int b, idx;
      bool valid = true;
      if (p.cache_len) {
        b = row;
        idx = cs_pre ? pos_pre : p.cache_len[row];
        valid = idx >= 0 && idx < p.cap && idx < p.max_pos;
      } else {
        b = row / p.seq;
        idx = qkv_pos(p, row) - p.kv_off;
      }
      const float *t = &tile[r * OP + hi * D];
      const float f = rowf(r);
      float lo[4], up[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo[e] = t[e0 + e] * f;
        up[e] = t[HALF + e0 + e] * f;
      }
      if (kind != 2 && p.rope_on) {
        f32x4 cs0, cs1;  // (cos, sin) of frequencies e0 .. e0 + 3
        if (cs_pre) {
          cs0 = cs_pre[0];
          cs1 = cs_pre[1];
        } else {
          const f32x4 *cs = reinterpret_cast<const f32x4 *>(p.rope + (size_t)row * HALF + e0);
          cs0 = cs[0];
          cs1 = cs[1];
        }
        const float c[4] = {cs0[0], cs0[2], cs1[0], cs1[2]}, sn[4] = {cs0[1], cs0[3], cs1[1], cs1[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = lo[e], bb = up[e];
          lo[e] = a * c[e] - bb * sn[e];
          up[e] = bb * c[e] + a * sn[e];
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
    };
    if constexpr (QPI > 0) {
#pragma unroll
      for (int k = 0; k < QPI; ++k) item(tid + k * NT, cspre[k], pospre[k]);
    } else {
      for (int it = tid; it < ER * per_row; it += NT) item(it, nullptr, 0);
    }
  }
}

template <typename W, int BM, int BN, int WM, int WN, int RB, int EPI, int S, int KW>
__global__ void __launch_bounds__(64 * WM * WN * KW)
gemm_kernel(const GemmParams p) {
  using T = Act<W>;  // MFMA operand type; weight fragments convert from W as they are read
  using TA = T;      // A element type as staged in LDS
  static_assert(sizeof(T) == sizeof(W), "storage and operand types have the same width");
  constexpr int EK = EPI & ~EPI_SPLIT;          // the epilogue; its B row order
  constexpr bool SPLIT = (EPI & EPI_SPLIT) != 0;  // K split over workgroups: partial sums out
  constexpr int NWG = WM * WN;               // waves per K group
  constexpr int NW = NWG * KW, NT = 64 * NW;
  constexpr int TM = BM / (32 * WM), TN = BN / (32 * WN);  // 32x32 MFMA tiles per wave
  static_assert(TM * 32 * WM == BM && TN * 32 * WN == BN, "wave layout must tile the block");
  constexpr int KE = RB / sizeof(W);         // K elements per stage
  constexpr int RA = KE * sizeof(TA);        // A bytes per row per stage
  constexpr int CPRA = RA / 16, CPR = RB / 16;  // 16-byte chunks per A / B row per stage
  constexpr int A_BYTES = BM * RA;           // stage layout: A rows, then B rows
  constexpr int STAGE_BYTES = A_BYTES + BN * RB;
  static_assert(A_BYTES % 1024 == 0 && (BN * RB) % 1024 == 0, "whole DMA instructions per operand");
  static_assert(CPRA >= 8 && CPR >= 8, "the XOR swizzle spans 8 chunks");
  constexpr int NINS = STAGE_BYTES / 1024;   // DMA wave-instructions per stage
  constexpr int IPW = NINS / NW;             // per wave
  static_assert(IPW * NW == NINS, "DMA instructions must split evenly over the waves");
  constexpr int KSTEPS = KE / 16;
  static_assert(KSTEPS % KW == 0, "K groups split the stage's K steps evenly");
  constexpr int CPF = sizeof(T) / 2;         // 16-byte chunks per 8-element fragment (1 or 2)
  // Waves raise their issue priority while they read fragments and issue MFMAs, so the
  // arbiter prefers the matrix work of one wave over the waits of another: the batch
  // 4 x seq 512 prefill 2.246 -> 2.214 ms (gate/up 19.1 -> 18.6 us, o_proj 11.6 -> 11.3).
  // Not on 256 x 256 tiles, where the SmolLM3-3B-shaped lm_head went 4.51 -> 4.90 ms.
  constexpr bool MFMA_PRIO = !(BM == 256 && BN == 256);
  constexpr int OP = BN + 4;                 // float pitch of the epilogue tile
  // The epilogue walks the tile in row chunks of ER rows (a multiple of 32) that fit
  // the staging LDS.
  constexpr int ER = (BM * OP * 4 <= S * STAGE_BYTES) ? BM
                     : (BM / 2 * OP * 4 <= S * STAGE_BYTES) ? BM / 2
                     : (BM / 4 * OP * 4 <= S * STAGE_BYTES) ? BM / 4 : 32;
  static_assert(ER * OP * 4 <= S * STAGE_BYTES, "epilogue chunk must fit the staging LDS");
  static_assert(S >= 2, "at least double buffering");
  static_assert((S - 2) * IPW <= 63, "vmcnt counts at most 63 outstanding loads");

  __shared__ __attribute__((aligned(16))) char smem[S * STAGE_BYTES];
  __shared__ float s_row[BM];  // per-row factor of the deferred RMSNorm (see GemmParams)
  float *tile = reinterpret_cast<float *>(smem);
  const uint32_t smem_base = lds_addr(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kw = wave / NWG;                 // K group
  const int wm = (wave % NWG) % WM, wn = (wave % NWG) / WM;

  // XCD-aware tile order (workgroup i runs on XCD i % 8; each XCD has its own L2
  // and whatever misses it streams from MALL or HBM). Column ownership: XCD x takes
  // a contiguous slice of N tiles, so every weight byte is fetched by one XCD only.
  // Row ownership: XCD x takes the M tiles of its row range (see xcd_mode for the
  // choice). Within an XCD, M runs fastest so that concurrent workgroups share a
  // weight tile.
  int tm, tn, split = 0;
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = p.N / BN;
  const int local = blockIdx.x / SMOL_XCDS, xcd = blockIdx.x % SMOL_XCDS;
  // K split (a grid of a few tiles): workgroup i takes tile i mod tiles, split
  // i / tiles, so the tiles of one split (which share A) run side by side.
  switch (SPLIT ? 3 : xcd_mode(p.M, p.N, p.K, BM, BN, (int)sizeof(W))) {
    case 1: {  // columns
      const int ntx = (tiles_n + SMOL_XCDS - 1) / SMOL_XCDS;
      tm = local % tiles_m;
      tn = xcd * ntx + local / tiles_m;
      if (tn >= tiles_n) return;  // whole workgroup
      break;
    }
    case 2: {  // rows
      const int mtx = rows_per_xcd(p.M, BM) / BM;
      tm = xcd * mtx + local % mtx;
      tn = local / mtx;
      if (tm >= tiles_m || tn >= tiles_n) return;  // whole workgroup
      break;
    }
    case 3: {  // K split
      const int t = blockIdx.x % (tiles_m * tiles_n);
      split = blockIdx.x / (tiles_m * tiles_n);
      tm = t % tiles_m;
      tn = t / tiles_m;
      break;
    }
    default:
      tm = blockIdx.x % tiles_m;
      tn = blockIdx.x / tiles_m;
  }
  const int m0 = tm * BM, n0 = tn * BN;

  // DMA sources. Stage byte q*1024 + 16*lane is written by wave instruction q:
  // chunk index q*64 + lane -> (row, slot) of the A or B rows; the slot receives the
  // row's chunk slot ^ lds_swz(row), an XOR swizzle that keeps fragment reads (32
  // rows, one chunk each) free of bank conflicts without padding.
  const char *src[IPW];
  int adv[IPW];  // bytes per stage along the source row
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int cidx = (wave * IPW + j) * 64 + lane;
    if (cidx < A_BYTES / 16) {
      const int r = cidx / CPRA;
      const int c = (cidx % CPRA) ^ lds_swz<CPRA>(r);
      src[j] = (const char *)((const TA *)p.A + (size_t)min(m0 + r, p.M - 1) * p.lda) + c * 16;
      adv[j] = RA;
    } else {
      const int cb = cidx - A_BYTES / 16;
      const int r = cb / CPR;
      const int c = (cb % CPR) ^ lds_swz<CPR>(r);
      src[j] = (const char *)b_row<W, EK, BN>(p, n0 + r) + c * 16;
      adv[j] = RB;
    }
  }
  const int nk = p.K / KE / (SPLIT ? p.ksplit : 1);  // stages of this workgroup
  if constexpr (SPLIT) {
#pragma unroll
    for (int j = 0; j < IPW; ++j) src[j] += (size_t)split * nk * adv[j];
  }
  auto issue = [&](int stage, int slot) {
#pragma unroll
    for (int j = 0; j < IPW; ++j)
      lds_dma16(src[j] + (size_t)stage * adv[j], smem_base + slot * STAGE_BYTES + (wave * IPW + j) * 1024);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){};

  // Epilogue operands that come from memory, loaded now so that their latency hides
  // under the K loop (older than every DMA below, so the ring's vmcnt accounting
  // holds). Items as in the epilogue walks. Residual: the thread's X values (4 floats
  // an item) and, for xs, the norm weights of those columns. QKV: the RoPE (cos, sin)
  // of the item's 4 frequencies and, in a decode step, the row's position.
  const bool scaled = SPLIT ? false : EPI == EPI_RESIDUAL ? p.xs != nullptr : p.ss_new != nullptr;
  constexpr int XPI = BM * BN / 4 / NT;
  constexpr bool XPRE = EPI == EPI_RESIDUAL && ER == BM && XPI >= 1 && XPI <= 4 && XPI * NT * 4 == BM * BN;
  f32x4 xpre[XPRE ? XPI : 1];
  float wpre[XPRE ? XPI : 1][4];
  if constexpr (XPRE) prefetch_residual<W, BN, NT, XPI>(p, m0, n0, tid, scaled, xpre, wpre);
  constexpr int QPI = BM * (BN / 8) / NT;  // QKV items (4 rotation pairs) per thread
  constexpr bool QPRE = EPI == EPI_QKV_ROPE && ER == BM && QPI >= 1 && QPI <= 2 && QPI * NT * 8 == BM * BN;
  f32x4 cspre[QPRE ? QPI : 1][2];
  int pospre[QPRE ? QPI : 1];
  if constexpr (QPRE) prefetch_qkv<BN, NT, QPI>(p, m0, tid, cspre, pospre);

#pragma unroll
  for (int st = 0; st < S - 1; ++st)
    if (st < nk) issue(st, st);

  static_assert(CPRA == CPR, "A and B rows share the swizzle");
  const int sw = lds_swz<CPR>(lane & 31);  // for every fragment row this lane reads (rows = lane mod 32)
  const int half = lane >> 5;

  // Row factors of the deferred RMSNorm, for the epilogue (made visible by its first
  // barrier). Loaded after the first stages are issued so that the latencies
  // overlap; these loads are older than every later DMA, so the ring's vmcnt
  // accounting holds (the compiler waits for them here, with stage 0).
  if (scaled && tid < BM) s_row[tid] = row_factor<EPI>(p, min(m0 + tid, p.M - 1));

  for (int kb = 0; kb < nk; ++kb) {
    // stage kb has landed (for this wave) once at most S-2 later stages are pending
    if (kb + S - 2 < nk)
      wait_vmcnt<(S - 2) * IPW>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();  // ... and for every wave; also all reads of stage kb-1 are done
    if (kb + S - 1 < nk) issue(kb + S - 1, (kb + S - 1) % S);  // refill the slot of stage kb-1
    const char *sa = smem + (kb % S) * STAGE_BYTES + (wm * 32 * TM + (lane & 31)) * RA;
    const char *sb = smem + (kb % S) * STAGE_BYTES + A_BYTES + (wn * 32 * TN + (lane & 31)) * RB;
    if constexpr (MFMA_PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int t = 0; t < KSTEPS / KW; ++t) {
      const int s = t * KW + kw;            // this group's K step within the stage
      Frag<T> fa[TM], fb[TN];
      const int c0 = (2 * s + half) * CPF;  // first chunk of this lane's 8 K values
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const char *row = sa + i * 32 * RA;
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
        const char *row = sb + j * 32 * RB;
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
    if constexpr (MFMA_PRIO) __builtin_amdgcn_s_setprio(0);
  }
  __syncthreads();  // every wave is done reading the stages: the epilogue tile reuses them

  // ------------------------------------------------------------ accumulators -> LDS
  // Row chunk ec holds tile rows [ec*ER, ec*ER + ER): the waves whose rows fall in it
  // write their accumulators (K group KW-1 first, then each lower group adds its
  // own, a fixed order), then the epilogue walks those rows.
#pragma unroll
  for (int ec = 0; ec < BM / ER; ++ec) {
    const int r_lo = ec * ER;
#pragma unroll
    for (int g = KW - 1; g >= 0; --g) {
      if (kw == g) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int rb = wm * 32 * TM + i * 32;  // first tile row of accumulator block i
          if (rb < r_lo || rb >= r_lo + ER) continue;
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              float &t = tile[(rb + acc_row(r, lane) - r_lo) * OP + wn * 32 * TN + j * 32 + (lane & 31)];
              t = (g == KW - 1) ? acc[i][j][r] : t + acc[i][j][r];
            }
        }
      }
      __syncthreads();
    }
    const int em0 = m0 + r_lo;  // first global row of this chunk
    if constexpr (SPLIT) {
      // a K split's share of the tile, unscaled: the reduction applies the epilogue
      float *P = p.part + (size_t)split * p.M * p.N;
      for (int it = tid; it < ER * BN / 4; it += NT) {
        const int r = it / (BN / 4), c = (it % (BN / 4)) * 4;
        if (em0 + r < p.M) store_vec<float, 4>(P + (size_t)(em0 + r) * p.N + n0 + c, &tile[r * OP + c]);
      }
    } else {
      epilogue_rows<W, BN, EK, NT, ER, OP, XPRE ? XPI : 0, QPRE ? QPI : 0>(p, tile, s_row + r_lo, scaled, em0, n0, tid,
                                                                          xpre, wpre, cspre, pospre);
    }
    __syncthreads();  // the next chunk overwrites the tile
  }
}

// The second half of a K-split GEMM: adds the ksplit partial tiles in split order
// (a fixed order, so results do not depend on scheduling) and applies the epilogue.
// A workgroup owns RM rows x BN columns; BN is the GEMM's tile width, so the SwiGLU
// gate/up column pairing and the RoPE heads line up with the GEMM's tiles.
template <typename W, int EPI, int BN, int RM, int NT>
__global__ void __launch_bounds__(NT) gemm_reduce_kernel(const GemmParams p) {
  constexpr int LPI = RM * BN / 4 / NT;  // float4 items of the tile per thread
  static_assert(LPI >= 1 && LPI * NT * 4 == RM * BN, "threads cover the tile");
  constexpr int OP = BN + 4;
  __shared__ __attribute__((aligned(16))) float tile[RM * OP];
  __shared__ float s_row[RM];
  const int tid = threadIdx.x;
  const int tiles_r = (p.M + RM - 1) / RM;
  const int m0 = ((int)blockIdx.x % tiles_r) * RM, n0 = ((int)blockIdx.x / tiles_r) * BN;
  const bool scaled = EPI == EPI_RESIDUAL ? p.xs != nullptr : p.ss_new != nullptr;

  constexpr int XPI = LPI;
  constexpr bool XPRE = EPI == EPI_RESIDUAL && XPI <= 4;
  f32x4 xpre[XPRE ? XPI : 1];
  float wpre[XPRE ? XPI : 1][4];
  if constexpr (XPRE) prefetch_residual<W, BN, NT, XPI>(p, m0, n0, tid, scaled, xpre, wpre);
  constexpr int QPI = RM * (BN / 8) / NT;
  constexpr bool QPRE = EPI == EPI_QKV_ROPE && QPI >= 1 && QPI <= 2 && QPI * NT * 8 == RM * BN;
  f32x4 cspre[QPRE ? QPI : 1][2];
  int pospre[QPRE ? QPI : 1];
  if constexpr (QPRE) prefetch_qkv<BN, NT, QPI>(p, m0, tid, cspre, pospre);

  f32x4 acc[LPI];
  const size_t split_stride = (size_t)p.M * p.N;
#pragma unroll
  for (int k = 0; k < LPI; ++k) {
    const int it = tid + k * NT;
    const int r = it / (BN / 4), c = (it % (BN / 4)) * 4;
    const float *src = p.part + (size_t)min(m0 + r, p.M - 1) * p.N + n0 + c;
    acc[k] = (f32x4){};
    for (int s0 = 0; s0 < p.ksplit; s0 += 8) {  // 8 loads in flight; indices clamped, extras masked
      f32x4 v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = *reinterpret_cast<const f32x4 *>(src + min(s0 + e, p.ksplit - 1) * split_stride);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (s0 + e < p.ksplit) acc[k] += v[e];
    }
  }
  if (scaled && tid < RM) s_row[tid] = row_factor<EPI>(p, min(m0 + tid, p.M - 1));
#pragma unroll
  for (int k = 0; k < LPI; ++k) {
    const int it = tid + k * NT;
    *reinterpret_cast<f32x4 *>(&tile[(it / (BN / 4)) * OP + (it % (BN / 4)) * 4]) = acc[k];
  }
  __syncthreads();
  epilogue_rows<W, BN, EPI, NT, RM, OP, XPRE ? XPI : 0, QPRE ? QPI : 0>(p, tile, s_row, scaled, m0, n0, tid, xpre, wpre,
                                                                        cspre, pospre);
}

// ---------------------------------------------------------------- launchers

// Whether a tile configuration meets the kernel's static requirements.
template <typename W, int BM, int BN, int WM, int WN, int RB, int S, int KW>
constexpr bool gemm_cfg_ok() {
  constexpr int KE = RB / sizeof(W);
  constexpr int stage = (BM + BN) * RB, nw = WM * WN * KW;
  return BM % (32 * WM) == 0 && BN % (32 * WN) == 0 && (BM * RB) % 1024 == 0 && (BN * RB) % 1024 == 0 &&
         RB >= 128 && (stage / 1024) % nw == 0 && (S - 2) * (stage / 1024 / nw) <= 63 && (KE / 16) % KW == 0 &&
         S * stage <= 160 * 1024 && nw <= 16;
}

// What every launch of an epilogue EPI on BN-wide tiles with ke K values per stage
// requires of the parameters.
template <int EPI>
static hipError_t check_params(const GemmParams &p, int BN, int ke) {
  if (p.N % BN != 0 || p.K % ke != 0) return hipErrorInvalidValue;
  if (EPI == EPI_QKV_ROPE && (p.head_dim > BN || BN % p.head_dim != 0 || !p.rope)) return hipErrorInvalidValue;
  if (EPI == EPI_RESIDUAL && p.ss_new && BN % 64 != 0) return hipErrorInvalidValue;  // sums per 64 columns
  const bool scaled = EPI == EPI_RESIDUAL ? p.xs != nullptr : p.ss_new != nullptr;
  if (scaled && (!p.ss_old || (EPI != EPI_RESIDUAL && p.ss_cols != p.K) || (EPI == EPI_RESIDUAL && !p.norm_w)))
    return hipErrorInvalidValue;
  if ((p.ss_new || scaled) && p.ss_cols % 64 != 0) return hipErrorInvalidValue;
  return hipSuccess;
}

template <typename W, int BM, int BN, int WM, int WN, int RB, int EPI, int S, int KW>
static hipError_t launch_cfg(const GemmParams &p, hipStream_t s) {
  if constexpr (!gemm_cfg_ok<W, BM, BN, WM, WN, RB, S, KW>()) {
    return hipErrorInvalidConfiguration;
  } else {
    const hipError_t e = check_params<EPI>(p, BN, RB / (int)sizeof(W));
    if (e != hipSuccess) return e;
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = p.N / BN;
    int tiles;
    switch (xcd_mode(p.M, p.N, p.K, BM, BN, (int)sizeof(W))) {
      case 1: tiles = SMOL_XCDS * ((tiles_n + SMOL_XCDS - 1) / SMOL_XCDS) * tiles_m; break;
      case 2: tiles = SMOL_XCDS * (rows_per_xcd(p.M, BM) / BM) * tiles_n; break;
      default: tiles = tiles_m * tiles_n;
    }
    return launch(gemm_kernel<W, BM, BN, WM, WN, RB, EPI, S, KW>, dim3(tiles), dim3(64 * WM * WN * KW), s, p);
  }
}

// K split for grids of few tiles (a decode step: M = batch). Such a grid streams all
// the weights through the few CUs that own a tile, each at what one workgroup's
// loads in flight allow (about 0.3 us per 128-byte stage). Dividing every 64 x 64
// tile's K stages over ks workgroups (ks a divisor of the stage count, at most
// SMOL_KSPLIT_MAX, at most 256 workgroups) spreads the weight stream over many CUs;
// gemm_reduce_kernel then adds the ks partial tiles in a fixed order and runs the
// epilogue. That second launch costs about 5 us (the floor of a dependent kernel
// here: dispatch, a cold first load, the store drain), so only long K loops split:
// measured at batch 64, the down projection (K = 1536, 24 stages) drops from 12.3
// to 4.9 + 4.6 us, while K = 576 (9 stages) takes 8 us unsplit and 10-11 us split.
#ifndef SMOL_KSPLIT_MAX
#define SMOL_KSPLIT_MAX 8
#endif
constexpr int SMOL_KSPLIT_MIN_STAGES = 16;
static int ksplit_plan(int M, int N, int K, int esz) {
  if (N % 64 != 0) return 1;
  const long tiles = (long)((M + 63) / 64) * (N / 64);
  if (tiles >= 128) return 1;
  const int nk = K / (128 / esz);
  if (nk < SMOL_KSPLIT_MIN_STAGES) return 1;
  int best = 1;
  for (int ks = 2; ks <= SMOL_KSPLIT_MAX && ks <= nk; ++ks)
    if (nk % ks == 0 && tiles * ks <= 256) best = ks;
  return best;
}

size_t gemm_part_floats(int M, int N, int K, int esz) {
  const int ks = ksplit_plan(M, N, K, esz);
  return ks > 1 ? (size_t)ks * M * N : 0;
}

template <typename W, int EPI>
static hipError_t launch_split(GemmParams p, int ks, hipStream_t s) {
  constexpr int RB = 128;
  hipError_t e = check_params<EPI>(p, 64, ks * (RB / (int)sizeof(W)));
  if (e != hipSuccess) return e;
  p.ksplit = ks;
  const int tiles = ((p.M + 63) / 64) * (p.N / 64);
  // A timed class spans both launches: from the GEMM's start to the reduction's end.
  hipEvent_t e0 = nullptr, e1 = nullptr;
  timing_take(&e0, &e1);
  constexpr int WM = 2, WN = 2, KW = 2;
  e = launch_ev(gemm_kernel<W, 64, 64, WM, WN, RB, EPI | EPI_SPLIT, 4, KW>, dim3(tiles * ks), dim3(64 * WM * WN * KW), s,
                e0, nullptr, p);
  if (e != hipSuccess) return e;
  constexpr int RM = 16, NT = EPI == EPI_QKV_ROPE ? 128 : 256;
  return launch_ev(gemm_reduce_kernel<W, EPI, 64, RM, NT>, dim3(((p.M + RM - 1) / RM) * (p.N / 64)), dim3(NT), s,
                   nullptr, e1, p);
}

// Tile choice, from sweeps on MI355X over the model's shapes (256-byte stages did
// not pay):
//   * a plain store or SwiGLU with >= 512 tiles of 256 x 256, a residual with >= 256
//     (one per CU): 256 x 256 in 4 x 4 waves, which halves the L2 -> LDS bytes per
//     FLOP of 128 x 128 (lm_head at batch 4 x seq 512: 160 us against 200; the
//     SmolLM3-3B shape at batch 2 x seq 4096: gate/up 1003 -> 870 us, down 451 -> 396,
//     o_proj 119 -> 105);
//   * >= 512 tiles of 128 x 128: 128 x 128 with the four waves side by side along N,
//     so each converted weight fragment feeds four MFMAs;
//   * >= 512 tiles of 64 x 128: the same 1 x 4 wave layout (gate/up);
//   * N a multiple of 192 but not of 128 with >= 256 tiles of 64 x 192 (QKV, o_proj
//     and down at 8192 rows): 64 x 192 in 2 x 2 waves, two K groups;
//   * otherwise 64 x 64 in a 2 x 2 wave layout, for parallelism on small N (o_proj,
//     down and QKV); 64 x 128 when a 128-wide head must stay in one tile for RoPE;
//     32 x 64 (1 x 2 waves, two K groups) on grids of fewer than 128 64 x 64 tiles.
// Grids of a few hundred tiles leave one wave per SIMD, whose LDS -> convert -> MFMA
// chain then runs exposed: those split each stage's K steps over two wave groups.
// Grids under 128 tiles (a decode step: M = batch) stream weights that are cold in
// L2 and MALL through few workgroups, each bounded by the bytes it stages (about
// 30 GB/s per CU); there a 4-deep ring keeps three stages of HBM reads in flight
// (measured 25-30% faster than 2 stages with cold weights), and 32-row tiles double
// the workgroups while each stages a quarter fewer bytes (batch-64 decode step 1.785
// -> 1.754 ms; with one K group, 1.866; rings of 6 or 8 stages, 1.86-1.87). In the
// prefill each layer's weights are also cold in L2 (they come from MALL or HBM): the
// residual GEMMs (o_proj, and down with its 24 stages) run a 3-deep ring (down
// 22.2 -> 18.8 us at batch 4 x seq 512; 4 stages or 4 wave groups gain nothing
// more). QKV and gate/up stay at 2: QKV gains nothing, and a third stage of the
// 64 x 128 gate/up tiles leaves room for two workgroups per CU instead of three, so
// its 768 workgroups no longer run in one round (18.7 -> 20.8 us).
template <typename T, int EPI>
static hipError_t launch_gemm(const GemmParams &p, hipStream_t s) {
  if (p.part && (EPI != EPI_QKV_ROPE || p.head_dim == 64)) {
    const int ks = ksplit_plan(p.M, p.N, p.K, sizeof(T));
    if (ks > 1) return launch_split<T, EPI>(p, ks, s);
  }
  const long tm128 = (p.M + 127) / 128, tm64 = (p.M + 63) / 64;
  const long t256 = p.N % 256 == 0 ? ((p.M + 255) / 256) * (long)(p.N / 256) : 0;
  if (((EPI == EPI_STORE || EPI == EPI_SWIGLU) && t256 >= 512) || (EPI == EPI_RESIDUAL && t256 >= 256))
    return launch_cfg<T, 256, 256, 4, 4, 128, EPI, 2, 1>(p, s);
  if (EPI != EPI_QKV_ROPE || p.head_dim == 64)
    if (tm64 * (p.N / 64) < 128 && p.N % 64 == 0) return launch_cfg<T, 32, 64, 1, 2, 128, EPI, 4, 2>(p, s);
  // Widths that 128 does not divide (576, 960) on grids of >= 256 tiles of 64 x 192: a
  // third fewer bytes staged per FLOP than 64 x 64, which is what bounds these GEMMs
  // (batch 1 x seq 8192: QKV 37 -> 32.5 us, o_proj 27 -> 23.5, down 46 -> 38.5; a
  // 3-deep ring for the residual ones, 1 x 2 waves in four K groups and 128 x 192 QKV
  // tiles were all slower).
  if (sizeof(T) == 2 && p.N % 192 == 0 && p.N % 128 != 0 && tm64 * (p.N / 192) >= 256 &&
      (EPI != EPI_QKV_ROPE || 192 % p.head_dim == 0))
    return launch_cfg<T, 64, 192, 2, 2, 128, EPI, 2, 2>(p, s);
  if (p.N % 128 == 0 && tm128 * (p.N / 128) >= 512) return launch_cfg<T, 128, 128, 1, 4, 128, EPI, 2, 2>(p, s);
  if (EPI == EPI_QKV_ROPE && p.head_dim == 128) return launch_cfg<T, 64, 128, 2, 2, 128, EPI, 2, 2>(p, s);
  if (EPI != EPI_QKV_ROPE && p.N % 128 == 0 && tm64 * (p.N / 128) >= 512)
    return launch_cfg<T, 64, 128, 1, 4, 128, EPI, 2, 2>(p, s);
  if (EPI == EPI_RESIDUAL) return launch_cfg<T, 64, 64, 2, 2, 128, EPI, 3, 2>(p, s);
  return launch_cfg<T, 64, 64, 2, 2, 128, EPI, 2, 2>(p, s);
}

static void set_norm_in(GemmParams &p, const NormIn &n, int H) {
  p.ss_new = const_cast<float *>(n.ss_new);
  p.ss_old = n.ss_old;
  p.ss_cols = H;
  p.eps = n.eps;
}

template <typename T>
hipError_t gemm_store(const Act<T> *A, const NormIn &nrm, const T *B, int M, int N, int K, void *C, int c_f32,
                      float *part, hipStream_t s) {
  GemmParams p{};
  p.part = part;
  p.A = A; p.lda = K; p.B0 = B; p.M = M; p.N = N; p.K = K; p.C = C; p.ldc = N; p.c_f32 = c_f32;
  set_norm_in(p, nrm, K);
  return launch_gemm<T, EPI_STORE>(p, s);
}

template <typename T>
hipError_t gemm_residual(const Act<T> *A, const T *B, int M, int N, int K, float *X, const NormOut &nrm, float *part,
                         hipStream_t s) {
  GemmParams p{};
  p.part = part;
  p.A = A; p.lda = K; p.B0 = B; p.M = M; p.N = N; p.K = K; p.C = X; p.ldc = N;
  p.ss_old = nrm.ss_old; p.ss_new = nrm.ss_new; p.norm_w = nrm.w; p.xs = nrm.xs; p.ss_cols = N; p.eps = nrm.eps;
  return launch_gemm<T, EPI_RESIDUAL>(p, s);
}

template <typename T>
hipError_t gemm_swiglu(const Act<T> *A, const NormIn &nrm, const T *Wg, const T *Wu, int M, int I, int K, Act<T> *Y,
                       float *part, hipStream_t s) {
  GemmParams p{};
  p.part = part;
  p.A = A; p.lda = K; p.B0 = Wg; p.B1 = Wu; p.M = M; p.N = 2 * I; p.K = K; p.C = Y; p.ldc = I;
  set_norm_in(p, nrm, K);
  return launch_gemm<T, EPI_SWIGLU>(p, s);
}

template <typename T>
hipError_t gemm_qkv_rope(const Act<T> *A, const NormIn &nrm, const T *Wq, const T *Wk, const T *Wv, const QkvOut &o,
                         float *part, hipStream_t s) {
  GemmParams p{};
  p.part = part;
  p.A = A; p.lda = o.hidden; p.B0 = Wq; p.B1 = Wk; p.B2 = Wv;
  p.M = o.M; p.N = o.nq_cols + 2 * o.nkv_cols; p.K = o.hidden;
  set_norm_in(p, nrm, o.hidden);
  p.nq_cols = o.nq_cols; p.nkv_cols = o.nkv_cols; p.head_dim = o.head_dim;
  p.q_out = o.q; p.k_out = o.k; p.v_out = o.v;
  p.seq = o.seq; p.cap = o.cap; p.n_kv = o.n_kv; p.pos0 = o.pos0; p.kv_off = o.kv_off; p.max_pos = o.max_pos;
  p.cache_len = o.cache_len;
  p.rope = o.rope;
  p.rope_on = o.rope_on;
  if (!o.rope || o.head_dim % 8 != 0) return hipErrorInvalidValue;
  return launch_gemm<T, EPI_QKV_ROPE>(p, s);
}

#define SMOL_INST(T)                                                                                          \
  template hipError_t gemm_store<T>(const Act<T> *, const NormIn &, const T *, int, int, int, void *, int,     \
                                    float *, hipStream_t);                                                     \
  template hipError_t gemm_residual<T>(const Act<T> *, const T *, int, int, int, float *, const NormOut &,     \
                                       float *, hipStream_t);                                                  \
  template hipError_t gemm_swiglu<T>(const Act<T> *, const NormIn &, const T *, const T *, int, int, int,      \
                                     Act<T> *, float *, hipStream_t);                                          \
  template hipError_t gemm_qkv_rope<T>(const Act<T> *, const NormIn &, const T *, const T *, const T *,        \
                                       const QkvOut &, float *, hipStream_t);
SMOL_INST(float)
SMOL_INST(bf16)

}  // namespace smol
