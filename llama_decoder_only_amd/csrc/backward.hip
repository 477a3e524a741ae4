// Backward pass of one decoder block in float32 on gfx950.
//
// What is differentiated is the pre-norm block h = x + attn(RMSNorm_a(x)),
// out = h + mlp(RMSNorm_m(h)) (nnterp "SmolLM3", "The block, in order"; abi96062
// components.py, TransformerBlock / RMSNorm / GroupedQueryAttention / SwiGLU_FFN;
// Sualeh77 model.py, "2." to "6."). The pages train this model but print no
// gradient formulas; the kernels below apply the chain rule to each step, and the
// host sequence that strings them together is in api.hip (smol_block_backward).
//
// Every contraction runs on v_mfma_f32_32x32x2f32 (float32 operands, float32
// accumulation). Three kernel families:
//
//  * bw_gemm: C[M, N] = sum_k A(m, k) B(k, n) with each operand either K-contiguous
//    (activations [M, K], weights [N, K] as nn.Linear stores them) or
//    index-contiguous (a weight [K, N] read along its rows for a data gradient; an
//    activation [K, M] read down its columns for a weight gradient, whose
//    contraction runs over the tokens). Both operands are staged k-major in LDS, so
//    the MFMA reads are the same for every layout. Fused epilogues: store, add into
//    C (gradient accumulation), add a residual, and the SwiGLU backward.
//
//  * attention: forward with the log-sum-exp kept, dQ, and dK/dV, FlashAttention-2
//    style (scores recomputed per tile, never stored). Scores are computed
//    transposed where that lets the accumulator feed the next MFMA directly: the
//    32x32 accumulator of S^T = K Q^T holds, in lane l, query l % 32 and the keys
//    of rows acc_row(r, l); that is exactly the B operand layout of a contraction
//    over keys if step j of that contraction takes, in lane half h, the key of
//    register j (key order inside a contraction is free as long as both operands
//    agree). So P^T and dS^T never go through LDS.
//
//  * row kernels: RMSNorm forward (keeps 1/rms), RMSNorm backward with per-block
//    column partials of the weight gradient (summed in a fixed order after), RoPE,
//    the per-query dot(dO, O), and the sum of the per-query-head dK/dV partials
//    over each kv head's group.
//
// No atomics: every float sum has a fixed order, so a call is deterministic.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace smol {

namespace {

constexpr float NEG_INF = -__builtin_huge_valf();

__device__ __forceinline__ f32x16 mfma2(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ GEMM

constexpr int GT = 64;         // tile rows and columns
constexpr int GK = 32;         // K per LDS stage
// LDS row length (floats) of a k-major stage X[k][index]. An index-contiguous
// operand is stored with 16-byte vector writes, so its rows stay 16-byte aligned
// (68). A K-contiguous one is transposed on the way in: each thread writes 4 rows
// k .. k+3 of one index, the 8 threads of an index group 8 different k chunks; rows
// of 66 floats spread those scalar writes over more banks than 68 (measured: the
// LDS bank-conflict cycles of such stages dropped, 2-4% off their GEMMs).
template <bool KC> constexpr int gld() { return KC ? GT + 2 : GT + 4; }

// Storage row `row` of a segmented operand (up to three matrices stacked along
// their rows, e.g. [W_q; W_k; W_v]).
__device__ __forceinline__ const float *seg_row(const BwOperand &o, int row) {
  if (row < o.seg0) return o.p0 + (size_t)row * o.ld;
  if (row < o.seg1) return o.p1 + (size_t)(row - o.seg0) * o.ld;
  return o.p2 + (size_t)(row - o.seg1) * o.ld;
}

// One operand's 64 (index) x 32 (k) stage into registers, two 16-byte loads per
// thread; zeros outside [0, n_idx) x [0, K).
//   KC: K-contiguous, storage row = index, element = k (8 threads per row);
//   else index-contiguous, storage row = k, element = index (16 threads per row).
template <bool KC>
__device__ __forceinline__ void stage_load(f32x4 (&v)[2], const BwOperand &o, int idx0, int n_idx, int k0, int K,
                                           int tid) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int f = tid + 256 * i;
    int row, elem;
    bool ok;
    if constexpr (KC) {
      const int ri = f >> 3, kc = f & 7;
      row = idx0 + ri;
      elem = k0 + kc * 4;
      ok = row < n_idx && elem < K;
    } else {
      const int kr = f >> 4, ic = f & 15;
      row = k0 + kr;
      elem = idx0 + ic * 4;
      ok = row < K && elem < n_idx;
    }
    v[i] = ok ? *reinterpret_cast<const f32x4 *>(seg_row(o, row) + elem) : (f32x4){0.f, 0.f, 0.f, 0.f};
  }
}

// The staged values into LDS, k-major: X[k][index].
template <bool KC>
__device__ __forceinline__ void stage_store(float (*X)[gld<KC>()], const f32x4 (&v)[2], int tid) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int f = tid + 256 * i;
    if constexpr (KC) {
      const int ri = f >> 3, kc = f & 7;
#pragma unroll
      for (int j = 0; j < 4; ++j) X[kc * 4 + j][ri] = v[i][j];
    } else {
      const int kr = f >> 4, ic = f & 15;
      *reinterpret_cast<f32x4 *>(&X[kr][ic * 4]) = v[i];
    }
  }
}

__device__ __forceinline__ float sigmoid(float g) { return 1.0f / (1.0f + expf(-g)); }

// Destination of C element (row, col): the row's segment picks the matrix.
__device__ __forceinline__ float *c_at(const BwGemm &p, int row, int col) {
  if (row < p.cseg0) return p.C + (size_t)row * p.ldc + col;
  if (row < p.cseg1) return p.C1 + (size_t)(row - p.cseg0) * p.ldc + col;
  return p.C2 + (size_t)(row - p.cseg1) * p.ldc + col;
}

// A 64 x 64 tile per workgroup of 4 waves, each wave one 32 x 32 quarter. K runs in
// stages of 32 through two LDS buffers: the next stage's global loads are in flight
// while the current one feeds the MFMAs; one barrier per stage. With a K split,
// workgroup i takes tile i % tiles and K range i / tiles, and writes its partial tile.
template <bool AK, bool BK, int EB, bool SPLIT>
__global__ __launch_bounds__(256) void bw_gemm_kernel(const BwGemm p) {
  __shared__ float As[2][GK][gld<AK>()];
  __shared__ float Bs[2][GK][gld<BK>()];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;
  const int ntn = (p.N + GT - 1) / GT;
  const int tiles = ntn * ((p.M + GT - 1) / GT);
  const int tile = SPLIT ? blockIdx.x % tiles : blockIdx.x;
  const int m0 = (tile / ntn) * GT, n0 = (tile % ntn) * GT;
  const int nk_all = (p.K + GK - 1) / GK;
  int kt0 = 0, kt1 = nk_all;
  if constexpr (SPLIT) {
    const int per = (nk_all + p.ksplit - 1) / p.ksplit, split = blockIdx.x / tiles;
    kt0 = min(split * per, nk_all);
    kt1 = min(kt0 + per, nk_all);
  }

  f32x16 acc = {};
  if (kt0 < kt1) {
    f32x4 ra[2], rb[2];
    stage_load<AK>(ra, p.a, m0, p.M, kt0 * GK, p.K, tid);
    stage_load<BK>(rb, p.b, n0, p.N, kt0 * GK, p.K, tid);
    stage_store<AK>(As[0], ra, tid);
    stage_store<BK>(Bs[0], rb, tid);
    __syncthreads();
    for (int kt = kt0; kt < kt1; ++kt) {
      const int cur = (kt - kt0) & 1;
      const bool more = kt + 1 < kt1;
      if (more) {
        stage_load<AK>(ra, p.a, m0, p.M, (kt + 1) * GK, p.K, tid);
        stage_load<BK>(rb, p.b, n0, p.N, (kt + 1) * GK, p.K, tid);
      }
#pragma unroll
      for (int kk = 0; kk < GK / 2; ++kk)
        acc = mfma2(As[cur][2 * kk + hl][wm * 32 + l32], Bs[cur][2 * kk + hl][wn * 32 + l32], acc);
      if (more) {
        stage_store<AK>(As[cur ^ 1], ra, tid);
        stage_store<BK>(Bs[cur ^ 1], rb, tid);
      }
      __syncthreads();
    }
  }

  const int col = n0 + wn * 32 + l32;
  if (col >= p.N) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = m0 + wm * 32 + acc_row(r, lane);
    if (row >= p.M) continue;
    const float v = acc[r];
    if constexpr (SPLIT) {
      p.part[((size_t)(blockIdx.x / tiles) * p.M + row) * p.N + col] = v;
    } else if constexpr (EB == BW_STORE) {
      *c_at(p, row, col) = v;
    } else if constexpr (EB == BW_ACCUM) {
      *c_at(p, row, col) += v;
    } else if constexpr (EB == BW_RESID) {
      *c_at(p, row, col) = p.R[(size_t)row * p.ldr + col] + v;
    } else {  // BW_SWIGLU: v = dL/dy_mlp at (row, col); gate and up from the forward
      float *c = c_at(p, row, col);
      const float g = p.G[(size_t)row * p.ldg + col], u = p.G[(size_t)row * p.ldg + p.half + col];
      const float sg = sigmoid(g), sl = g * sg;
      c[0] = v * u * (sg * (1.0f + g * (1.0f - sg)));  // d silu(g)/dg = s (1 + g (1 - s))
      c[p.half] = v * sl;
      p.Y[(size_t)row * p.ldy + col] = sl * u;
    }
  }
}

// The K split's partial tiles added in split order, then the epilogue. One thread
// per 4 consecutive columns (N is a multiple of 4).
template <int EB>
__global__ __launch_bounds__(256) void bw_split_reduce_kernel(const BwGemm p) {
  const int n4 = p.N / 4;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= p.M * n4) return;
  const int row = i / n4, col = (i % n4) * 4;
  const size_t mn = (size_t)p.M * p.N, at = (size_t)row * p.N + col;
  f32x4 v = *reinterpret_cast<const f32x4 *>(p.part + at);
  for (int k = 1; k < p.ksplit; ++k) v += *reinterpret_cast<const f32x4 *>(p.part + k * mn + at);
  float *c = c_at(p, row, col);
  if constexpr (EB == BW_ACCUM) v += *reinterpret_cast<const f32x4 *>(c);
  if constexpr (EB == BW_RESID) v += *reinterpret_cast<const f32x4 *>(p.R + (size_t)row * p.ldr + col);
  *reinterpret_cast<f32x4 *>(c) = v;
}

template <bool AK, bool BK, int EB>
hipError_t bw_gemm_launch(const BwGemm &p, hipStream_t s) {
  const int tiles = ((p.M + GT - 1) / GT) * ((p.N + GT - 1) / GT);
  if constexpr (EB != BW_SWIGLU) {
    if (p.ksplit > 1) {  // timed as one operation: start at the first kernel, stop after the reduce
      hipEvent_t e0 = nullptr, e1 = nullptr;
      timing_take(&e0, &e1);
      hipError_t e = launch_ev(bw_gemm_kernel<AK, BK, EB, true>, dim3(tiles * p.ksplit), dim3(256), s, e0, nullptr, p);
      if (e != hipSuccess) return e;
      return launch_ev(bw_split_reduce_kernel<EB>, dim3((p.M * (p.N / 4) + 255) / 256), dim3(256), s, nullptr, e1, p);
    }
  }
  return launch(bw_gemm_kernel<AK, BK, EB, false>, dim3(tiles), dim3(256), s, p);
}

// ------------------------------------------------------------------ attention

__device__ __forceinline__ bool visible(const BwAttn &a, int b, int tq, int tk) {
  return tk <= tq && tq < a.T && (a.window == 0 || tk > tq - a.window) &&
         (a.key_mask == nullptr || a.key_mask[(size_t)b * a.T + tk] != 0);
}

// Rows row0 .. row0 + 64 NP - 1 (NP blocks of 64) of two column blocks of [B*T, ld]
// matrices into LDS [64 NP][D + 1] (the +1 spreads a column read over all banks);
// zeros past T. All 128 NP threads of the workgroup take part.
template <int D, int NP>
__device__ __forceinline__ void stage_rows2(float *X, float *Y, const float *xs, const float *ys, int ldx, int ldy,
                                            int b, int T, int row0, int tid) {
  constexpr int LD = D + 1;
  for (int f = tid; f < 64 * NP * D / 4; f += 128 * NP) {
    const int r = f / (D / 4), c4 = f % (D / 4);
    const int t = row0 + r;
    f32x4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
    if (t < T) {
      x = *reinterpret_cast<const f32x4 *>(xs + ((size_t)b * T + t) * ldx + c4 * 4);
      y = *reinterpret_cast<const f32x4 *>(ys + ((size_t)b * T + t) * ldy + c4 * 4);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      X[r * LD + c4 * 4 + j] = x[j];
      Y[r * LD + c4 * 4 + j] = y[j];
    }
  }
}

// The half of a row that a lane feeds into a contraction over d: lane half h takes
// d = h * D/2 + s at step s (a bijection, shared by both operands).
template <int D>
__device__ __forceinline__ void load_half_row(float (&v)[D / 2], const float *row, int hl) {
#pragma unroll
  for (int s = 0; s < D / 2; s += 4) {
    const f32x4 x = *reinterpret_cast<const f32x4 *>(row + hl * (D / 2) + s);
    v[s] = x[0];
    v[s + 1] = x[1];
    v[s + 2] = x[2];
    v[s + 3] = x[3];
  }
}

// Inverse RoPE of a gradient held as 32 x 32 accumulator tiles over d (tile t holds
// d = 32 t + acc_row(r, lane)): the rotation at the row's position is orthogonal, so
// its transpose (the rotation by -angle) carries the gradient back to the
// projection. cs: the row's (cos, sin) per frequency.
template <int D>
__device__ __forceinline__ void rotate_back(f32x16 (&g)[D / 32], const float2 *cs, int lane) {
  constexpr int TH = D / 64;  // tiles per half: pair (i, i + D/2) sits in tiles t, t + TH
#pragma unroll
  for (int t = 0; t < TH; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float2 c = cs[t * 32 + acc_row(r, lane)];
      const float x = g[t][r], y = g[t + TH][r];
      g[t][r] = x * c.x + y * c.y;
      g[t + TH][r] = y * c.x - x * c.y;
    }
  }
}

// The three attention kernels share one work split: a workgroup of 2 NP waves owns
// 64 rows (queries, or keys for dK/dV) of one (sequence, query head), blockIdx.x the
// (sequence, head) and blockIdx.y the row block (the heaviest first); wave w takes the
// 32 rows of group w & 1 and the blocks of 64 columns (keys, or queries) whose index
// is w >> 1 modulo NP, NP blocks staged in LDS per round. The parities' partial
// results meet in LDS at the end and are combined in parity order. NP is 4 where
// the registers and LDS allow two such workgroups' worth of waves per CU (forward
// and dQ at head dim 64), else 2.

// Forward attention, keeping the log-sum-exp (base 2) of every query's scores for
// the backward.
template <int D, int NP>
__global__ __launch_bounds__(128 * NP) void bw_attn_fwd_kernel(const BwAttn a) {
  constexpr int LD = D + 1, HD = D / 2, NT = D / 32, CS = NT * 16 + 2;
  __shared__ float Ks[64 * NP * LD], Vs[64 * NP * LD];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hl = lane >> 5;
  const int rg = w & 1, par = w >> 1;
  const int qb = gridDim.y - 1 - blockIdx.y, b = blockIdx.x / a.nq, hd = blockIdx.x % a.nq, g = hd / a.G;
  const int tq = qb * 64 + rg * 32 + l32;
  const bool qok = tq < a.T;
  const size_t rowq = (size_t)b * a.T + min(tq, a.T - 1);
  float qreg[HD];
  load_half_row<D>(qreg, a.qkv + rowq * a.ld + hd * D, hl);
  const float *kbase = a.qkv + (a.nq + g) * D, *vbase = a.qkv + (a.nq + a.nkv + g) * D;

  f32x16 oacc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) oacc[t] = (f32x16){};
  float m_run = NEG_INF, l_run = 0.f;
  const int kb_hi = min(qb * 64 + 63, a.T - 1) / 64;
  const int kb_lo = a.window > 0 ? max(0, qb * 64 - a.window + 1) / 64 : 0;
  for (int kb0 = kb_lo; kb0 <= kb_hi; kb0 += NP) {
    __syncthreads();
    stage_rows2<D, NP>(Ks, Vs, kbase, vbase, a.ld, a.ld, b, a.T, kb0 * 64, tid);
    __syncthreads();
    const int kb = kb0 + par;
    if (kb > kb_hi) continue;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int r0 = par * 64 + c * 32;  // LDS row of this 32-key sub-block
      f32x16 st = {};
      const float *kr = Ks + (r0 + l32) * LD + hl * HD;
#pragma unroll
      for (int s = 0; s < HD; ++s) st = mfma2(kr[s], qreg[s], st);
      float p[16], mx = NEG_INF;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tk = kb * 64 + c * 32 + acc_row(r, lane);
        p[r] = (qok && visible(a, b, tq, tk)) ? st[r] * a.scale2 : NEG_INF;
        mx = fmaxf(mx, p[r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float mu = m_new == NEG_INF ? 0.f : m_new;
      float ls = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = exp2f(p[r] - mu);
        ls += p[r];
      }
      ls += __shfl_xor(ls, 32, 64);
      const float f = exp2f(m_run - mu);
      l_run = l_run * f + ls;
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        oacc[t] *= f;
#pragma unroll
        for (int j = 0; j < 16; ++j)
          oacc[t] = mfma2(Vs[(r0 + acc_row(j, lane)) * LD + t * 32 + l32], p[j], oacc[t]);
      }
    }
  }
  // parities 1 .. NP-1 hand (O, m, l) to parity 0 of the same row group, which merges
  // them in parity order
  __syncthreads();
  if (par > 0) {
    float *xch = Ks + (((par - 1) * 2 + rg) * 64 + lane) * CS;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) xch[t * 16 + r] = oacc[t][r];
    xch[NT * 16] = m_run;
    xch[NT * 16 + 1] = l_run;
  }
  __syncthreads();
  if (par > 0 || !qok) return;
#pragma unroll
  for (int q = 1; q < NP; ++q) {
    const float *xch = Ks + (((q - 1) * 2 + rg) * 64 + lane) * CS;
    const float m2 = xch[NT * 16], l2 = xch[NT * 16 + 1];
    const float mm = fmaxf(m_run, m2), mu = mm == NEG_INF ? 0.f : mm;
    const float f1 = exp2f(m_run - mu), f2 = exp2f(m2 - mu);
    l_run = l_run * f1 + l2 * f2;
    m_run = mm;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[t][r] = oacc[t][r] * f1 + xch[t * 16 + r] * f2;
  }
  const float inv = 1.0f / l_run;  // a query with no visible key: 0 / 0, NaN
  float *orow = a.o + rowq * (size_t)(a.nq * D) + hd * D;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) orow[t * 32 + acc_row(r, lane)] = oacc[t][r] * inv;
  if (hl == 0) a.lse[((size_t)b * a.nq + hd) * a.T + tq] = m_run + log2f(l_run);
}

// dQ: for every visible key block, P = exp2(S log2(e)/sqrt(d) - lse),
// dS = P (dO V^T - rowsum(dO O)), dQ += dS K; then dQ / sqrt(d), rotated back on a
// rotary block, into dqkv.
template <int D, int NP>
__global__ __launch_bounds__(128 * NP) void bw_attn_dq_kernel(const BwAttn a) {
  constexpr int LD = D + 1, HD = D / 2, NT = D / 32, CS = NT * 16;
  __shared__ float Ks[64 * NP * LD], Vs[64 * NP * LD];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hl = lane >> 5;
  const int rg = w & 1, par = w >> 1;
  const int qb = gridDim.y - 1 - blockIdx.y, b = blockIdx.x / a.nq, hd = blockIdx.x % a.nq, g = hd / a.G;
  const int tq = qb * 64 + rg * 32 + l32;
  const bool qok = tq < a.T;
  const size_t rowq = (size_t)b * a.T + min(tq, a.T - 1);
  float qreg[HD], doreg[HD];
  load_half_row<D>(qreg, a.qkv + rowq * a.ld + hd * D, hl);
  load_half_row<D>(doreg, a.dO + rowq * (size_t)(a.nq * D) + hd * D, hl);
  const size_t stat = ((size_t)b * a.nq + hd) * a.T + min(tq, a.T - 1);
  const float lse = a.lse[stat], dsum = a.dsum[stat];
  const float *kbase = a.qkv + (a.nq + g) * D, *vbase = a.qkv + (a.nq + a.nkv + g) * D;

  f32x16 dq[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) dq[t] = (f32x16){};
  const int kb_hi = min(qb * 64 + 63, a.T - 1) / 64;
  const int kb_lo = a.window > 0 ? max(0, qb * 64 - a.window + 1) / 64 : 0;
  for (int kb0 = kb_lo; kb0 <= kb_hi; kb0 += NP) {
    __syncthreads();
    stage_rows2<D, NP>(Ks, Vs, kbase, vbase, a.ld, a.ld, b, a.T, kb0 * 64, tid);
    __syncthreads();
    const int kb = kb0 + par;
    if (kb > kb_hi) continue;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int r0 = par * 64 + c * 32;
      f32x16 st = {}, dp = {};
      const float *kr = Ks + (r0 + l32) * LD + hl * HD;
      const float *vr = Vs + (r0 + l32) * LD + hl * HD;
#pragma unroll
      for (int s = 0; s < HD; ++s) {
        st = mfma2(kr[s], qreg[s], st);
        dp = mfma2(vr[s], doreg[s], dp);
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tk = kb * 64 + c * 32 + acc_row(r, lane);
        const float pr = (qok && visible(a, b, tq, tk)) ? exp2f(st[r] * a.scale2 - lse) : 0.f;
        ds[r] = pr * (dp[r] - dsum);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          dq[t] = mfma2(Ks[(r0 + acc_row(j, lane)) * LD + t * 32 + l32], ds[j], dq[t]);
    }
  }
  __syncthreads();
  if (par > 0) {
    float *xch = Ks + (((par - 1) * 2 + rg) * 64 + lane) * CS;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) xch[t * 16 + r] = dq[t][r];
  }
  __syncthreads();
  if (par > 0 || !qok) return;
#pragma unroll
  for (int q = 1; q < NP; ++q) {  // the parities' partial sums, added in parity order
    const float *xch = Ks + (((q - 1) * 2 + rg) * 64 + lane) * CS;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[t][r] += xch[t * 16 + r];
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) dq[t] *= a.scale;
  if (a.rope_on) rotate_back<D>(dq, a.rope_cs + rowq * (D / 2), lane);
  float *out = a.dqkv + rowq * a.ld + hd * D;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) out[t * 32 + acc_row(r, lane)] = dq[t][r];
}

// dK and dV of 64 keys over every query block that can see them: dV += P^T dO,
// dK += dS^T Q / sqrt(d). Written as this query head's partial (rotated back on a
// rotary block); bw_kv_reduce_kernel sums the partials of the query heads that
// share a kv head.
template <int D>
__global__ __launch_bounds__(256) void bw_attn_dkdv_kernel(const BwAttn a) {
  constexpr int LD = D + 1, HD = D / 2, NT = D / 32, CS = 2 * NT * 16, UC = D == 64 ? 2 : 1;
  __shared__ float Qs[128 * LD], Os[128 * LD], Ls[128], Ds[128];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hl = lane >> 5;
  const int kg = w & 1, par = w >> 1;
  const int kb = blockIdx.y, b = blockIdx.x / a.nq, hd = blockIdx.x % a.nq, g = hd / a.G;
  const int tk = kb * 64 + kg * 32 + l32;
  const bool kok = tk < a.T;
  const size_t rowk = (size_t)b * a.T + min(tk, a.T - 1);
  float kreg[HD], vreg[HD];
  load_half_row<D>(kreg, a.qkv + rowk * a.ld + (a.nq + g) * D, hl);
  load_half_row<D>(vreg, a.qkv + rowk * a.ld + (a.nq + a.nkv + g) * D, hl);
  const size_t stat0 = ((size_t)b * a.nq + hd) * a.T;

  f32x16 dk[NT], dv[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) dk[t] = dv[t] = (f32x16){};
  const int q_last = a.window > 0 ? min(a.T - 1, kb * 64 + 63 + a.window - 1) : a.T - 1;
  const int qb_hi = q_last / 64;
  for (int qb0 = kb; qb0 <= qb_hi; qb0 += 2) {
    __syncthreads();
    stage_rows2<D, 2>(Qs, Os, a.qkv + hd * D, a.dO + hd * D, a.ld, a.nq * D, b, a.T, qb0 * 64, tid);
    if (tid < 128) {
      const int t = qb0 * 64 + tid;
      Ls[tid] = t < a.T ? a.lse[stat0 + t] : 0.f;
      Ds[tid] = t < a.T ? a.dsum[stat0 + t] : 0.f;
    }
    __syncthreads();
    const int qb = qb0 + par;
    if (qb > qb_hi) continue;
#pragma unroll UC  // (head dim 128: one sub-block at a time, or the registers spill)
    for (int c = 0; c < 2; ++c) {
      const int r0 = par * 64 + c * 32;  // LDS row of this 32-query sub-block
      f32x16 st = {}, dp = {};
      const float *qr = Qs + (r0 + l32) * LD + hl * HD;
      const float *orow = Os + (r0 + l32) * LD + hl * HD;
#pragma unroll
      for (int s = 0; s < HD; ++s) {
        st = mfma2(qr[s], kreg[s], st);
        dp = mfma2(orow[s], vreg[s], dp);
      }
      float pr[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = r0 + acc_row(r, lane);
        const int tq = qb0 * 64 + qi;
        pr[r] = (kok && visible(a, b, tq, tk)) ? exp2f(st[r] * a.scale2 - Ls[qi]) : 0.f;
        ds[r] = pr[r] * (dp[r] - Ds[qi]);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int qi = r0 + acc_row(j, lane);
          dv[t] = mfma2(Os[qi * LD + t * 32 + l32], pr[j], dv[t]);
          dk[t] = mfma2(Qs[qi * LD + t * 32 + l32], ds[j], dk[t]);
        }
    }
  }
  __syncthreads();
  float *xch = Qs + (kg * 64 + lane) * CS;
  if (par == 1) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        xch[t * 16 + r] = dk[t][r];
        xch[(NT + t) * 16 + r] = dv[t][r];
      }
  }
  __syncthreads();
  if (par == 1 || !kok) return;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[t][r] = (dk[t][r] + xch[t * 16 + r]) * a.scale;
      dv[t][r] += xch[(NT + t) * 16 + r];
    }
  if (a.rope_on) rotate_back<D>(dk, a.rope_cs + rowk * (D / 2), lane);
  const size_t M = (size_t)a.B * a.T;
  float *pk = a.part + ((size_t)hd * M + rowk) * D;
  float *pv = a.part + ((size_t)(a.nq + hd) * M + rowk) * D;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pk[t * 32 + acc_row(r, lane)] = dk[t][r];
      pv[t * 32 + acc_row(r, lane)] = dv[t][r];
    }
}

// dsum[b, h, t] = sum_e dO[m, h*D + e] O[m, h*D + e] (the softmax backward's row term).
__global__ __launch_bounds__(256) void bw_rowdot_kernel(const float *dO, const float *O, float *dsum, int M, int T,
                                                        int nq, int D) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= M * nq) return;
  const int m = i / nq, hd = i % nq;
  const f32x4 *x = reinterpret_cast<const f32x4 *>(dO + (size_t)m * nq * D + hd * D);
  const f32x4 *y = reinterpret_cast<const f32x4 *>(O + (size_t)m * nq * D + hd * D);
  float s = 0.f;
  for (int e = 0; e < D / 4; ++e) {
    const f32x4 u = x[e], v = y[e];
    s += u[0] * v[0] + u[1] * v[1] + u[2] * v[2] + u[3] * v[3];
  }
  dsum[((size_t)(m / T) * nq + hd) * T + m % T] = s;
}

// dqkv's k and v columns: the sum, in head order, of the partials of the G query
// heads of each kv head. One thread per 4 floats.
__global__ __launch_bounds__(256) void bw_kv_reduce_kernel(const float *part, float *dqkv, int M, int nq, int nkv,
                                                           int G, int D, int ld) {
  const int per_row = 2 * nkv * D / 4;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= M * per_row) return;
  const int m = i / per_row, rest = i % per_row;
  const int which = rest / (nkv * D / 4), within = rest % (nkv * D / 4);  // 0: k, 1: v
  const int g = within / (D / 4), e = (within % (D / 4)) * 4;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < G; ++j)
    s += *reinterpret_cast<const f32x4 *>(part + ((size_t)(which * nq + g * G + j) * M + m) * D + e);
  *reinterpret_cast<f32x4 *>(dqkv + (size_t)m * ld + (nq + which * nkv + g) * D + e) = s;
}

// The RoPE table of the call: cs[m * D/2 + i] = (cos, sin) of (pos0 + m % T) * omega_i
// (rope_cos_sin: the angle formed and reduced in double).
__global__ __launch_bounds__(256) void bw_rope_table_kernel(float2 *cs, int M, int T, int half, int pos0,
                                                            const InvFreq f) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= M * half) return;
  const int m = i / half, j = i % half;
  cs[i] = rope_cos_sin(pos0 + m % T, f.v[j]);
}

// RoPE on the q and k columns of qkv, in place: pair (j, j + D/2) of every head
// rotated by the row's angle j (Sualeh77 model.py, "3. RoPE").
__global__ __launch_bounds__(256) void bw_rope_kernel(float *qkv, int M, int ld, int heads, int D, const float2 *cs) {
  const int half = D / 2;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= M * heads * half) return;
  const int m = i / (heads * half), rest = i % (heads * half);
  const int h = rest / half, j = rest % half;
  const float2 c = cs[(size_t)m * half + j];
  float *z = qkv + (size_t)m * ld + h * D;
  const float x = z[j], y = z[j + half];
  z[j] = x * c.x - y * c.y;
  z[j + half] = y * c.x + x * c.y;
}

// u = w * x * r, r = 1 / sqrt(mean(x^2) + eps) per row (abi96062 components.py,
// RMSNorm); r is kept for the backward. One wave per row.
__global__ __launch_bounds__(256) void bw_rms_fwd_kernel(const float *x, const float *w, float *u, float *r, int M,
                                                         int H, float eps) {
  const int lane = threadIdx.x & 63, row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float *xr = x + (size_t)row * H;
  float ss = 0.f;
  for (int c = lane * 4; c < H; c += 256) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(xr + c);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = wave_sum(ss);
  const float rr = 1.0f / sqrtf(ss / (float)H + eps);
  for (int c = lane * 4; c < H; c += 256) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(xr + c);
    const f32x4 wv = *reinterpret_cast<const f32x4 *>(w + c);
    *reinterpret_cast<f32x4 *>(u + (size_t)row * H + c) = wv * v * rr;
  }
  if (lane == 0) r[row] = rr;
}

// RMSNorm backward for u = w * n, n = x * r: with dn = du * w,
//   dx = resid + r * (dn - n * mean(dn * n))
// (resid: the gradient that reaches x around the sublayer), and the workgroup's
// column sums of du * n over its rows (the weight gradient before the final sum):
// each wave sums its rows, waves 1-3 hand theirs to wave 0 through LDS, which adds
// them in wave order. 16 rows per workgroup, 4 per wave; NC = 16-byte columns per
// lane (H <= 256 NC).
constexpr int RMS_ROWS = 16;
template <int NC>
__global__ __launch_bounds__(256) void bw_rms_bwd_kernel(const float *du, const float *x, const float *r,
                                                         const float *w, const float *resid, float *dx, float *part,
                                                         int M, int H) {
  __shared__ f32x4 red[3][NC * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f32x4 colacc[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) colacc[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < RMS_ROWS / 4; ++i) {
    const int row = blockIdx.x * RMS_ROWS + wave * (RMS_ROWS / 4) + i;
    if (row >= M) break;
    const float rr = r[row];
    const size_t o = (size_t)row * H;
    f32x4 g[NC], n[NC];
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = (lane + 64 * j) * 4;
      g[j] = n[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (c < H) {
        g[j] = *reinterpret_cast<const f32x4 *>(du + o + c);
        n[j] = *reinterpret_cast<const f32x4 *>(x + o + c) * rr;
        const f32x4 dn = g[j] * *reinterpret_cast<const f32x4 *>(w + c);
        dot += dn[0] * n[j][0] + dn[1] * n[j][1] + dn[2] * n[j][2] + dn[3] * n[j][3];
      }
    }
    dot = wave_sum(dot) / (float)H;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = (lane + 64 * j) * 4;
      if (c < H) {
        const f32x4 dn = g[j] * *reinterpret_cast<const f32x4 *>(w + c);
        const f32x4 rs = *reinterpret_cast<const f32x4 *>(resid + o + c);
        *reinterpret_cast<f32x4 *>(dx + o + c) = rs + rr * (dn - n[j] * dot);
        colacc[j] += g[j] * n[j];
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < NC; ++j) red[wave - 1][lane + 64 * j] = colacc[j];
  }
  __syncthreads();
  if (wave > 0) return;
  float *pr = part + (size_t)blockIdx.x * H;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c = (lane + 64 * j) * 4;
    if (c < H)
      *reinterpret_cast<f32x4 *>(pr + c) =
          ((colacc[j] + red[0][lane + 64 * j]) + red[1][lane + 64 * j]) + red[2][lane + 64 * j];
  }
}

// dw[c] (+)= sum over the partial rows. 64 columns per workgroup of 16 waves; wave
// v sums rows v, v + 16, ... and the 16 wave sums are added in wave order.
__global__ __launch_bounds__(1024) void bw_colsum_kernel(const float *part, int nrows, int H, float *dw,
                                                         int accumulate) {
  __shared__ float red[16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  float s = 0.f;
  if (c < H)
    for (int i = wave; i < nrows; i += 16) s += part[(size_t)i * H + c];
  red[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && c < H) {
    float t = red[0][lane];
#pragma unroll
    for (int v = 1; v < 16; ++v) t += red[v][lane];
    dw[c] = accumulate ? dw[c] + t : t;
  }
}

// bfloat16 -> float32 (exact: the bits move to the top half), 8 elements per thread.
__global__ __launch_bounds__(256) void bw_widen_kernel(const bf16 *src, float *dst, size_t n) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= n) return;
  if (i + 8 <= n) {
    const Chunk16 c = ld16(src + i);
    f32x4 lo, hi;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo[j] = __uint_as_float(c[j >> 1] << ((j & 1) ? 0 : 16) & 0xffff0000u);
      hi[j] = __uint_as_float(c[2 + (j >> 1)] << ((j & 1) ? 0 : 16) & 0xffff0000u);
    }
    *reinterpret_cast<f32x4 *>(dst + i) = lo;
    *reinterpret_cast<f32x4 *>(dst + i + 4) = hi;
  } else {
    for (size_t j = i; j < n; ++j) dst[j] = (float)src[j];
  }
}

}  // namespace

// ------------------------------------------------------------------ launchers

// Few tiles and a long K (weight gradients contract over all B*T tokens): split K
// until about 1024 workgroups run, at most 8 ways and at least 4 stages (128 of K)
// per split. Not for the SwiGLU epilogue, which needs the whole sum at once.
int bw_gemm_ksplit(int M, int N, int K, int epi) {
  if (epi == BW_SWIGLU) return 1;
  const int tiles = ((M + GT - 1) / GT) * ((N + GT - 1) / GT);
  const int stages = (K + GK - 1) / GK;
  int ks = std::min(8, 1024 / std::max(tiles, 1));
  ks = std::min(ks, stages / 4);
  return std::max(ks, 1);
}

size_t bw_gemm_part_floats(int M, int N, int K, int epi) {
  const int ks = bw_gemm_ksplit(M, N, K, epi);
  return ks > 1 ? (size_t)ks * M * N : 0;
}

hipError_t bw_gemm(int layout, int epi, const BwGemm &p, hipStream_t s) {
  if (p.M < 1 || p.N < 1 || p.K < 1) return hipErrorInvalidValue;
  if (p.ksplit > 1 && (p.part == nullptr || p.N % 4 || epi == BW_SWIGLU || p.ldc % 4 || (epi == BW_RESID && p.ldr % 4)))
    return hipErrorInvalidValue;
  const bool ak = layout == BW_NT || layout == BW_NN, bk = layout == BW_NT;
  // 16-byte loads: the contiguous extent of each operand and its row length must be
  // multiples of 4 floats
  if ((ak ? p.K : p.M) % 4 || p.a.ld % 4 || (bk ? p.K : p.N) % 4 || p.b.ld % 4) return hipErrorInvalidValue;
#define BW_CASE(L, A, B)                                                           \
  if (layout == L) {                                                               \
    switch (epi) {                                                                 \
      case BW_STORE: return bw_gemm_launch<A, B, BW_STORE>(p, s);                  \
      case BW_ACCUM: return bw_gemm_launch<A, B, BW_ACCUM>(p, s);                  \
      case BW_RESID: return bw_gemm_launch<A, B, BW_RESID>(p, s);                  \
      case BW_SWIGLU: return bw_gemm_launch<A, B, BW_SWIGLU>(p, s);                \
    }                                                                              \
  }
  BW_CASE(BW_NT, true, true)
  BW_CASE(BW_NN, true, false)
  BW_CASE(BW_TN, false, false)
#undef BW_CASE
  return hipErrorInvalidValue;
}

hipError_t bw_attention(int which, const BwAttn &a, hipStream_t s) {
  // blocks of 64 rows along y, dispatched after x: the causally heaviest blocks (last
  // queries; first keys) first, so a second round of workgroups holds the lightest
  const dim3 grid(a.B * a.nq, (a.T + 63) / 64);
  if (a.D == 64) {
    if (which == 0) return launch(bw_attn_fwd_kernel<64, 4>, grid, dim3(512), s, a);
    if (which == 1) return launch(bw_attn_dq_kernel<64, 4>, grid, dim3(512), s, a);
    return launch(bw_attn_dkdv_kernel<64>, grid, dim3(256), s, a);
  }
  if (a.D == 128) {
    if (which == 0) return launch(bw_attn_fwd_kernel<128, 2>, grid, dim3(256), s, a);
    if (which == 1) return launch(bw_attn_dq_kernel<128, 2>, grid, dim3(256), s, a);
    return launch(bw_attn_dkdv_kernel<128>, grid, dim3(256), s, a);
  }
  return hipErrorInvalidValue;
}

hipError_t bw_rowdot(const float *dO, const float *O, float *dsum, int M, int T, int nq, int D, hipStream_t s) {
  return launch(bw_rowdot_kernel, dim3((M * nq + 255) / 256), dim3(256), s, dO, O, dsum, M, T, nq, D);
}

hipError_t bw_kv_reduce(const float *part, float *dqkv, int M, int nq, int nkv, int G, int D, int ld, hipStream_t s) {
  const int n = M * (2 * nkv * D / 4);
  return launch(bw_kv_reduce_kernel, dim3((n + 255) / 256), dim3(256), s, part, dqkv, M, nq, nkv, G, D, ld);
}

hipError_t bw_rope_table(float2 *cs, int M, int T, int D, int pos0, const InvFreq &f, hipStream_t s) {
  if (D / 2 > 64) return hipErrorInvalidValue;
  const int n = M * (D / 2);
  return launch(bw_rope_table_kernel, dim3((n + 255) / 256), dim3(256), s, cs, M, T, D / 2, pos0, f);
}

hipError_t bw_rope(float *qkv, int M, int ld, int heads, int D, const float2 *cs, hipStream_t s) {
  const int n = M * heads * (D / 2);
  return launch(bw_rope_kernel, dim3((n + 255) / 256), dim3(256), s, qkv, M, ld, heads, D, cs);
}

hipError_t bw_rms_fwd(const float *x, const float *w, float *u, float *r, int M, int H, float eps, hipStream_t s) {
  if (H % 4 || H > 4096) return hipErrorInvalidValue;
  return launch(bw_rms_fwd_kernel, dim3((M + 3) / 4), dim3(256), s, x, w, u, r, M, H, eps);
}

int bw_rms_part_rows(int M) { return (M + RMS_ROWS - 1) / RMS_ROWS; }

hipError_t bw_rms_bwd(const float *du, const float *x, const float *r, const float *w, const float *resid, float *dx,
                      float *part, int M, int H, hipStream_t s) {
  if (H % 4 || H > 4096) return hipErrorInvalidValue;
  const dim3 grid((M + RMS_ROWS - 1) / RMS_ROWS), block(256);
  const int nc = (H / 4 + 63) / 64;
  if (nc <= 1) return launch(bw_rms_bwd_kernel<1>, grid, block, s, du, x, r, w, resid, dx, part, M, H);
  if (nc <= 2) return launch(bw_rms_bwd_kernel<2>, grid, block, s, du, x, r, w, resid, dx, part, M, H);
  if (nc <= 3) return launch(bw_rms_bwd_kernel<3>, grid, block, s, du, x, r, w, resid, dx, part, M, H);
  if (nc <= 4) return launch(bw_rms_bwd_kernel<4>, grid, block, s, du, x, r, w, resid, dx, part, M, H);
  if (nc <= 8) return launch(bw_rms_bwd_kernel<8>, grid, block, s, du, x, r, w, resid, dx, part, M, H);
  return launch(bw_rms_bwd_kernel<16>, grid, block, s, du, x, r, w, resid, dx, part, M, H);
}

hipError_t bw_widen(const bf16 *src, float *dst, size_t n, hipStream_t s) {
  if ((uintptr_t)src % 16 || (uintptr_t)dst % 16) return hipErrorInvalidValue;
  return launch(bw_widen_kernel, dim3((unsigned)((n + 2047) / 2048)), dim3(256), s, src, dst, n);
}

hipError_t bw_colsum(const float *part, int nrows, int H, float *dw, int accumulate, hipStream_t s) {
  return launch(bw_colsum_kernel, dim3((H + 63) / 64), dim3(1024), s, part, nrows, H, dw, accumulate);
}

}  // namespace smol
