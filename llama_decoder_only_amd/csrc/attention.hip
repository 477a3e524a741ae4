// Causal grouped-query attention, prefill (flash-style, online softmax).
//
// softmax(q k^T / sqrt(d) + causal) v with query head h reading kv head
// h / G, G = n_heads / n_kv (Sualeh77 model.py, "4. Attention"; abi96062
// components.py, GroupedQueryAttention; nnterp "SmolLM3", "Grouped-query attention").
//
// One workgroup owns (sequence b, kv head g, a block of 32*QW queries) and runs
// G*QW waves: every query head of the group, 32 queries per wave. Each 64-key
// tile of K and V is staged in LDS once and read by all G heads, so the group's
// K/V are fetched once instead of G times (no repeat_interleave copy).
//
// A wave computes S^T = K . Q^T with 32x32x16 MFMAs, so its lane holds one query
// (lane % 32) and half of that query's keys in registers: the row max / sum of
// the online softmax needs only in-register reductions plus one exchange with
// lane ^ 32. P then feeds O^T = V^T . P^T straight from those registers; V is
// written to LDS transposed ([d][key]) so each lane reads 4 consecutive keys.
// Keys come in tiles in increasing order, so tile 0 (always visible) fixes a
// finite running max before any fully masked tile can occur.
#include "common.h"
#include "kernels.h"

namespace smol {

template <typename W, int D, int G, int QW>
__global__ void __launch_bounds__(64 * G * QW)
attn_prefill_kernel(const AttnArgs a) {
  using T = Act<W>;  // operand type of q, p and o; cached k, v (type W) convert on staging
  constexpr int NW = G * QW, NT = 64 * NW, BQ = 32 * QW, BKV = 64;
  constexpr int EPC = 16 / sizeof(T);
  constexpr int KP = D + EPC;    // K row pitch (elements)
  constexpr int VP = BKV + EPC;  // V^T row pitch (elements)
  constexpr int CPR = D / EPC;   // chunks per key row
  constexpr int CH = BKV * CPR;  // chunks per K (or V) tile
  constexpr int MAXC = (2 * CH + NT - 1) / NT;
  constexpr int DS = D / 16;     // MFMA K-steps over the head dim
  constexpr int DT = D / 32;     // 32-row tiles of O^T

  __shared__ __attribute__((aligned(16))) T Ks[2][BKV * KP];
  __shared__ __attribute__((aligned(16))) T Vt[2][D * VP];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int half = lane >> 5, ql = lane & 31;
  const int nqb = (a.T + BQ - 1) / BQ;
  const int per = a.B * a.n_kv;
  const int qb = nqb - 1 - (int)blockIdx.x / per;  // longest (latest) query blocks first
  const int rem = (int)blockIdx.x % per;
  const int b = rem / a.n_kv, g = rem % a.n_kv;
  const int h = g * G + w / QW;
  const int q0 = qb * BQ + (w % QW) * 32;
  const int qt = min(q0 + ql, a.T - 1);
  const bool wave_live = q0 < a.T;
  const int ldq = a.n_heads * D;

  Frag<T> qf[DS];
  {
    const T *qp = (const T *)a.q + (size_t)(b * a.T + qt) * ldq + h * D + half * 8;
#pragma unroll
    for (int s = 0; s < DS; ++s) load_frag(qf[s], qp + 16 * s);
  }

  const int last_q = min(a.T - 1, qb * BQ + BQ - 1);
  const int nkeys = last_q + a.q_key_off + 1;
  const int ntiles = (nkeys + BKV - 1) / BKV;
  const int wave_kmax = min(a.T - 1, q0 + 31) + a.q_key_off;
  const int my_kmax = qt + a.q_key_off;

  const W *kbase_ptr = (const W *)a.k + (size_t)(b * a.n_kv + g) * a.cap * D;
  const W *vbase_ptr = (const W *)a.v + (size_t)(b * a.n_kv + g) * a.cap * D;

  Chunk16 pre[MAXC];
  auto fetch = [&](int kt) {
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = min(tid + i * NT, 2 * CH - 1);  // surplus threads re-read the last chunk
      const int cc = c < CH ? c : c - CH;
      const int key = min(kt * BKV + cc / CPR, nkeys - 1);
      const W *src = (c < CH ? kbase_ptr : vbase_ptr) + (size_t)key * D + (cc % CPR) * EPC;
      pre[i] = ld16(src);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = tid + i * NT;
      const Chunk16 cv = to_operand<W>(pre[i]);
      if (c < CH) {
        st16(&Ks[buf][(c / CPR) * KP + (c % CPR) * EPC], cv);
      } else if (c < 2 * CH) {
        const int cc = c - CH;
        const int key = cc / CPR, d0 = (cc % CPR) * EPC;
#pragma unroll
        for (int j = 0; j < EPC; ++j) Vt[buf][(d0 + j) * VP + key] = chunk_elem<T>(cv, j);
      }
    }
  };

  const float c_log2 = 1.4426950408889634f / sqrtf((float)D);
  f32x16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;

  fetch(0);
  stash(0);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int cur = kt & 1;
    fetch(min(kt + 1, ntiles - 1));  // branch-free prefetch (the last one is a harmless re-read)
    __builtin_amdgcn_sched_barrier(0);  // issue the loads before this tile's math
    const int k0 = kt * BKV;
    if (wave_live && k0 <= wave_kmax) {
      f32x16 s[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
      for (int st = 0; st < DS; ++st) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          Frag<T> kf;
          load_frag(kf, &Ks[cur][(32 * i + ql) * KP + 16 * st + half * 8]);
          mma_32x32x16(s[i], kf, qf[st]);
        }
      }
      const bool need_mask = k0 + BKV - 1 > q0 + a.q_key_off;
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = s[i][r] * c_log2;
          if (need_mask && k0 + 32 * i + acc_row(r, lane) > my_kmax) v = -INFINITY;
          s[i][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);
      float ls = 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2f(s[i][r] - m_new);
          s[i][r] = p;
          ls += p;
        }
      l_run = l_run * alpha + ls;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
#pragma unroll
      for (int sg = 0; sg < 4; ++sg) {
        Frag<T> pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) pf.v[e] = from_f32<T>(s[sg >> 1][8 * (sg & 1) + e]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const T *vp = &Vt[cur][(32 * dt + ql) * VP + 16 * sg + 4 * half];
          Frag<T> vf;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vf.v[e] = vp[e];
            vf.v[4 + e] = vp[8 + e];
          }
          mma_32x32x16(o[dt], vf, pf);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    stash(cur ^ 1);
    __syncthreads();
  }

  if (!wave_live || q0 + ql >= a.T) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  T *op = (T *)a.o + (size_t)(b * a.T + q0 + ql) * ldq + h * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) op[32 * dt + acc_row(r, lane)] = from_f32<T>(o[dt][r] * inv);
}

template <typename T, int D, int G>
static hipError_t launch_attn_g(const AttnArgs &a, hipStream_t s) {  // T: storage type
  // Two query sub-blocks per wave group when that still gives enough workgroups.
  const long wg2 = (long)a.B * a.n_kv * ((a.T + 63) / 64);
  if (G == 1 || wg2 >= 256) {
    const int nqb = (a.T + 63) / 64;
    hipLaunchKernelGGL((attn_prefill_kernel<T, D, G, 2>), dim3(nqb * a.B * a.n_kv), dim3(64 * G * 2), 0, s, a);
  } else {
    const int nqb = (a.T + 31) / 32;
    hipLaunchKernelGGL((attn_prefill_kernel<T, D, G, 1>), dim3(nqb * a.B * a.n_kv), dim3(64 * G), 0, s, a);
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_attn_d(const AttnArgs &a, hipStream_t s) {
  switch (a.n_heads / a.n_kv) {
    case 1: return launch_attn_g<T, D, 1>(a, s);
    case 2: return launch_attn_g<T, D, 2>(a, s);
    case 3: return launch_attn_g<T, D, 3>(a, s);
    case 4: return launch_attn_g<T, D, 4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t attention_prefill(const AttnArgs &a, hipStream_t s) {
  if (a.head_dim == 64) return launch_attn_d<T, 64>(a, s);
  if (a.head_dim == 128) return launch_attn_d<T, 128>(a, s);
  return hipErrorInvalidValue;
}

template hipError_t attention_prefill<float>(const AttnArgs &, hipStream_t);
template hipError_t attention_prefill<bf16>(const AttnArgs &, hipStream_t);

}  // namespace smol
