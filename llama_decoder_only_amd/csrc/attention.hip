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
// K and V tiles stream through an S-deep LDS ring filled by direct global->LDS
// copies in their cache layout ([key][d], 16-byte chunks XOR-swizzled per row).
// A wave computes S^T = K . Q^T with 32x32x16 MFMAs, so its lane holds one query
// (lane % 32) and half of that query's keys in registers: the row max / sum of
// the online softmax needs only in-register reductions plus one exchange with
// lane ^ 32. P then feeds O^T = V^T . P^T straight from those registers; the V^T
// fragments come from transposing LDS reads (ds_read_b64_tr_b16). K and V of a bf16
// cache enter bf16 MFMAs as they were copied, with no conversion pass.
// Keys come in tiles in increasing order, so without a key mask tile 0 (always
// visible) fixes a finite running max before any fully masked tile can occur; with
// one, a row may see no key yet (or ever): its max stays -inf, its probabilities 0,
// and a row that never sees a key ends as 0/0 = NaN.
#include "common.h"
#include "kernels.h"

namespace smol {

// Slot permutation of the K/V tiles: 16-byte chunk c of key row r sits at slot
// c ^ att_slot(r), att_slot(r) = 2 (r mod 4) + (r / 4 mod 2), a bijection of r mod 8.
// K fragment reads (one chunk from each of 8 consecutive rows per LDS cycle) then hit 8
// distinct slots, and so do the transposing V reads, whose 16-lane groups take two
// adjacent chunks (c, c + 1; c even) of 4 consecutive rows: the rows' slots differ in
// bits 1-2, the two chunks in bit 0. (With c ^ (r mod 8) those 8 blocks fell on 4
// slots, a 2-way conflict on every V read.)
__device__ __forceinline__ int att_slot(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

// Byte offset of element (row, col) of an ES-byte type in a swizzled LDS tile with RB-byte rows.
template <int RB, int ES>
__device__ __forceinline__ int swz(int row, int col) {
  constexpr int EPC = 16 / ES;
  return row * RB + (((col / EPC) ^ att_slot(row)) << 4) + (col % EPC) * ES;
}

typedef __fp16 half4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

// 4 x 16-bit transposed read (gfx950 ds_read_b64_tr_b16). Within each group of 16
// lanes, lane 4r + c receives element c of the 8-byte blocks addressed by lanes
// 4j + r, j = 0..3 (an in-bounds probe on the hardware fixed this mapping).
__device__ __forceinline__ u16x4 lds_read_tr16(const char *p) {
  const half4 v = __builtin_amdgcn_ds_read_tr16_b64_v4f16((__attribute__((address_space(3))) half4 *)p);
  return __builtin_bit_cast(u16x4, v);
}

typedef __attribute__((address_space(3))) char lds_char;

// Max of x over lanes l and l ^ 32 (gfx950 v_permlane32_swap: one VALU exchange of the
// two halves instead of an LDS permute and its address arithmetic).
__device__ __forceinline__ float max_lane32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// A lane's LDS address for this round, opaque to the optimiser: the reads at fixed
// offsets from it then use the instructions' immediate offsets, where left alone the
// compiler hoisted every (lane offset + immediate) sum out of the loop into a register
// of its own and added the round's base to each one (16 more VGPRs and 32 more VALU
// instructions per round).
__device__ __forceinline__ const lds_char *lds_base(const char *p) {
  const lds_char *q = (const lds_char *)p;
  asm volatile("" : "+v"(q));
  return q;
}


// How far (log2 units) a tile's max may pass the running reference max before the
// reference moves (p = exp2(s - m_ref) <= 2^8 meanwhile).
constexpr float ATTN_REF_SLACK = 8.0f;

// MASKED: the launch has a key mask or a sliding window (a query at key index i then
// sees only indices > i - window; rounds wholly before the block's first window are
// skipped). A separate instantiation: the mask's byte loads inside the ring loop make
// the compiler drain every outstanding load (it cannot see the ring's direct-to-LDS
// copies), which the unmasked kernel must not pay.
//
// Operands: a bf16 cache feeds bf16 MFMAs straight from LDS (no conversion); q, stored
// float16, is scaled by log2(e)/sqrt(d) once and rounded to bf16, and p is rounded to
// bf16 for the P.V product, its row sum adding exactly the rounded values
// (v_dot2_f32_bf16): the operand precision of a bf16 attention. A float cache keeps
// float operands throughout.
// bf16 cache: the running reference max m enters the score MFMAs as one more K step,
// ones in K against -m split into three bf16 parts (hi + mid + lo: exact for a float)
// in q's place, so they return s*log2(e)/sqrt(d) - m and p is one v_exp_f32. float
// cache: one FMA per score.
template <typename W, int D, int G, int QW, int KS, int S, bool MASKED>
__global__ void __launch_bounds__(64 * G * QW * KS)
attn_prefill_kernel(const AttnArgs a) {
  using QT = Act<W>;  // how q and o are stored (float16 for a bf16 model)
  using T = W;        // MFMA operand type: bf16 or float, as the cache
  constexpr int NW = G * QW * KS, BQ = 32 * QW, BKV = 64;
  constexpr int ES = sizeof(W);
  constexpr int RB = D * ES;                       // bytes per key row
  constexpr int CPR = RB / 16;                     // 16-byte chunks per key row
  constexpr int TILE_BYTES = BKV * RB;             // K (or V) bytes per tile
  constexpr int STAGE_BYTES = KS * 2 * TILE_BYTES; // one round: KS tiles of K and V
  constexpr int NINS = STAGE_BYTES / 1024;         // DMA wave-instructions per round
  constexpr int IPW = (NINS + NW - 1) / NW;        // per wave (surplus waves repeat the last one)
  constexpr int DS = D / 16;                       // MFMA K-steps over the head dim
  constexpr int DT = D / 32;                       // 32-row tiles of O^T
  constexpr int PSTATE = DT * 16 + 2;              // floats per lane of a partial state
  static_assert(S >= 2, "ring depth");
  static_assert(KS == 1 || (KS - 1) * G * QW * PSTATE * 64 * 4 <= S * STAGE_BYTES, "partials fit the ring");

  __shared__ __attribute__((aligned(16))) char smem[S * STAGE_BYTES];
  const uint32_t smem_base = lds_addr(smem);

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, ql = lane & 31;
  const int hq = w % (G * QW), ks = w / (G * QW);  // (head, query sub-block) and key split
  const int nqb = (a.T + BQ - 1) / BQ;
  const int per = a.B * a.n_kv;
  const int qb = nqb - 1 - (int)blockIdx.x / per;  // longest (latest) query blocks first
  const int rem = (int)blockIdx.x % per;
  const int b = rem / a.n_kv, g = rem % a.n_kv;
  const int h = g * G + hq / QW;
  const int q0 = qb * BQ + (hq % QW) * 32;
  const int qt = min(q0 + ql, a.T - 1);
  const bool wave_live = q0 < a.T;
  const int ldq = a.n_heads * D;
  const float c_log2 = 1.4426950408889634f / sqrtf((float)D);

  // q fragments, scaled into the log2 domain (using the loads here also makes the
  // compiler wait for them now: left to the key loop, its vmcnt waits, which count the
  // ring's DMAs too, would stall every round on the copies just issued)
  Frag<T> qf[DS];
  {
    Frag<QT> raw[DS];
    const QT *qp = (const QT *)a.q + (size_t)(b * a.T + qt) * ldq + h * D + half * 8;
#pragma unroll
    for (int st = 0; st < DS; ++st) load_frag(raw[st], qp + 16 * st);
#pragma unroll
    for (int st = 0; st < DS; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qf[st].v[e] = from_f32<T>((float)raw[st].v[e] * (ES == 2 ? c_log2 : 1.f));
      }
  }

  const int last_q = min(a.T - 1, qb * BQ + BQ - 1);
  const int nkeys = last_q + a.q_key_off + 1;
  const int ntiles = (nkeys + BKV - 1) / BKV;
  const int nrounds = (ntiles + KS - 1) / KS;
  const int wave_kmax = min(a.T - 1, q0 + 31) + a.q_key_off;
  const int my_kmax = qt + a.q_key_off;

  const W *kbase_ptr = (const W *)a.k + (size_t)(b * a.n_kv + g) * a.cap * D;
  const W *vbase_ptr = (const W *)a.v + (size_t)(b * a.n_kv + g) * a.cap * D;

  // DMA: instruction q of a round fills LDS bytes [q*1024, q*1024 + 1024) of the stage:
  // chunk index q*64 + lane -> (tile of the round, K or V, key row, slot); the slot
  // receives the row's chunk slot ^ att_slot(row). An instruction's 64 lanes stay inside
  // one tile of K or of V (a tile is 64 * CPR chunks), so its source is a wave-uniform
  // base, which moves with the round, plus a fixed 32-bit byte offset per lane: the
  // copies of a full round take the global_load_lds form with an SGPR base. Only a round
  // that reaches past the last key (the final one) clamps each lane's key instead.
  static_assert((BKV * CPR) % 64 == 0, "an instruction covers one tile");
  const W *dma_tile[IPW];    // K or V base of the instruction's tile within a round (uniform)
  int dma_t0[IPW];           // that tile's first key within the round (uniform)
  uint32_t dma_lane[IPW];    // the lane's byte offset from the tile's first key row
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int q = min(w * IPW + j, NINS - 1);
    const int part = q * 64 / (BKV * CPR);  // 2 * tile_in_round + (0 = K, 1 = V)
    const int cidx = q * 64 + lane;
    const int row = (cidx % (BKV * CPR)) / CPR;
    const int c = (cidx % CPR) ^ att_slot(row);
    dma_tile[j] = ((part & 1) == 0 ? kbase_ptr : vbase_ptr) + (size_t)(part >> 1) * BKV * D;
    dma_t0[j] = (part >> 1) * BKV;
    dma_lane[j] = (uint32_t)(row * RB + c * 16);
  }
  auto issue = [&](int r, int slot) {
    const int key0 = r * KS * BKV;
    if (key0 + KS * BKV <= nkeys) {
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const int q = min(w * IPW + j, NINS - 1);
        const W *base = dma_tile[j] + (size_t)key0 * D;
        asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(dma_lane[j]), "s"(base),
                     "{m0}"(smem_base + slot * STAGE_BYTES + q * 1024) : "memory");
      }
    } else {
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const int q = min(w * IPW + j, NINS - 1);
        const int key = min(key0 + dma_t0[j] + (int)(dma_lane[j] / RB), nkeys - 1);
        lds_dma16((const char *)dma_tile[j] + (size_t)(key - dma_t0[j]) * RB + dma_lane[j] % RB,
                  smem_base + slot * STAGE_BYTES + q * 1024);
      }
    }
  };

  // Per-lane LDS offsets of the K fragments (S^T = K Q^T) and of the V^T fragment
  // sources for the transposed reads, fixed for the whole loop. att_slot depends on the
  // row modulo 8 only, so rows 8 apart sit exactly 8 row lengths apart: one offset per K
  // step (K) or per 32-dim tile (V) serves every row group, the rest is an immediate.
  int koff[DS];
#pragma unroll
  for (int st = 0; st < DS; ++st) koff[st] = swz<RB, ES>(ql, 16 * st + half * 8);
  int voff[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    // lane l supplies 4 dims starting at 16*((l/16)%2) + 4*(l%4) of key row
    // 16 sg + 8 pp + 4*(l/32) + (l%16)/4; the transposed read then returns dim
    // (l % 32) of the 4 keys 16 sg + 8 pp + 4 half + (0..3).
    const int sl = lane & 15;
    voff[dt] = ES == 2 ? swz<RB, ES>(4 * half + (sl >> 2), 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (sl & 3)) : 0;
  }

  f32x16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = (f32x16){};
  // m_run: the reference max (log2 domain; -inf until the lane's query has seen a key).
  // bf16: kx / qx, the extra K step of the scores: k indices 0-2 (lanes of half 0,
  // elements 0-2) hold 1 in K and the three bf16 parts of -m_run in q (0 while m_run is
  // -inf), every other index 0.
  float m_run = -INFINITY, l_run = 0.f;
  Frag<T> kx, qx;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    kx.v[e] = from_f32<T>((e < 3 && half == 0) ? 1.f : 0.f);
    qx.v[e] = from_f32<T>(0.f);
  }
  constexpr bool XSTEP = ES == 2;

  // first round that holds a key some query of the block may see (0 without a window)
  const int rf = (MASKED && a.window > 0) ? max(0, qb * BQ + a.q_key_off - a.window + 1) / (KS * BKV) : 0;
  const int nr = nrounds - rf;  // rounds walked; walk step `step` is round rf + step, in slot step % S
#pragma unroll
  for (int st = 0; st < S - 1; ++st)
    if (st < nr) issue(rf + st, st);

  for (int step = 0; step < nr; ++step) {
    const int r = rf + step;
    if (step + S - 2 < nr)
      wait_vmcnt<(S - 2) * IPW>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();  // round r landed for every wave; slot of round r-1 is free
    if (step + S - 1 < nr) issue(r + S - 1, (step + S - 1) % S);
    const int kt = r * KS + ks;  // this wave's tile
    // this wave's K tile of the round in LDS (a scalar: the per-lane offsets add to it)
    const int kt_off = __builtin_amdgcn_readfirstlane((step % S) * STAGE_BYTES + ks * 2 * TILE_BYTES);
    const char *ks_ptr = smem + kt_off;
    const char *vs = ks_ptr + TILE_BYTES;
    const int k0 = kt * BKV;
    if (wave_live && kt < ntiles && k0 <= wave_kmax) {
      // ---- S^T = K . Q^T - m (lane: one query, 32 of its keys in two 32-key tiles)
      f32x16 s[2] = {(f32x16){}, (f32x16){}};
      if constexpr (XSTEP) {
        mma_32x32x16(s[0], kx, qx);
        mma_32x32x16(s[1], kx, qx);
      }
      // With four key groups (short sequences: 16 waves per workgroup) a wave raises its
      // issue priority over its MFMA loops, so others' softmax fills the gaps.
      if constexpr (KS == 4) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int st = 0; st < DS; ++st) {
        const lds_char *kp = lds_base(ks_ptr + koff[st]);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int row = 32 * i + ql;
          Frag<T> kf;
          if constexpr (ES == 2) {
            kf.v = __builtin_bit_cast(decltype(kf.v), *(const __attribute__((address_space(3))) Chunk16 *)(kp + 32 * i * RB));
          } else {
            const Chunk16 lo = *reinterpret_cast<const Chunk16 *>(ks_ptr + swz<RB, ES>(row, 16 * st + half * 8));
            const Chunk16 hi = *reinterpret_cast<const Chunk16 *>(ks_ptr + swz<RB, ES>(row, 16 * st + half * 8 + 4));
            kf.v = (f32x8){__uint_as_float(lo[0]), __uint_as_float(lo[1]), __uint_as_float(lo[2]), __uint_as_float(lo[3]),
                           __uint_as_float(hi[0]), __uint_as_float(hi[1]), __uint_as_float(hi[2]), __uint_as_float(hi[3])};
          }
          mma_32x32x16(s[i], kf, qf[st]);
        }
      }
      if constexpr (KS == 4) __builtin_amdgcn_s_setprio(0);
      // ---- online softmax. A key split may meet tiles where some of its queries see no
      // key yet: their max stays -inf and their probabilities 0.
      const bool need_mask = k0 + BKV - 1 > q0 + a.q_key_off;
      if constexpr (MASKED) {
        unsigned long long kb = ~0ull;  // bit j: key k0 + j may be attended (lane j loads its byte)
        if (a.key_mask) {
          const int kj = k0 + lane;
          kb = __ballot(kj < nkeys && a.key_mask[(size_t)b * a.mask_ld + kj] != 0);
        }
        const int kmin = a.window > 0 ? my_kmax - a.window + 1 : 0;  // this query's window
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int j = 32 * i + acc_row(e, lane);
            if (!((kb >> j) & 1ull) || k0 + j < kmin) s[i][e] = -INFINITY;
          }
      }
      // The causal cut, on the tiles that cross the diagonal only (a branch on a wave-
      // uniform condition: left as a select inside the max loop, the compiler evaluated
      // the 32 compares on every tile).
      if (__builtin_expect(need_mask, 0)) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            if (k0 + 32 * i + acc_row(rr, lane) > my_kmax) s[i][rr] = -INFINITY;
      }
      if constexpr (!XSTEP) {
        const float mb = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) s[i][rr] = fmaf(s[i][rr], c_log2, -mb);
      }
      float mx = -INFINITY;  // the tile's max of s * c - m (s * c while m_run is -inf)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[i][rr]);
      mx = max_lane32(mx);
      // The reference moves only when a tile's max passes it by more than 2^8 (softmax is
      // unchanged by the reference; p <= 256 stays far inside bf16's and float's range), so
      // the rescale of O, l and the tile's scores runs on few tiles: the first, and the
      // rare later jumps.
      const bool grow = mx > (m_run == -INFINITY ? -INFINITY : ATTN_REF_SLACK);
      if (__any(grow)) {
        const float mb = m_run == -INFINITY ? 0.f : m_run;
        const float m_new = grow ? mb + mx : m_run;  // the new reference: the tile's max
        const float sh = grow ? m_new - mb : 0.f;  // the scores' reference moves up by sh
        const float alpha = m_new == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
#pragma unroll
        for (int i = 0; i < 2; ++i) s[i] -= sh;
        m_run = m_new;
        if constexpr (XSTEP) {
          // -m_run as hi + mid + lo, each the bf16 rounding of what the parts before
          // leave: 3 x 8 significant bits hold the float exactly, and the MFMA's float
          // sum of the three is exact too
          const float nm = (half == 0 && m_run != -INFINITY) ? -m_run : 0.f;
          const T hi = from_f32<T>(nm);
          const float r1 = nm - (float)hi;
          const T mid = from_f32<T>(r1);
          qx.v[0] = hi;
          qx.v[1] = mid;
          qx.v[2] = from_f32<T>(r1 - (float)mid);
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) s[i][rr] = __builtin_amdgcn_exp2f(s[i][rr]);
      // ---- O^T += V^T . P^T. Element e of a lane's 8 values in key step sg is key
      // 16 sg + 8 (e / 4) + 4 half + e % 4, for P (from the score registers) and V alike.
      // With bf16 operands the row sum l adds the rounded p the MFMAs take, two at a time
      // (v_dot2_f32_bf16 against (1, 1), float accumulation).
      float ls = 0.f;
      if constexpr (KS == 4) __builtin_amdgcn_s_setprio(1);
      const lds_char *vp[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vp[dt] = lds_base(vs + voff[dt]);
#pragma unroll
      for (int sg = 0; sg < 4; ++sg) {
        Frag<T> pf;
        if constexpr (ES == 2) {
          typedef __bf16 b2 __attribute__((ext_vector_type(2)));
          typedef float f2 __attribute__((ext_vector_type(2)));
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float p0 = s[sg >> 1][8 * (sg & 1) + e], p1 = s[sg >> 1][8 * (sg & 1) + e + 1];
            const b2 pk = __builtin_convertvector((f2){p0, p1}, b2);
            pf.v[e] = pk[0];
            pf.v[e + 1] = pk[1];
            ls = __builtin_amdgcn_fdot2_f32_bf16(pk, (b2){(__bf16)1.0f, (__bf16)1.0f}, ls, false);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pf.v[e] = s[sg >> 1][8 * (sg & 1) + e];
            ls += s[sg >> 1][8 * (sg & 1) + e];
          }
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          Frag<T> vf;
          if constexpr (ES == 2) {
            typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
            u32x4v raw;
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
              const u16x4 t = __builtin_bit_cast(u16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                  (__attribute__((address_space(3))) half4 *)(vp[dt] + (16 * sg + 8 * pp) * RB)));
              raw[2 * pp] = (uint32_t)t[0] | ((uint32_t)t[1] << 16);
              raw[2 * pp + 1] = (uint32_t)t[2] | ((uint32_t)t[3] << 16);
            }
            vf.v = __builtin_bit_cast(decltype(vf.v), raw);
          } else {
            const int d = 32 * dt + ql;
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int row = 16 * sg + 8 * pp + 4 * half + e;
                vf.v[4 * pp + e] = *reinterpret_cast<const float *>(vs + row * RB + (((d >> 2) ^ att_slot(row)) << 4) + (d & 3) * 4);
              }
          }
          mma_32x32x16(o[dt], vf, pf);
        }
      }
      if constexpr (KS == 4) __builtin_amdgcn_s_setprio(0);
      l_run += ls;
    }
  }

  if constexpr (KS > 1) {
    // ---- merge the key splits: splits 1..KS-1 park (o, m, l) in LDS, split 0 folds
    // them into its own state. A split that saw no key has max -inf and weight 0
    // (split 0 saw tile 0, so without a mask its max is finite).
    __syncthreads();  // every wave is done with the ring
    float *part = reinterpret_cast<float *>(smem);
    if (ks > 0) {
      float *pw = part + ((ks - 1) * G * QW + hq) * PSTATE * 64;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) pw[(dt * 16 + rr) * 64 + lane] = o[dt][rr];
      pw[(DT * 16) * 64 + lane] = m_run;
      pw[(DT * 16 + 1) * 64 + lane] = l_run;
    }
    __syncthreads();
    if (ks > 0) return;
    float m_tot = m_run;
#pragma unroll
    for (int k = 1; k < KS; ++k) m_tot = fmaxf(m_tot, part[(((k - 1) * G * QW + hq) * PSTATE + DT * 16) * 64 + lane]);
    const float f0 = (MASKED && m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_tot);
    l_run *= f0;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= f0;
#pragma unroll
    for (int k = 1; k < KS; ++k) {
      const float *pr = part + ((k - 1) * G * QW + hq) * PSTATE * 64;
      const float mk = pr[(DT * 16) * 64 + lane];
      const float fk = (mk == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mk - m_tot);
      l_run += fk * pr[(DT * 16 + 1) * 64 + lane];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) o[dt][rr] += fk * pr[(dt * 16 + rr) * 64 + lane];
    }
  }

  if (!wave_live || q0 + ql >= a.T) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  QT *op = (QT *)a.o + (size_t)(b * a.T + q0 + ql) * ldq + h * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) op[32 * dt + acc_row(rr, lane)] = from_f32<QT>(o[dt][rr] * inv);
}

template <typename T, int D, int G, int QW, int KS>
static hipError_t launch_attn_cfg(const AttnArgs &a, hipStream_t s) {
  // LDS ring: 3 rounds when a round is small, else 2.
  constexpr int ROUND = KS * 2 * 64 * D * (int)sizeof(T);
  constexpr int S = (3 * ROUND <= 98304) ? 3 : 2;
  const int nqb = (a.T + 32 * QW - 1) / (32 * QW);
  const dim3 grid(nqb * a.B * a.n_kv), block(64 * G * QW * KS);
  if (a.key_mask || a.window > 0) return launch(attn_prefill_kernel<T, D, G, QW, KS, S, true>, grid, block, s, a);
  return launch(attn_prefill_kernel<T, D, G, QW, KS, S, false>, grid, block, s, a);
}

template <typename T, int D, int G>
static hipError_t launch_attn_g(const AttnArgs &a, hipStream_t s) {  // T: storage type
  // Short sequences have few key tiles per query block and too few workgroups to
  // fill the chip: split each block's keys over 4 wave groups (one workgroup per
  // 32 queries). Long ones have work enough; 64 queries per workgroup halve the
  // K/V traffic per query, and at head_dim 64 two key groups still pay: the longest
  // query blocks, which bound the kernel, walk half their keys each (1 x 8192:
  // 260 -> 162 us; four groups of 32 queries 199, two of 32 257, one of 64 260;
  // float caches keep one group, whose registers would spill).
  // The split count is capped so that a 2-round ring of KS K+V tile pairs fits LDS.
  constexpr int PAIR = 2 * 64 * D * (int)sizeof(T);
  constexpr bool can4 = 2 * 4 * PAIR <= 160 * 1024 && G * 4 <= 16;
  constexpr bool can2 = 2 * 2 * PAIR <= 160 * 1024 && G * 2 <= 16;
  const int keys = a.T + a.q_key_off;
  if (can4 && keys <= 1024) return launch_attn_cfg<T, D, G, 1, can4 ? 4 : 1>(a, s);
  const bool big = G == 1 || (long)a.B * a.n_kv * ((a.T + 63) / 64) >= 256;
  // head_dim 128 (bf16) past 2048 keys with work enough: 64 queries, one key group
  // (SmolLM3-3B shape at batch 2 x seq 4096: 283 -> 230 us; one group of 32 queries 432)
  const bool d128_long = D == 128 && sizeof(T) == 2 && keys > 2048 && big;
  if (can2 && keys <= 4096 && !d128_long) return launch_attn_cfg<T, D, G, 1, can2 ? 2 : 1>(a, s);
  if constexpr (D == 64 && can2 && G <= 3 && sizeof(T) == 2)
    return big ? launch_attn_cfg<T, D, G, 2, 2>(a, s) : launch_attn_cfg<T, D, G, 1, 2>(a, s);
  if (big) return launch_attn_cfg<T, D, G, 2, 1>(a, s);
  return launch_attn_cfg<T, D, G, 1, 1>(a, s);
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
