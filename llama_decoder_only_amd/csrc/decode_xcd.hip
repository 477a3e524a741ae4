// The decode step of a bfloat16 SmolLM2-shaped model as one persistent launch,
// partitioned by XCD.
//
// What it computes is the decode step of the pages: every layer of the stack runs
// once on the new token of each sequence, whose key and value join the cache at
// position P = cache_len[b], and the new token attends to keys 0 .. P (Sualeh77
// model.py, "4. Attention", the cache branch; "7. Top-level", cached generation).
//
// Why one launch: at batch 64 every projection of a layer is a few megabytes of
// weights against 64 rows, so as separate kernels each is bound by its launch,
// its first memory round trip and its store drain (about 7 us apiece, seven per
// layer), not by bytes. Here the 256 workgroups stay resident for the whole step
// and move from phase to phase behind barriers.
//
// Why by XCD: the step is independent per sequence, so XCD g (workgroups with
// blockIdx.x % 8 == g, which the hardware places on XCD g) owns the sequences
// b = g, g + 8, ... (at most 16 rows) and runs the whole stack for them alone.
// Everything one phase hands to the next stays inside that XCD's L2: producers
// write with plain stores, consumers read with agent-coherent (sc1) loads, which
// see the lines the XCD's L2 holds dirty; a barrier is a flag per workgroup that
// its group polls. No fence writes back or invalidates an L2 (on this part such a
// fence costs tens of microseconds). Each XCD reads the full weights; the copies
// the other seven XCDs read at about the same time come from the memory-side
// cache (MALL), not from HBM.
//
// Phases of one layer, each ending at the group barrier:
//   QKV   u = RMSNorm(x; attn_norm), q k v = u W^T (RoPE on q, k); k, v into the
//         cache at P                                  (16-column MFMA tiles)
//   ATTN  split-K attention of the new query over keys k_lo .. P, one wavefront
//         per (row, kv head, split), all G query heads of the group per key
//   MERGE the splits of each (row, head) combined into o
//   OPROJ x += o W_o^T
//   GATE  u = RMSNorm(x; mlp_norm), y = silu(u W_g^T) * (u W_u^T)
//   DOWN  x += y W_d^T
// Before the first layer the embedding rows are gathered; after the last, the
// final RMSNorm leaves the head's operand (xs times 2^-8, with its row sums of
// squares) for the tied lm_head GEMM, which runs as its own launch.
//
// Weights: a phase's MFMA B fragments (16 B of one weight row per lane) are loaded
// into registers right after the workgroup arrives at the barrier before that
// phase, so their memory latency overlaps the wait. The contraction of each tile is
// split over the workgroup's eight wavefronts by K step and summed through LDS.
//
// Failure: a step whose barriers are still waiting ~1 s after it started (a workgroup that
// never became resident) sets the abort word; every workgroup then leaves, and the
// group's head operand rows are set to NaN, so that the step's logits come out NaN. The
// limit is a kernel argument (decode_xcd_deadline_ticks), which lets a test force the
// path from the host.
#include "common.h"
#include "kernels.h"
#include "decode_xcd.h"

#include <cstdlib>

namespace smol {

namespace {

constexpr int DX_WAVES = 4, DX_THREADS = 64 * DX_WAVES;
constexpr int DX_ROWS = 16;                 // rows per XCD group: the MFMA tile's M
constexpr int DX_D = 64;                    // head_dim
constexpr int DX_KPAD = DX_KMAX + 8;        // LDS row of the staged A operand of the down projection (f16)
constexpr int DX_KPAD_H = DX_HMAX + 8;      // the same for the contractions over the hidden size
constexpr int DX_TMAX = 2 * DX_UMAX;        // tiles per workgroup and phase
constexpr int SC1 = 16;                     // buffer-op cache policy: agent-coherent

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dx_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ Chunk16 ld_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, SC1);
}
__device__ __forceinline__ float ld_sc1_f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, SC1));
}
__device__ __forceinline__ uint32_t poll_u32(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int xcc_id() { return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 15; }

// --------------------------------------------------------------- group barrier
struct DxSync {
  uint32_t *flags;  // this group's flags, one per workgroup, 16 words apart
  uint32_t *abort;
  int nwx, m;
  uint32_t phase;
  unsigned long long deadline;
};

// Every store of this workgroup is complete, then its flag says so.
__device__ __forceinline__ void dx_arrive(DxSync &s, bool drain = true) {
  if (drain) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  ++s.phase;
  if (threadIdx.x == 0) *(volatile uint32_t *)(s.flags + s.m * 16) = s.phase;
}

// Wait until every workgroup of the group has arrived; false: the step is aborted.
__device__ __forceinline__ bool dx_wait(DxSync &s, int *bad) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    for (;;) {
      const uint32_t f = lane < s.nwx ? poll_u32(s.flags + lane * 16) : s.phase;
      if (__all(f >= s.phase)) break;
      if (poll_u32(s.abort) != 0) { if (lane == 0) *bad = 1; break; }
      if (wall_clock64() > s.deadline) {
        if (lane == 0) {
          __hip_atomic_store(s.abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          *bad = 1;
        }
        break;
      }
    }
  }
  __syncthreads();
  return *bad == 0;
}

// --------------------------------------------------------------- GEMM phases
// A phase computes 16-column output tiles ("units") for the group's rows; unit u
// goes to workgroup u % nwx. Tile t = (k, mat) of a workgroup is its k-th unit's
// matrix mat (gate/up have two). Wavefront w of the workgroup's four takes the K
// steps w, w + 4, ... of every tile: fragment fr[t * IMAX + i] is K step w + 4 i.

// Weights of local unit k, matrix mat: the unit's first row (uniform) and the row
// offset of lane slot `slot` (output column) in elements (32-bit, per lane).
struct DxRows {
  const bf16 *w0, *w1, *w2;
  int kind;  // 0 QKV, 1 o_proj / down, 2 gate/up
  int K, nq, nkv, nwx, m;
  __device__ __forceinline__ const bf16 *base(int k, int mat) const {
    const int u = m + k * nwx;
    if (kind == 0) {
      const int hsl = u >> 2, c = u & 3;
      if (hsl < nq) return w0 + (size_t)(hsl * DX_D + c * 8) * K;
      if (hsl < nq + nkv) return w1 + (size_t)((hsl - nq) * DX_D + c * 8) * K;
      return w2 + (size_t)((hsl - nq - nkv) * DX_D + c * 16) * K;
    }
    return (kind == 2 && mat ? w1 : w0) + (size_t)(u * 16) * K;
  }
  // q or k units take dims c*8 + (slot & 7) and their rotation partners 32 above
  __device__ __forceinline__ uint32_t lane_rows(int k, int slot) const {
    const int hsl = (m + k * nwx) >> 2;
    const bool pairs = kind == 0 && hsl < nq + nkv;
    return (uint32_t)((pairs ? (slot & 7) + (slot >> 3) * 32 : slot) * K);
  }
};

template <int TMAX, int IMAX, int MATS, int N, int NW = DX_WAVES>
__device__ __forceinline__ void dx_prefetch(Chunk16 (&fr)[N], const DxRows &r, int nu, int KS) {
  static_assert(TMAX * IMAX <= N, "fragment registers");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int slot = lane & 15, kq = lane >> 4;
  // every slot of the phase is written by every wavefront (zero where unused; only the
  // first NW load), so that no fragment of an earlier phase stays live across this one
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    const int k = t / MATS, mat = t % MATS;
    const int kk = k < nu ? k : 0;
    const bf16 *p = r.base(kk, mat);
    const uint32_t lo = r.lane_rows(kk, slot) + 8 * kq + 32 * w;
#pragma unroll
    for (int i = 0; i < IMAX; ++i) {
      Chunk16 v = {0u, 0u, 0u, 0u};
      if (w < NW && k < nu && w + NW * i < KS) v = ld16(p + (lo + 32 * NW * i));
      fr[t * IMAX + i] = v;
    }
  }
}

// Direct copies of a phase's B fragments into LDS ([tile][K step][lane] x 16 bytes), all
// by the calling wavefront.
template <int MATS>
__device__ __forceinline__ void dx_weights_to_lds(const DxRows &r, int nu, int KS, uint32_t bl) {
  const int lane = threadIdx.x & 63, slot = lane & 15, kq = lane >> 4;
  for (int t = 0; t < nu * MATS; ++t) {
    const int k = t / MATS, mat = t % MATS;
    const bf16 *p = r.base(k, mat) + r.lane_rows(k, slot) + 8 * kq;
    for (int s = 0; s < KS; ++s)
      asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(p + 32 * s), "{m0}"(bl + (uint32_t)((t * KS + s) * 1024))
                   : "memory");
  }
}

// acc[t] = this wavefront's share of tile t; then the eight shares are summed in
// LDS and wavefront t (MATS = 1) or k (MATS = 2, both of unit k's tiles) holds the
// result: rows 4 (lane / 16) + i, column lane % 16.
// B fragments from registers (fr) or, with BLDS, from LDS at BL laid out
// [tile][K step][lane] x 16 bytes (KS steps per tile). K step s goes to wavefront s % NW.
template <int TMAX, int IMAX, int MATS, int N, int NW, int LDA, bool BLDS>
__device__ __forceinline__ void dx_mma(Chunk16 (&fr)[N], const char *BL, int nu, int KS, const bf16 *Ah, const bf16 *Al, f32x4 *red,
                                       f32x4 (&res)[2]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = lane & 15, kq = lane >> 4;
  f32x4 acc[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // K step outermost: the A fragments (hi, lo) of a step serve every tile. No branches
  // inside (they would copy the accumulators at every join): a step past K reads a
  // valid A step and a zero B fragment, an unused tile multiplies a zero B fragment.
  if (w < NW) {
#pragma unroll
    for (int i = 0; i < IMAX; ++i) {
      const int s = w + NW * i;
      const int sa = s < KS ? s : KS - 1;
      const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(Ah + row * LDA + 32 * sa + 8 * kq);
      const bf16x8 al = *reinterpret_cast<const bf16x8 *>(Al + row * LDA + 32 * sa + 8 * kq);
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {
        Chunk16 bw;
        if constexpr (BLDS) {
          const bool ok = s < KS && t / MATS < nu;
          const Chunk16 rd = *reinterpret_cast<const Chunk16 *>(BL + ((size_t)((ok ? t : 0) * KS + sa) * 64 + lane) * 16);
          bw = ok ? rd : (Chunk16){0u, 0u, 0u, 0u};
        } else {
          bw = fr[t * IMAX + i];  // zero where the step or the tile is unused (dx_prefetch)
        }
        const bf16x8 b = __builtin_bit_cast(bf16x8, bw);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b, acc[t], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // red may alias the staged A operand
  const int nt = nu * MATS;
  if (w < NW) {
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
      if (t < nt) red[(w * DX_TMAX + t) * 64 + lane] = acc[t];
  }
  __syncthreads();
  if (w < nu) {
#pragma unroll
    for (int mat = 0; mat < MATS; ++mat) {
      const int t = MATS == 1 ? w : w * 2 + mat;
      f32x4 s4 = red[t * 64 + lane];
#pragma unroll
      for (int v = 1; v < NW; ++v) s4 += red[(v * DX_TMAX + t) * 64 + lane];
      res[mat] = s4;
    }
  }
  // red is reused by the next phase only after its barrier
}

// The staged A operand is the exact-ish sum of two bf16 tiles, hi = bf16(u) and
// lo = bf16(u - hi) (16 significant bits; a float16 value is represented exactly), so
// that the MFMAs take the bf16 weights as they are: two bf16 MFMAs per fragment, no
// conversion of B.
__device__ __forceinline__ void dx_split4(bf16 *h, bf16 *l, const float (&u)[4]) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 hv, lv;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hv[e] = (bf16)u[e];
    lv[e] = (bf16)(u[e] - (float)hv[e]);
  }
  *reinterpret_cast<bf16x4 *>(h) = hv;
  *reinterpret_cast<bf16x4 *>(l) = lv;
}

// Stage u = RMSNorm(x rows; w) of the group's rows (hi into Ah, lo into Al). Thread t
// serves row t / TPR (16 rows x TPR threads), columns 4 (t % TPR) + 4 TPR i. The norm
// weights of those columns arrive in wb (dx_norm_prefetch, issued just before, so that
// both round trips overlap; requesting them before the phase's barrier instead, with
// the weight fragments, measured slower).
constexpr int DX_TPR = DX_THREADS / DX_ROWS, DX_NIT = (DX_HMAX + 4 * DX_TPR - 1) / (4 * DX_TPR);
__device__ __forceinline__ void dx_norm_prefetch(uint2 (&wb)[DX_NIT], const bf16 *w, int H, int R) {
  const int t = threadIdx.x, j = t / DX_TPR, c = t % DX_TPR;
#pragma unroll
  for (int i = 0; i < DX_NIT; ++i) {
    const int col = 4 * c + 4 * DX_TPR * i;
    wb[i] = make_uint2(0u, 0u);
    if (j < R && col < H) wb[i] = *reinterpret_cast<const uint2 *>(w + col);
  }
}

template <int LDA>
__device__ __forceinline__ void dx_stage_norm(bf16 *Ah, bf16 *Al, __amdgpu_buffer_rsrc_t xr, const uint2 (&wb)[DX_NIT],
                                              int H, float eps, int g, int R) {
  const int t = threadIdx.x, j = t / DX_TPR, c = t % DX_TPR;
  const int b = g + 8 * j;
  f32x4 v[DX_NIT];
#pragma unroll
  for (int i = 0; i < DX_NIT; ++i) {
    const int col = 4 * c + 4 * DX_TPR * i;
    v[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    if (j < R && col < H) {
      const Chunk16 ch = ld_sc1(xr, (uint32_t)((b * H + col) * 4));
      v[i] = (f32x4){__uint_as_float(ch[0]), __uint_as_float(ch[1]), __uint_as_float(ch[2]), __uint_as_float(ch[3])};
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < DX_NIT; ++i) ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
#pragma unroll
  for (int o = DX_TPR / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  if (j < R) {
#pragma unroll
    for (int i = 0; i < DX_NIT; ++i) {
      const int col = 4 * c + 4 * DX_TPR * i;
      if (col < H) {
        const float u[4] = {v[i][0] * r * __uint_as_float(wb[i].x << 16), v[i][1] * r * __uint_as_float(wb[i].x & 0xffff0000u),
                            v[i][2] * r * __uint_as_float(wb[i].y << 16), v[i][3] * r * __uint_as_float(wb[i].y & 0xffff0000u)};
        dx_split4(Ah + j * LDA + col, Al + j * LDA + col, u);
      }
    }
  }
  __syncthreads();
}

// Stage float16 rows [R, K] (row stride ld elements) of the group (hi into Ah, lo into
// Al), by the first NT threads only: the others may have copies in flight that must
// not be waited for here. Every load of a thread (16 bytes each, at most IT) is
// requested before any is used.
template <int LDA, int NT, int KMAXS>
__device__ __forceinline__ void dx_stage_rows(bf16 *Ah, bf16 *Al, __amdgpu_buffer_rsrc_t src, int ld, int K, int g,
                                              int R) {
  constexpr int IT = (DX_ROWS * KMAXS / 8 + NT - 1) / NT;
  const int per_row = K / 8, n = R * per_row;
  if (threadIdx.x < NT) {
    Chunk16 v[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int it = min((int)threadIdx.x + i * NT, n - 1);
      const int j = it / per_row, c = (it % per_row) * 8;
      v[i] = ld_sc1(src, (uint32_t)(((size_t)(g + 8 * j) * ld + c) * 2));
    }
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int it = threadIdx.x + i * NT;
      if (it < n) {
        const int j = it / per_row, c = (it % per_row) * 8;
        float u0[4], u1[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u0[e] = (float)chunk_elem<f16>(v[i], e);
          u1[e] = (float)chunk_elem<f16>(v[i], 4 + e);
        }
        dx_split4(Ah + j * LDA + c, Al + j * LDA + c, u0);
        dx_split4(Ah + j * LDA + c + 4, Al + j * LDA + c + 4, u1);
      }
    }
  }
  __syncthreads();
}

}  // namespace

// ------------------------------------------------------------------ attention item
// One wavefront's item: keys [k0, k1) of kv head h of row b (position P), all G query
// heads of the group. Lane (kr = lane / 8, dl = lane % 8) holds dims 8 dl .. 8 dl + 7
// of keys kb + kr + 8 i (i < DX_KPL) of each block of DX_BLK keys; the next block's
// keys and values are requested before the current block is used. Online softmax over the blocks in
// base 2 (scores carry log2(e) / sqrt(d)); the partial (max, sum, o) goes to part.
namespace {

constexpr int DX_BLK = 32;                 // keys per block
constexpr int DX_SLOT = 2 * DX_BLK * DX_D * 2;  // LDS bytes of one block: its keys, then its values
constexpr int DX_NSLOT = 4;                // blocks in flight per wavefront
constexpr float DX_REF_SLACK = 8.0f;       // log2 units a score may pass the softmax reference
constexpr int DX_CPB = DX_BLK * DX_D * 2 / 1024;  // 1 KB copies per block and matrix (4)

typedef __fp16 dx_half4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// 16-byte chunk c of key row r sits at chunk slot c ^ perm(r) of its 128-byte row, a
// bijection of r mod 8 under which the K fragment reads (16 rows, one chunk each) and
// the transposing V reads (4 rows x 2 adjacent chunks per 16 lanes) meet distinct banks.
__device__ __forceinline__ int dx_perm(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

// Direct copy of 16 bytes per lane into LDS (lane l's bytes land at lds_base + 16 l),
// agent-coherent (the new token's row was written in this launch by another CU).
__device__ __forceinline__ void dx_dma16(const void *g, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off sc1" ::"v"(g), "{m0}"(lds_base) : "memory");
}
__device__ __forceinline__ void dx_wait_blocks(int younger) {  // at most `younger` blocks' copies outstanding
  if (younger >= 3) wait_vmcnt<3 * 2 * DX_CPB>();
  else if (younger == 2) wait_vmcnt<2 * 2 * DX_CPB>();
  else if (younger == 1) wait_vmcnt<2 * DX_CPB>();
  else wait_vmcnt<0>();
}
static_assert(DX_NSLOT == 4, "dx_wait_blocks counts up to three younger blocks");

// Request block blk of the item (keys k0 + DX_BLK blk ..) into its ring slot: copy i
// of a matrix covers rows 8 i .. 8 i + 7; lane l fills row 8 i + l / 8, chunk slot l % 8
// with the row's chunk (l % 8) ^ perm(row). Rows past k1 repeat row k1 - 1.
__device__ __forceinline__ void dx_kv_issue(const bf16 *kb_, const bf16 *vb_, uint32_t wring, int k0, int blk, int k1,
                                            int lane) {
  const int kb = k0 + blk * DX_BLK;
  const uint32_t slot = wring + (uint32_t)((blk % DX_NSLOT) * DX_SLOT);
#pragma unroll
  for (int i = 0; i < DX_CPB; ++i) {
    const int row = 8 * i + (lane >> 3);
    const int key = min(kb + row, k1 - 1);
    const int chunk = (lane & 7) ^ dx_perm(row);
    dx_dma16(kb_ + (size_t)key * DX_D + chunk * 8, slot + i * 1024);
    dx_dma16(vb_ + (size_t)key * DX_D + chunk * 8, slot + DX_CPB * 1024 + i * 1024);
  }
}

// One block of the item on bf16 MFMAs, the cache's own type (no conversion). S^T =
// K Q^T (keys x heads, 16x16x32; the G heads are columns 0 .. G-1 of a zero-padded 16)
// with q as the exact sum of two bf16 parts (q is float16: 11 significant bits fit in
// 8 + 8): lane l holds keys 4 g + i (tile 0) and 16 + 4 g + i (tile 1) of head l % 16,
// g = l / 16. Those eight probabilities, split the same way into bf16 hi + lo, are
// directly the B operands of O^T = V^T P^T (dims x heads) with the contraction order
// "key 4 g + e, then 16 + 4 g + e"; the V^T operand takes the same order from two
// transposing reads. Scores carry log2(e) / sqrt(d); online softmax in base 2.
template <bool MASKED>
__device__ __forceinline__ void dx_kv_block_mfma(const char *slot, int kb, int k1, int lane, const uint8_t *mrow,
                                                 const bf16x8 (&qh)[2], const bf16x8 (&ql)[2], float &mx, float &lsum,
                                                 f32x4 (&o)[4]) {
  const int g = lane >> 4, l16 = lane & 15;
  const char *ks = slot, *vs = slot + DX_CPB * 1024;
  f32x4 st[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    st[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const int row = 16 * mt + l16;
#pragma unroll
    for (int kst = 0; kst < 2; ++kst) {
      const int chunk = 4 * kst + g;  // dims 32 kst + 8 g
      const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(ks + row * 128 + ((chunk ^ dx_perm(row)) << 4));
      st[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qh[kst], st[mt], 0, 0, 0);
      st[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, ql[kst], st[mt], 0, 0, 0);
    }
  }
  const float c_log2 = 1.4426950408889634f * 0.125f;  // log2(e) / sqrt(64)
  float sc[8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kb + 16 * mt + 4 * g + i;
      bool keep = key < k1;
      if constexpr (MASKED) keep = keep && mrow[min(key, k1 - 1)] != 0;
      sc[4 * mt + i] = keep ? st[mt][i] * c_log2 : -INFINITY;
    }
  float bm = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
  bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
  bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
  // mx is a reference, not the running max: it moves (and the state is rescaled) only
  // when a score passes it by more than 2^8, so p = exp2(s - mx) stays <= 256
  if (__any(bm > mx + DX_REF_SLACK)) {
    const float mn = fmaxf(mx, bm);
    const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mx - mn);  // exp2(-inf) = 0
    lsum *= alpha;
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] *= alpha;
    mx = mn;
  }
  const float mu = mx == -INFINITY ? 0.f : mx;  // nothing kept yet: weights 0
  bf16x8 ph, pl;
  float ps = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float pv = __builtin_amdgcn_exp2f(sc[e] - mu);
    const bf16 hi = (bf16)pv;
    ph[e] = hi;
    pl[e] = (bf16)(pv - (float)hi);
    ps += pv;
  }
  lsum += ps;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    uint32_t raw[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 16 * h + 4 * g + (l16 >> 2);
      const int dim = 16 * t + 4 * (l16 & 3);
      const char *src = vs + row * 128 + (((dim >> 3) ^ dx_perm(row)) << 4) + (dim & 7) * 2;
      const dx_half4 v = __builtin_amdgcn_ds_read_tr16_b64_v4f16((__attribute__((address_space(3))) dx_half4 *)src);
      const u32x2_t u = __builtin_bit_cast(u32x2_t, v);
      raw[2 * h] = u[0];
      raw[2 * h + 1] = u[1];
    }
    const bf16x8 vf = __builtin_bit_cast(bf16x8, (Chunk16){raw[0], raw[1], raw[2], raw[3]});
    o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, ph, o[t], 0, 0, 0);
    o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pl, o[t], 0, 0, 0);
  }
}

}  // namespace

// ------------------------------------------------------------------ the kernel
template <int G, bool MASKED>
__global__ void __launch_bounds__(DX_THREADS, 1) decode_xcd_kernel(const DecodeXcdArgs a) {
  // LDS, one union: [A operand of the hidden-size contractions | reduction buffer] (the
  // latter written after the former is read), then the gate/up weight fragments, which
  // the down projection's wide A operand replaces once they are used; in the attention
  // phase the wavefronts' K/V rings cover it all. Then q of the attention items.
  constexpr int AH_BYTES = DX_ROWS * DX_KPAD_H * 2, AD_BYTES = DX_ROWS * DX_KPAD * 2;  // one bf16 tile
  constexpr int LO_BYTES = 2 * AH_BYTES > DX_WAVES * DX_TMAX * 64 * 16 ? 2 * AH_BYTES : DX_WAVES * DX_TMAX * 64 * 16;
  constexpr int GW_BYTES = 2 * DX_UMAX * (DX_HMAX / 32) * 1024;
  static_assert(2 * AD_BYTES <= GW_BYTES, "the down operand fits the weight region");
  constexpr int RING_BYTES = DX_WAVES * DX_NSLOT * DX_SLOT;
  constexpr int UNION_BYTES = LO_BYTES + GW_BYTES > RING_BYTES ? LO_BYTES + GW_BYTES : RING_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[UNION_BYTES];
  __shared__ __attribute__((aligned(16))) f16 qs[DX_WAVES][16][DX_D];  // the item's G heads, zero-padded to 16
  bf16 *Ah = reinterpret_cast<bf16 *>(smem), *Al = reinterpret_cast<bf16 *>(smem + AH_BYTES);
  f32x4 *red = reinterpret_cast<f32x4 *>(smem);
  char *GW = smem + LO_BYTES;
  bf16 *Adh = reinterpret_cast<bf16 *>(smem + LO_BYTES), *Adl = reinterpret_cast<bf16 *>(smem + LO_BYTES + AD_BYTES);
  __shared__ float2 rope[DX_ROWS][DX_D / 2];
  __shared__ int pos[DX_ROWS];
  __shared__ int bad;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = blockIdx.x & 7, m = blockIdx.x >> 3;
  const int nwx = a.nwx;
  const int R = (a.B - g + 7) / 8;  // rows of this group: b = g + 8 j, j < R
  const int H = a.H, I = a.I, nq = a.nq, nkv = a.nkv;
  const int B = a.B;

  if (tid == 0) {
    bad = 0;
    if (xcc_id() != g) atomicOr(a.ctrl + DX_CTRL_ERR, 1u);  // placement differs: the L2 exchange is not safe
  }
  if (tid < DX_ROWS) pos[tid] = tid < R ? a.cache_len[g + 8 * tid] : -1;
  for (int i = tid; i < UNION_BYTES / 16; i += DX_THREADS) reinterpret_cast<Chunk16 *>(smem)[i] = (Chunk16){0, 0, 0, 0};
  for (int i = tid; i < DX_WAVES * 16 * DX_D / 8; i += DX_THREADS) reinterpret_cast<Chunk16 *>(&qs[0][0][0])[i] = (Chunk16){0, 0, 0, 0};
  __syncthreads();
  for (int e = tid; e < DX_ROWS * DX_D / 2; e += DX_THREADS) {  // RoPE (cos, sin) of each row's position
    const int j = e / (DX_D / 2), i = e % (DX_D / 2);
    rope[j][i] = j < R ? rope_cos_sin(pos[j], a.inv_freq[i]) : make_float2(1.f, 0.f);
  }

  DxSync sy{a.ctrl + DX_CTRL_WORDS + g * nwx * 16, a.ctrl + DX_CTRL_ABORT, nwx, m, 0u, wall_clock64() + a.deadline};
  const __amdgpu_buffer_rsrc_t xr = dx_rsrc(a.x, (uint32_t)((size_t)B * H * 4));
  const __amdgpu_buffer_rsrc_t qr = dx_rsrc(a.q, (uint32_t)((size_t)B * H * 2));
  const __amdgpu_buffer_rsrc_t orr = dx_rsrc(a.o, (uint32_t)((size_t)B * H * 2));
  const __amdgpu_buffer_rsrc_t yr = dx_rsrc(a.y, (uint32_t)((size_t)B * I * 2));
  const __amdgpu_buffer_rsrc_t pr = dx_rsrc(a.part, (uint32_t)((size_t)B * nq * a.sp * (DX_D + 2) * 4));

  // unit counts of the four GEMM phases, and this workgroup's share of each
  const int nu_qkv_all = (nq + 2 * nkv) * 4, nu_h_all = H / 16, nu_i_all = I / 16;
  auto share = [&](int n) { return m < n ? (n - m + nwx - 1) / nwx : 0; };
  const int nu_qkv = share(nu_qkv_all), nu_h = share(nu_h_all), nu_i = share(nu_i_all);
  const int KS_H = H / 32, KS_I = I / 32;
  // K steps per wavefront, at most: the contractions over H on four or (o_proj) three
  // wavefronts, the one over I on four
  constexpr int IM_H = (DX_HMAX / 32 + DX_WAVES - 1) / DX_WAVES, IM_H3 = (DX_HMAX / 32 + 2) / 3;
  constexpr int IM_I = (DX_KMAX / 32 + DX_WAVES - 1) / DX_WAVES;
  constexpr int UR = DX_UREG;  // units per workgroup of the phases fed from registers

  // the B fragments of the next GEMM phase, requested when the workgroup arrives at
  // the barrier before it; every phase writes all the slots it uses (zero where idle)
  constexpr int NFR = UR * (IM_I > IM_H3 ? IM_I : IM_H3);
  Chunk16 fr[NFR];
  uint2 nw[DX_NIT];  // the next norm stage's weights
  f32x4 res[2];

  // ---- embedding rows: workgroup m < R gathers row j = m
  {
    const DxLayer &L0 = a.layer[0];
    DxRows rq{L0.wq, L0.wk, L0.wv, 0, H, nq, nkv, nwx, m};
    if (m < R) {
      const int b = g + 8 * m;
      const int id = a.ids[b];
      const bool ok = id >= 0 && id < a.V;
      for (int c = tid * 4; c < H; c += DX_THREADS * 4) {
        f32x4 v;
        if (ok) {
          const uint2 e = *reinterpret_cast<const uint2 *>(a.embed + (size_t)id * H + c);
          v = (f32x4){__uint_as_float(e.x << 16), __uint_as_float(e.x & 0xffff0000u), __uint_as_float(e.y << 16),
                      __uint_as_float(e.y & 0xffff0000u)};
        } else {
          const float n = __builtin_nanf("");
          v = (f32x4){n, n, n, n};
        }
        *reinterpret_cast<f32x4 *>(a.x + (size_t)b * H + c) = v;
      }
    }
    dx_arrive(sy);
    dx_prefetch<UR, IM_H, 1, NFR>(fr, rq, nu_qkv, KS_H);
    if (!dx_wait(sy, &bad)) goto aborted;
  }

  for (int l = 0; l < a.L; ++l) {
    const DxLayer &Ly = a.layer[l];
    const bool rope_on = !(a.nope_every > 0 && (l + 1) % a.nope_every == 0);
    const int window = (!rope_on && a.window > 0) ? a.window : 0;
    bf16 *kc = a.kc + (size_t)l * B * nkv * a.cap * DX_D;
    bf16 *vc = a.vc + (size_t)l * B * nkv * a.cap * DX_D;

    // ---- QKV + RoPE; k, v into the cache at P
    dx_norm_prefetch(nw, Ly.an, H, R);
    dx_stage_norm<DX_KPAD_H>(Ah, Al, xr, nw, H, a.eps, g, R);
    dx_mma<UR, IM_H, 1, NFR, DX_WAVES, DX_KPAD_H, false>(fr, nullptr, nu_qkv, KS_H, Ah, Al, red, res);
    if (w < nu_qkv) {
      const int u = m + w * nwx, hsl = u >> 2, c = u & 3, slot = lane & 15;
      const int kind = hsl < nq ? 0 : (hsl < nq + nkv ? 1 : 2);
      float other[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) other[i] = __shfl_xor(res[0][i], 8, 64);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 4 * (lane >> 4) + i;
        if (j >= R) continue;
        const int b = g + 8 * j;
        float v = res[0][i];
        int col;
        if (kind != 2) {
          const int f = c * 8 + (slot & 7);  // frequency index; dims f and f + 32
          col = f + (slot >> 3) * 32;
          if (rope_on) {
            const float2 cs = rope[j][f];
            v = slot < 8 ? v * cs.x - other[i] * cs.y : v * cs.x + other[i] * cs.y;
          }
        } else {
          col = c * 16 + slot;
        }
        if (kind == 0) {
          a.q[(size_t)b * H + hsl * DX_D + col] = (f16)v;
        } else {
          const int P = pos[j];
          if (P >= 0 && P < a.cap && P < a.max_pos) {
            const int head = kind == 1 ? hsl - nq : hsl - nq - nkv;
            bf16 *dst = (kind == 1 ? kc : vc) + (((size_t)b * nkv + head) * a.cap + P) * DX_D + col;
            *dst = (bf16)v;
          }
        }
      }
    }
    dx_arrive(sy);

    // ---- attention: item it = (pair, split), pair = (row j, kv head h); wavefront w * nwx + m.
    // Keys and values stream through the wavefront's LDS ring, DX_NSLOT blocks in
    // flight. The first blocks that lie wholly below P (not written in this step) are
    // requested before the barrier, except by wavefront 0, which polls the barrier (the
    // poll's loads would wait for its copies: loads complete in order). Handing wavefront
    // 0's first blocks to wavefront 1, with a sync after the barrier, measured slower.
    {
      const int sp = a.sp;
      struct Item {
        bool has;
        int b, h, s, P, k0, k1;
      };
      auto item = [&](int wv) {
        Item t;
        const int it = wv * nwx + m;
        t.has = it < R * nkv * sp;
        const int pair = t.has ? it / sp : 0;
        t.s = t.has ? it % sp : 0;
        const int j = pair / nkv;
        t.h = pair % nkv;
        t.b = g + 8 * j;
        t.P = t.has ? pos[j] : -1;
        const bool valid = t.P >= 0 && t.P < a.cap && t.P < a.max_pos;
        const int k_lo = valid ? (window > 0 ? max(0, t.P - window + 1) : 0) : 0;
        const int n = valid ? t.P + 1 - k_lo : 0;
        t.k0 = k_lo + (int)((long)t.s * n / sp);
        t.k1 = k_lo + (int)((long)(t.s + 1) * n / sp);
        return t;
      };
      // the first blocks of an item that can be requested before the barrier
      auto early_blocks = [&](const Item &t) {
        const int nb = t.k1 > t.k0 ? (t.k1 - t.k0 + DX_BLK - 1) / DX_BLK : 0;
        int e = 0;
        while (e < nb && e < DX_NSLOT && t.k0 + (e + 1) * DX_BLK <= t.P) ++e;
        return e;
      };
      const Item me = item(w);
      const bool has = me.has;
      const int b = me.b, h = me.h, s = me.s, P = me.P, k0 = me.k0, k1 = me.k1;
      const int nblk = k1 > k0 ? (k1 - k0 + DX_BLK - 1) / DX_BLK : 0;
      const size_t kvbase = ((size_t)b * nkv + h) * a.cap * DX_D;
      const bf16 *kb_ = kc + kvbase, *vb_ = vc + kvbase;
      const uint32_t wring_off = (uint32_t)(w * DX_NSLOT * DX_SLOT);
      const uint32_t wring = lds_addr(smem) + wring_off;
      const int first = nblk < DX_NSLOT ? nblk : DX_NSLOT;
      const int early = early_blocks(me);
      if (w != 0)
        for (int e = 0; e < early; ++e) dx_kv_issue(kb_, vb_, wring, k0, e, k1, lane);
      if (!dx_wait(sy, &bad)) goto aborted;
      int issued = w != 0 ? early : 0;
      if (has) {
        // q of the G heads into rows 0 .. G-1 of the wave's zero-padded tile, then the
        // remaining first blocks
        if (lane < 8 * G)
          dx_dma16(a.q + (size_t)b * H + (h * G + (lane >> 3)) * DX_D + (lane & 7) * 8, lds_addr(&qs[w][0][0]));
        wait_vmcnt<0>();
        const int gq = lane >> 4, l16 = lane & 15;
        bf16x8 qh[2], ql[2];  // q = qh + ql exactly
#pragma unroll
        for (int kst = 0; kst < 2; ++kst) {
          const f16x8 qv = *reinterpret_cast<const f16x8 *>(&qs[w][l16][32 * kst + 8 * gq]);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float f = (float)qv[e];
            const bf16 hi = (bf16)f;
            qh[kst][e] = hi;
            ql[kst][e] = (bf16)(f - (float)hi);
          }
        }
        while (issued < first) {
          dx_kv_issue(kb_, vb_, wring, k0, issued, k1, lane);
          ++issued;
        }
        float mx = -INFINITY, lsum = 0.f;
        f32x4 o[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) o[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
        const uint8_t *mrow = a.key_mask ? a.key_mask + (size_t)b * a.mask_ld : nullptr;
        for (int blk = 0; blk < nblk; ++blk) {
          dx_wait_blocks(issued - blk - 1);
          dx_kv_block_mfma<MASKED>(smem + wring_off + (blk % DX_NSLOT) * DX_SLOT, k0 + blk * DX_BLK, k1, lane, mrow,
                                   qh, ql, mx, lsum, o);
          if (blk + DX_NSLOT < nblk) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the slot's reads are done
            dx_kv_issue(kb_, vb_, wring, k0, blk + DX_NSLOT, k1, lane);
            ++issued;
          }
        }
        // the row sum over the four lane groups (each summed its own keys)
        lsum += __shfl_xor(lsum, 16, 64);
        lsum += __shfl_xor(lsum, 32, 64);
        if (l16 < G) {
          float *pp = a.part + (((size_t)b * nq + h * G + l16) * sp + s) * (DX_D + 2);
          if (gq == 0) {
            pp[0] = mx;
            pp[1] = lsum;
          }
#pragma unroll
          for (int t = 0; t < 4; ++t) *reinterpret_cast<f32x4 *>(pp + 2 + 16 * t + 4 * gq) = o[t];
        }
      }
    }
    {
      dx_arrive(sy);
      if (!dx_wait(sy, &bad)) goto aborted;
    }

    // ---- merge the splits of (row j, head hh): wavefront w * nwx + m, lane = dim
    {
      const int sp = a.sp;
      const int it = w * nwx + m;
      if (it < R * nq) {
        const int j = it / nq, hh = it % nq, b = g + 8 * j;
        const int P = pos[j];
        const bool valid = P >= 0 && P < a.cap && P < a.max_pos;
        const uint32_t base = (uint32_t)(((size_t)b * nq + hh) * sp * (DX_D + 2) * 4);
        float M = -INFINITY, l = 0.f, o = 0.f;
        for (int s0 = 0; s0 < sp; s0 += 8) {
          float ms[8], ls[8], os[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t off = base + (uint32_t)(min(s0 + i, sp - 1) * (DX_D + 2) * 4);
            ms[i] = ld_sc1_f(pr, off);
            ls[i] = ld_sc1_f(pr, off + 4);
            os[i] = ld_sc1_f(pr, off + 8 + lane * 4);
          }
          float mr = M;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (s0 + i < sp) mr = fmaxf(mr, ms[i]);
          const float f = M == -INFINITY ? 0.f : exp2f(M - mr);
          l *= f;
          o *= f;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (s0 + i < sp) {
              const float fi = ms[i] == -INFINITY ? 0.f : exp2f(ms[i] - mr);
              l += fi * ls[i];
              o += fi * os[i];
            }
          M = mr;
        }
        a.o[(size_t)b * H + hh * DX_D + lane] = valid ? (f16)(o / l) : (f16)__builtin_nanf("");
      }
    }
    {
      // o_proj's fragments on wavefronts 0-2; wavefront 3 copies the gate/up weights into
      // LDS and does no loads or stores of its own until the gate/up phase uses them
      DxRows ro{Ly.wo, nullptr, nullptr, 1, H, nq, nkv, nwx, m};
      DxRows rg{Ly.wg, Ly.wu, nullptr, 2, H, nq, nkv, nwx, m};
      dx_arrive(sy);
      dx_prefetch<UR, IM_H3, 1, NFR, 3>(fr, ro, nu_h, KS_H);
      if (w == 3) dx_weights_to_lds<2>(rg, nu_i, KS_H, lds_addr(GW));
      if (!dx_wait(sy, &bad)) goto aborted;
    }

    // ---- o_proj + residual
    dx_stage_rows<DX_KPAD_H, 192, DX_HMAX>(Ah, Al, orr, H, H, g, R);
    dx_mma<UR, IM_H3, 1, NFR, 3, DX_KPAD_H, false>(fr, nullptr, nu_h, KS_H, Ah, Al, red, res);
    if (w < nu_h) {
      const int col = (m + w * nwx) * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 4 * (lane >> 4) + i;
        if (j < R) {
          const size_t idx = (size_t)(g + 8 * j) * H + col;
          const float old = ld_sc1_f(xr, (uint32_t)(idx * 4));
          a.x[idx] = old + res[0][i];
        }
      }
    }
    dx_arrive(sy, w != 3);  // wavefront 3 stored nothing and has its copies in flight
    if (!dx_wait(sy, &bad)) goto aborted;

    // ---- gate/up + SwiGLU
    wait_vmcnt<0>();  // the weight copies have landed (the barrier in the staging publishes them)
    dx_norm_prefetch(nw, Ly.mn, H, R);
    dx_stage_norm<DX_KPAD_H>(Ah, Al, xr, nw, H, a.eps, g, R);
    dx_mma<2 * DX_UMAX, IM_H, 2, NFR, DX_WAVES, DX_KPAD_H, true>(fr, GW, nu_i, KS_H, Ah, Al, red, res);
    if (w < nu_i) {
      const int col = (m + w * nwx) * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 4 * (lane >> 4) + i;
        if (j < R) {
          const float z = res[0][i];
          a.y[(size_t)(g + 8 * j) * I + col] = (f16)(z / (1.0f + __expf(-z)) * res[1][i]);
        }
      }
    }
    {
      DxRows rd{Ly.wd, nullptr, nullptr, 1, I, nq, nkv, nwx, m};
      dx_arrive(sy);
      dx_prefetch<UR, IM_I, 1, NFR>(fr, rd, nu_h, KS_I);
      if (!dx_wait(sy, &bad)) goto aborted;
    }

    // ---- down + residual
    dx_stage_rows<DX_KPAD, DX_THREADS, DX_KMAX>(Adh, Adl, yr, I, I, g, R);
    dx_mma<UR, IM_I, 1, NFR, DX_WAVES, DX_KPAD, false>(fr, nullptr, nu_h, KS_I, Adh, Adl, red, res);
    if (w < nu_h) {
      const int col = (m + w * nwx) * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 4 * (lane >> 4) + i;
        if (j < R) {
          const size_t idx = (size_t)(g + 8 * j) * H + col;
          const float old = ld_sc1_f(xr, (uint32_t)(idx * 4));
          a.x[idx] = old + res[0][i];
        }
      }
    }
    {
      dx_arrive(sy);
      const DxLayer &Ln = a.layer[l + 1 < a.L ? l + 1 : l];  // the last layer re-reads its own
      DxRows rq{Ln.wq, Ln.wk, Ln.wv, 0, H, nq, nkv, nwx, m};
      dx_prefetch<UR, IM_H, 1, NFR>(fr, rq, nu_qkv, KS_H);
      if (!dx_wait(sy, &bad)) goto aborted;
    }
  }

  // ---- final RMSNorm: the head's operand xs = final_norm * x * r * 2^-8 and the row
  // sums of squares per 64 columns (both buffers the head reads), workgroup m < R
  if (m < R) {
    __shared__ float part_ss[DX_THREADS / 16];
    const int b = g + 8 * m;
    const int c = tid * 4;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    float q = 0.f;
    if (c < H) {
      const Chunk16 ch = ld_sc1(xr, (uint32_t)(((size_t)b * H + c) * 4));
      v = (f32x4){__uint_as_float(ch[0]), __uint_as_float(ch[1]), __uint_as_float(ch[2]), __uint_as_float(ch[3])};
      q = v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) q += __shfl_xor(q, o, 64);  // 16 lanes = 64 columns
    if ((tid & 15) == 0) {
      part_ss[tid >> 4] = q;
      if (c < H) {
        a.ss_p[(size_t)(c >> 6) * B + b] = q;
        a.ss_q[(size_t)(c >> 6) * B + b] = q;
      }
    }
    __syncthreads();
    float tot = 0.f;
    for (int i = 0; i < H / 64; ++i) tot += part_ss[i];
    const float r = 1.0f / sqrtf(tot / (float)H + a.eps);
    if (c < H) {
      const uint2 wb = *reinterpret_cast<const uint2 *>(a.final_norm + c);
      const float w0 = __uint_as_float(wb.x << 16), w1 = __uint_as_float(wb.x & 0xffff0000u);
      const float w2 = __uint_as_float(wb.y << 16), w3 = __uint_as_float(wb.y & 0xffff0000u);
      const f16x4 h = {(f16)(v[0] * r * w0 * SMOL_XS_SCALE), (f16)(v[1] * r * w1 * SMOL_XS_SCALE),
                       (f16)(v[2] * r * w2 * SMOL_XS_SCALE), (f16)(v[3] * r * w3 * SMOL_XS_SCALE)};
      *reinterpret_cast<f16x4 *>(a.xs + (size_t)b * H + c) = h;
    }
  }
  return;

aborted:
  // the step did not complete: the group's head rows become NaN
  if (m < R) {
    const int b = g + 8 * m;
    for (int c = tid; c < H; c += DX_THREADS) a.xs[(size_t)b * H + c] = (f16)__builtin_nanf("");
    for (int c = tid; c < H / 64; c += DX_THREADS) {
      a.ss_p[(size_t)c * B + b] = 1.f;
      a.ss_q[(size_t)c * B + b] = 1.f;
    }
  }
}

__global__ void dx_clear_kernel(uint32_t *ctrl, int words) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < words; i += gridDim.x * blockDim.x) ctrl[i] = 0u;
}

// Barrier deadline in ticks of the 100 MHz shader clock: 1 s, or SMOL_DECODE_DEADLINE_TICKS
// (read at every call: a test sets a tiny value to drive the abort path).
unsigned long long decode_xcd_deadline_ticks() {
  const char *e = getenv("SMOL_DECODE_DEADLINE_TICKS");
  if (e && *e) {
    const unsigned long long v = strtoull(e, nullptr, 10);
    if (v > 0) return v;
  }
  return 100000000ull;
}

int decode_xcd_groups_per_xcd() {
  static int nwx = -1;
  if (nwx < 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 0;
    nwx = (cus % SMOL_XCDS == 0) ? cus / SMOL_XCDS : 0;
  }
  return nwx;
}

bool decode_xcd_fits(int B, int H, int nq, int nkv, int d, int I, int L, int cap, int nwx) {
  if (d != DX_D || nwx < 8 || nwx > 64 || B < 1 || B > 8 * DX_ROWS || L < 1 || L > DX_LMAX) return false;
  if (nq % nkv != 0 || nq / nkv < 1 || nq / nkv > 4) return false;
  if (H % 64 != 0 || H > DX_HMAX || I % 32 != 0 || I > DX_KMAX) return false;
  if ((nq + 2 * nkv) * 4 > DX_UREG * nwx || H / 16 > DX_UREG * nwx || I / 16 > DX_UMAX * nwx) return false;
  if ((size_t)cap * DX_D * 2 >= (1ull << 31) || (size_t)B * nq * 32 * (DX_D + 2) * 4 >= (1ull << 31)) return false;
  const int npair = (B + 7) / 8 * nkv;
  if (npair > nwx * DX_WAVES || (B + 7) / 8 * nq > nwx * DX_WAVES) return false;
  return true;
}

int decode_xcd_splits(int B, int nkv, int nwx) {
  const int npair = (B + 7) / 8 * nkv;
  return std::max(1, std::min(DX_SPMAX, nwx * DX_WAVES / npair));
}

// Sized for the largest group count decode_xcd_fits admits (64 workgroups per XCD),
// so that the host can size the workspace without asking the device.
size_t decode_xcd_part_floats(int B, int nq, int nkv) {
  return (size_t)B * nq * decode_xcd_splits(B, nkv, 64) * (DX_D + 2);
}

size_t decode_xcd_ctrl_words(int nwx) { return (size_t)SMOL_XCDS * nwx * 16 + DX_CTRL_WORDS; }

hipError_t decode_xcd(const DecodeXcdArgs &a, hipStream_t s) {
  const int words = (int)decode_xcd_ctrl_words(a.nwx);
  hipLaunchKernelGGL(dx_clear_kernel, dim3(16), dim3(256), 0, s, a.ctrl, words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(SMOL_XCDS * a.nwx), block(DX_THREADS);
  const bool masked = a.key_mask != nullptr;
  switch (a.nq / a.nkv) {
    case 1: return masked ? launch(decode_xcd_kernel<1, true>, grid, block, s, a) : launch(decode_xcd_kernel<1, false>, grid, block, s, a);
    case 2: return masked ? launch(decode_xcd_kernel<2, true>, grid, block, s, a) : launch(decode_xcd_kernel<2, false>, grid, block, s, a);
    case 3: return masked ? launch(decode_xcd_kernel<3, true>, grid, block, s, a) : launch(decode_xcd_kernel<3, false>, grid, block, s, a);
    case 4: return masked ? launch(decode_xcd_kernel<4, true>, grid, block, s, a) : launch(decode_xcd_kernel<4, false>, grid, block, s, a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace smol
