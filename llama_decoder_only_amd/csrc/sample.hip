// Next-token choice from one row of logits per sequence: greedy, or temperature /
// top-k / top-p filtered sampling with a uniform number supplied by the caller.
//
// What is computed (Sualeh77 model.py, "7. Top-level SmolLM2-135M Model
// Architecture", generate; abi96062 model.py, SmolLM2Model.generate):
//   temperature == 0: the index of the largest logit (the lowest such index on ties);
//   otherwise, with z = logit / temperature:
//     top-k (0 < k < V): drop every token whose logit is below the k-th largest
//       logit (tokens equal to it stay);
//     top-p (p < 1): order the remaining tokens by logit, descending (equal logits by
//       ascending index), take their softmax probabilities and drop each token after
//       the first whose preceding tokens already hold more than p of the mass;
//     sample from the softmax of the kept z: the first index j, in vocabulary order,
//       whose cumulative probability exceeds u (inverse CDF with the caller's u).
// A row holding a NaN gives -1; so does a sampled row whose largest logit is not
// finite (its softmax is undefined).
//
// One workgroup of 1024 threads per row; the row is copied to LDS when it fits (else
// read again in every pass) and values compare as order-preserving 32-bit keys.
// Pass 1 finds the maximum (and ends greedy choice). Sampling then bins the tokens by
// their distance below the maximum and accumulates, per bin, the count and the mass
// as integers (each weight in units of 2^-40, so the sums do not depend on the
// order of accumulation). The bins holding the top-k and top-p cuts are sorted
// exactly (bitonic, by key then index) to place each cut on its token; per-step
// masses of the kept tokens then locate the draw in vocabulary order. A cut bin with
// more than LIST_MAX tokens falls back to radix selects (8-bit digits by count for
// top-k, 4-bit digits by float mass for top-p, sums in a fixed order) and a wave-
// ordered scan for the draw.
#include "common.h"
#include "kernels.h"

namespace smol {

namespace {

constexpr int NT = 1024, NWV = NT / 64;
constexpr int NBIN = 2048;        // value bins below the maximum logit, BIN_SCALE per logit unit
constexpr float BIN_SCALE = 16.f;
constexpr int LIST_MAX = 2048;    // tokens of one bin sorted exactly
constexpr float FIX = 1099511627776.0f;  // fixed-point scale of token weights: 2^40
typedef unsigned long long u64;

// Order-preserving key: a > b (as floats, -0 == +0) <=> key(a) > key(b).
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(__fadd_rn(f, 0.0f));  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <typename T>
__device__ __forceinline__ float ld(const T *row, int i) {
  return to_f32(row[i]);
}

// Sum over the block, taken in a fixed order (a shuffle tree per wave, then the wave
// sums in wave order); every thread gets the same value.
__device__ float block_sum(float v, float *red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_down(v, o, 64);
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NWV; ++i) s += red[i];
  __syncthreads();
  return s;
}

__device__ int block_sum_int(int v, int *red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_down(v, o, 64);
  if (lane == 0) red[w] = v;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int i = 0; i < NWV; ++i) s += red[i];
  __syncthreads();
  return s;
}

// Inclusive scan over the 64 lanes of a wave (fixed order).
template <typename V>
__device__ __forceinline__ V wave_incl_scan(V v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const V t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Shared memory of the binned path: counts and fixed-point masses per bin (later the
// per-thread masses of the row), and one bin's tokens as sortable (key, ~index) pairs.
struct BinShared {
  uint32_t cnt[NBIN];
  union {
    u64 mass[NBIN];
    u64 steps[NT];
  } a;
  u64 list[LIST_MAX];
  u64 red[NWV];
  int list_n;
};

// A weight in [0, 1] as an integer number of 2^-40 units (exact sums in any order).
__device__ __forceinline__ u64 fixw(float w) { return (u64)(w * FIX); }

// Inclusive scan of one u64 per thread over the block, in thread order (exact).
__device__ u64 block_incl_scan_u64(u64 v, u64 *red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_incl_scan<u64>(v);
  if (lane == 63) red[w] = v;
  __syncthreads();
  u64 before = 0;
  for (int i = 0; i < w; ++i) before += red[i];
  __syncthreads();
  return before + v;
}

// Wave 0: the first index b < nb whose running sum of arr (in index order) exceeds
// thr, and the sum before it; -1 when the whole sum stays <= thr. Exact (integers).
template <typename V>
__device__ void first_crossing(const V *arr, int nb, V thr, int *bin, V *before) {
  const int lane = threadIdx.x & 63;
  const int per = (nb + 63) / 64, lo = min(nb, lane * per), hi = min(nb, lo + per);
  V sum = 0;
  for (int j = lo; j < hi; ++j) sum += arr[j];
  const V incl = wave_incl_scan<V>(sum);
  const V excl = incl - sum;
  const bool mine = excl <= thr && incl > thr;
  const unsigned long long m = __ballot(mine);
  if (m == 0) {
    *bin = -1;
    *before = incl;  // lane-independent only in lane 63; callers use bin < 0 alone
    return;
  }
  const int owner = __ffsll((long long)m) - 1;
  int b = -1;
  V c = excl;
  if (lane == owner) {
    for (int j = lo; j < hi; ++j) {
      if (c + arr[j] > thr) {
        b = j;
        break;
      }
      c += arr[j];
    }
  }
  *bin = __shfl(b, owner, 64);
  *before = __shfl(c, owner, 64);
}

struct SampleShared {
  uint32_t hist[256];
  float fbin[NWV][16];
  float fred[NWV];
  int ired[NWV];
  uint32_t kred[NWV];
  int xred[NWV];
  float wave_total[NWV];
  int wave_ties[NWV];
  uint32_t sel_key;
  int sel_want;
  int answer;
};

}  // namespace

// The value whose key is k (the inverse of fkey; -0 comes back as +0).
__device__ __forceinline__ float kval(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// The row as seen by one lane. Lane `lane` of wave w holds the elements
// i = w * 64 * n + k * 64 + lane, k < n: each wave owns a contiguous range of the
// vocabulary, walked in 64-element steps. CACHE: the row is copied to LDS once and
// every pass reads it there; otherwise every pass reads it from memory (any V).
template <typename T, bool CACHE>
struct Row {
  const T *row;
  const T *lds;
  int V, n, base;
  __device__ __forceinline__ int idx(int k) const { return base + k * 64; }
  __device__ __forceinline__ bool valid(int k) const { return idx(k) < V; }
  __device__ __forceinline__ float val(int i) const { return CACHE ? to_f32(lds[i]) : ld(row, i); }
  __device__ __forceinline__ uint32_t key(int k) const {  // 0 for positions past the row
    if (!valid(k)) return 0u;
    return fkey(val(idx(k)));
  }
};

constexpr int CACHE_BYTES = 112 * 1024;

template <typename T, bool CACHE>
__global__ void __launch_bounds__(NT) sample_kernel(const T *logits, long row_stride, int V, float temperature,
                                                    int top_k, float top_p, const float *uniforms, int32_t *next_ids) {
  __shared__ SampleShared sh;
  __shared__ BinShared bs;
  __shared__ __attribute__((aligned(16))) char cache[CACHE ? CACHE_BYTES : 16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  Row<T, CACHE> rk;
  rk.row = logits + (size_t)blockIdx.x * row_stride;
  rk.lds = reinterpret_cast<const T *>(cache);
  rk.V = V;
  rk.n = (V + NT - 1) / NT;
  rk.base = w * 64 * rk.n + lane;
  const int n = rk.n;

  // ---- pass 1: (the copy to LDS,) maximum (lowest index on ties), NaN check
  int nan = 0;
  uint32_t kmax = 0;
  int imax = 0x7fffffff;
  {
    // 16-byte loads, 8 in flight per thread (element order per thread ascends, so a
    // strict > keeps the lowest index); a row that is not 16-byte aligned, and the
    // tail past the last whole chunk, go element by element.
    constexpr int EPV = 16 / (int)sizeof(T);
    T *c = reinterpret_cast<T *>(cache);
    auto take = [&](int i, T x) {
      if constexpr (CACHE) c[i] = x;
      const float f = to_f32(x);
      nan |= f != f;
      const uint32_t key = fkey(f);
      if (key > kmax) kmax = key, imax = i;
    };
    const bool vec = (reinterpret_cast<uintptr_t>(rk.row) & 15) == 0;
    const int nch = vec ? V / EPV : 0;
    for (int c0 = tid; c0 < nch; c0 += 8 * NT) {
      Chunk16 ch[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (c0 + j * NT < nch) ch[j] = ld16(rk.row + (size_t)(c0 + j * NT) * EPV);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (c0 + j * NT < nch) {
          const int i0 = (c0 + j * NT) * EPV;
          if constexpr (CACHE) st16(c + i0, ch[j]);
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            const T x = chunk_elem<T>(ch[j], e);
            const float f = to_f32(x);
            nan |= f != f;
            const uint32_t key = fkey(f);
            if (key > kmax) kmax = key, imax = i0 + e;
          }
        }
    }
    for (int i = nch * EPV + tid; i < V; i += NT) take(i, rk.row[i]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t k2 = __shfl_xor(kmax, o, 64);
    const int i2 = __shfl_xor(imax, o, 64);
    if (k2 > kmax || (k2 == kmax && i2 < imax)) kmax = k2, imax = i2;
  }
  if (lane == 0) sh.kred[w] = kmax, sh.xred[w] = imax;
  nan = block_sum_int(nan, sh.ired);  // also orders the writes above (and the LDS copy)
  kmax = sh.kred[0];
  imax = sh.xred[0];
  for (int i = 1; i < NWV; ++i)
    if (sh.kred[i] > kmax || (sh.kred[i] == kmax && sh.xred[i] < imax)) kmax = sh.kred[i], imax = sh.xred[i];
  const float lmax = kval(kmax);
  if (nan || (temperature > 0.f && !isfinite(lmax))) {
    if (tid == 0) next_ids[blockIdx.x] = -1;
    return;
  }
  if (!(temperature > 0.f)) {
    if (tid == 0) next_ids[blockIdx.x] = imax;
    return;
  }
  const float inv_t = 1.0f / temperature;
  // exp2-based hardware exp (relative error a few 1e-6, far below the rounding margins
  // the draw and the cuts are decided with)
  auto weight = [&](uint32_t key) { return __expf((kval(key) - lmax) * inv_t); };

  // ---- binned path. Tokens fall into bins by (lmax - logit) * BIN_SCALE, so a bin
  // holds a contiguous range of the descending order. Counts and fixed-point masses
  // per bin locate the bins that hold the top-k and top-p cuts; those bins' tokens
  // are sorted exactly ((key, index) pairs) to place each cut on its token. Every sum
  // is an integer, so the order of accumulation does not matter. A cut bin with more
  // than LIST_MAX tokens takes the radix path below instead.
  {
    auto bin_of = [&](float f) {
      const float d = (lmax - f) * BIN_SCALE;
      return d < (float)(NBIN - 1) ? (int)d : NBIN - 1;
    };
    const bool use_k = top_k > 0 && top_k < V, use_p = top_p < 1.0f;
    if (use_k || use_p) {  // counts (every cut sorts its bin), masses for top-p
      for (int i = tid; i < NBIN; i += NT) bs.cnt[i] = 0, bs.a.mass[i] = 0;
      __syncthreads();
      for (int k = 0; k < n; ++k) {
        if (!rk.valid(k)) continue;
        const float f = rk.val(rk.idx(k));
        const int b = bin_of(f);
        atomicAdd(&bs.cnt[b], 1u);
        if (use_p) {
          const u64 q = fixw(weight(fkey(f)));
          if (q) __hip_atomic_fetch_add(&bs.a.mass[b], q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
      __syncthreads();
    }
    // Gather and sort (descending (key, -index)) the tokens of bin b; false when they
    // do not fit the list.
    auto sort_bin = [&](int b) -> int {
      const int c = (int)bs.cnt[b];
      if (c > LIST_MAX) return -1;
      if (tid == 0) bs.list_n = 0;
      __syncthreads();
      for (int k = 0; k < n; ++k) {
        if (!rk.valid(k)) continue;
        const int i = rk.idx(k);
        const float f = rk.val(i);
        if (bin_of(f) == b) {
          const int pos = atomicAdd(&bs.list_n, 1);
          bs.list[pos] = ((u64)fkey(f) << 32) | (u64)(0xffffffffu - (uint32_t)i);
        }
      }
      int np = 1;
      while (np < c) np <<= 1;
      __syncthreads();
      for (int i = c + tid; i < np; i += NT) bs.list[i] = 0;  // padding sorts last
      __syncthreads();
      for (int size = 2; size <= np; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
          for (int t = tid; t < np / 2; t += NT) {
            const int lo = 2 * stride * (t / stride) + (t % stride), hi = lo + stride;
            const bool desc = (lo & size) == 0;
            const u64 x = bs.list[lo], y = bs.list[hi];
            if ((x < y) == desc) bs.list[lo] = y, bs.list[hi] = x;
          }
          __syncthreads();
        }
      return c;
    };
    // The first list position (of c) at which base + the running mass of the entries
    // exceeds thr, and the mass through it; -1 if none. Entries with keys below kmin
    // count 0.
    auto list_crossing = [&](int c, u64 base, u64 thr, uint32_t kmin, u64 *through) -> int {
      u64 v0 = 0, v1 = 0;
      const int e0 = 2 * tid, e1 = 2 * tid + 1;
      if (e0 < c && (uint32_t)(bs.list[e0] >> 32) >= kmin) v0 = fixw(weight((uint32_t)(bs.list[e0] >> 32)));
      if (e1 < c && (uint32_t)(bs.list[e1] >> 32) >= kmin) v1 = fixw(weight((uint32_t)(bs.list[e1] >> 32)));
      const u64 incl = block_incl_scan_u64(v0 + v1, bs.red);
      const u64 c0 = base + incl - v1, c1 = base + incl;
      int pos = 0x7fffffff;
      if (v0 && c0 > thr) pos = e0;
      else if (v1 && c1 > thr) pos = e1;
      if (tid == 0) bs.list_n = 0x7fffffff;
      __syncthreads();
      if (pos != 0x7fffffff) atomicMin(&bs.list_n, pos);
      __syncthreads();
      const int p = bs.list_n == 0x7fffffff ? -1 : bs.list_n;
      if (p >= 0 && (p == e0 || p == e1)) bs.red[0] = p == e0 ? c0 : c1;
      __syncthreads();
      *through = p >= 0 ? bs.red[0] : 0;
      __syncthreads();
      return p;
    };

    bool ok = true;
    uint32_t kcut = 0;     // kept: key > kcut, or key == kcut with index <= ilim
    int ilim = 0x7fffffff;
    u64 total = 0;         // top-k kept mass (for the top-p threshold)
    int kbin = NBIN;       // bins before kbin hold only tokens above the top-k cut
    u64 mass_k = 0;        // mass of those bins
    uint32_t kth = 0;
    int kc = 0;            // tokens of bin kbin (sorted in the list)
    // top-k
    if (use_k) {
      int b;
      uint32_t before;
      if (w == 0) first_crossing<uint32_t>(bs.cnt, NBIN, (uint32_t)(top_k - 1), &b, &before);
      if (tid == 0) bs.red[0] = (u64)b, bs.red[1] = before;
      __syncthreads();
      kbin = (int)(long long)bs.red[0];
      const uint32_t cnt_before = (uint32_t)bs.red[1];
      __syncthreads();
      kc = sort_bin(kbin);
      if (kc < 0) {
        ok = false;
      } else {
        kth = (uint32_t)(bs.list[top_k - 1 - cnt_before] >> 32);
        kcut = kth;
      }
      if (ok && use_p) {  // the mass of the tokens top-k keeps
        u64 m = 0;
        for (int j = tid; j < NBIN && j < kbin; j += NT) m += bs.a.mass[j];
        m = block_incl_scan_u64(m, bs.red);  // thread NT-1 holds the total
        if (tid == NT - 1) bs.red[2] = m;
        __syncthreads();
        mass_k = bs.red[2];
        __syncthreads();
        u64 part = 0;  // the mass of the kept part of bin kbin
        for (int e = tid; e < kc; e += NT) {
          const uint32_t key = (uint32_t)(bs.list[e] >> 32);
          if (key >= kth) part += fixw(weight(key));
        }
        part = block_incl_scan_u64(part, bs.red);
        if (tid == NT - 1) bs.red[3] = part;
        __syncthreads();
        total = mass_k + bs.red[3];
        __syncthreads();
      }
    } else if (use_p) {
      u64 m = 0;
      for (int j = tid; j < NBIN; j += NT) m += bs.a.mass[j];
      m = block_incl_scan_u64(m, bs.red);
      if (tid == NT - 1) bs.red[2] = m;
      __syncthreads();
      total = bs.red[2];
      __syncthreads();
    }
    // top-p: the token at which the descending running mass first exceeds top_p * total
    if (ok && use_p) {
      const u64 P = (u64)((double)top_p * (double)total);
      int b;
      u64 before;
      if (w == 0) first_crossing<u64>(bs.a.mass, kbin < NBIN ? kbin : NBIN, P, &b, &before);
      if (tid == 0) bs.red[0] = (u64)(long long)b, bs.red[1] = before;
      __syncthreads();
      const int pb = (int)(long long)bs.red[0];
      u64 base = bs.red[1];
      __syncthreads();
      int c = kc;
      uint32_t kmin = kth;
      if (pb >= 0) {          // the cut lies in bin pb, above the top-k bin
        c = sort_bin(pb);
        kmin = 0;
      } else {                // the cut lies in the top-k bin (whose list is sorted)
        base = mass_k;
      }
      if (c < 0) {
        ok = false;
      } else {
        u64 through;
        const int pos = list_crossing(c, base, P, kmin, &through);
        if (pos < 0) {
          ok = false;  // cannot happen with exact sums; leave it to the radix path
        } else {
          const u64 e = bs.list[pos];
          kcut = (uint32_t)(e >> 32);
          ilim = (int)(0xffffffffu - (uint32_t)e);
          (void)through;
        }
      }
    }
    if (ok) {
      auto kept_w = [&](int i) -> u64 {
        const float f = rk.val(i);
        const uint32_t key = fkey(f);
        const bool keep = key > kcut || (key == kcut && i <= ilim);
        return keep ? fixw(weight(key)) : 0;
      };
      // thread t sums the kept mass of tokens [t C, t C + C) in index order (C a
      // multiple of 8: a cached bfloat16 row is read 16 bytes at a time)
      const int C = ((V + NT - 1) / NT + 7) / 8 * 8, lo = min(V, tid * C), hi = min(V, lo + C);
      auto chunk_mass = [&](int a, int b, int stop_at, u64 base, u64 thr, int *hit) -> u64 {
        u64 acc = base;
        if constexpr (CACHE && sizeof(T) == 2) {
          for (int i0 = a; i0 < b; i0 += 8) {
            const Chunk16 ch = ld16(rk.lds + i0);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int i = i0 + e;
              if (i >= b) break;
              const float f = to_f32(chunk_elem<T>(ch, e));
              const uint32_t key = fkey(f);
              const u64 v = (key > kcut || (key == kcut && i <= ilim)) ? fixw(weight(key)) : 0;
              if (stop_at && v && acc + v > thr) {
                *hit = i;
                return acc;
              }
              acc += v;
            }
          }
        } else {
          for (int i = a; i < b; ++i) {
            const u64 v = kept_w(i);
            if (stop_at && v && acc + v > thr) {
              *hit = i;
              return acc;
            }
            acc += v;
          }
        }
        return acc;
      };
      int unused = -1;
      const u64 cs = chunk_mass(lo, hi, 0, 0, 0, &unused);
      __syncthreads();
      bs.a.steps[tid] = cs;
      const u64 incl = block_incl_scan_u64(cs, bs.red);
      if (tid == NT - 1) bs.red[0] = incl;
      __syncthreads();
      const u64 target = (u64)((double)uniforms[blockIdx.x] * (double)bs.red[0]);
      if (w == 0) {
        int t;
        u64 before;
        first_crossing<u64>(bs.a.steps, NT, target, &t, &before);
        if (lane == 0) {
          int ans = -1;
          if (t >= 0) {
            const int tl = min(V, t * C), th = min(V, tl + C);
            chunk_mass(tl, th, 1, before, target, &ans);
          }
          next_ids[blockIdx.x] = ans;
        }
      }
      return;
    }
    __syncthreads();
  }

  // ---- top-k: key of the k-th largest logit (radix select, 8-bit digits, MSB first)
  uint32_t kth = 0;  // keep keys >= kth
  if (top_k > 0 && top_k < V) {
    uint32_t prefix = 0, mask = 0;
    int want = top_k;  // rank still wanted within the current prefix
    for (int d = 24; d >= 0; d -= 8) {
      for (int i = tid; i < 256; i += NT) sh.hist[i] = 0;
      __syncthreads();
#pragma unroll 4
      for (int k = 0; k < n; ++k) {
        const uint32_t key = rk.key(k);
        if (rk.valid(k) && (key & mask) == prefix) atomicAdd(&sh.hist[(key >> d) & 255], 1u);
      }
      __syncthreads();
      if (w == 0) {  // lane j owns bins 4j .. 4j+3; find the bin holding rank `want`, from the top
        uint32_t c[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) c[e] = sh.hist[4 * lane + e];
        const uint32_t s = c[0] + c[1] + c[2] + c[3];
        // incl: count in this lane's bins and every higher lane's (a suffix scan)
        uint32_t incl = s;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t t = __shfl_down(incl, o, 64);
          if (lane + o < 64) incl += t;
        }
        uint32_t above = incl - s;
        if (above < (uint32_t)want && (uint32_t)want <= incl) {
          for (int e = 3; e >= 0; --e) {
            if ((uint32_t)want <= above + c[e]) {
              sh.sel_key = (uint32_t)(4 * lane + e);
              sh.sel_want = want - (int)above;
              break;
            }
            above += c[e];
          }
        }
      }
      __syncthreads();
      prefix |= sh.sel_key << d;
      mask |= 255u << d;
      want = sh.sel_want;
      __syncthreads();
    }
    kth = prefix;
  }

  // ---- top-p: the token at which the descending cumulative mass first exceeds p
  // (radix select by mass, 4-bit digits). Tokens above key kp stay, and the first
  // n_tie tokens (by index) whose key equals kp.
  uint32_t kp = 0;
  int n_tie = 0x7fffffff;
  if (top_p < 1.0f) {
    float z = 0.f;
#pragma unroll 4
    for (int k = 0; k < n; ++k) {
      const uint32_t key = rk.key(k);
      if (rk.valid(k) && key >= kth) z += weight(key);
    }
    const float P = top_p * block_sum(z, sh.fred);
    uint32_t prefix = 0, mask = 0;
    float above = 0.f;  // mass of the kept tokens with keys above the current range
    bool crossed = true;
    for (int d = 28; d >= 0; d -= 4) {
      float bin[16];
#pragma unroll
      for (int b = 0; b < 16; ++b) bin[b] = 0.f;
      for (int k = 0; k < n; ++k) {
        const uint32_t key = rk.key(k);
        if (rk.valid(k) && key >= kth && (key & mask) == prefix) {
          const uint32_t dg = (key >> d) & 15;
          const float e = weight(key);
#pragma unroll
          for (int b = 0; b < 16; ++b) bin[b] += dg == (uint32_t)b ? e : 0.f;
        }
      }
#pragma unroll
      for (int b = 0; b < 16; ++b) {
        float v = bin[b];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_down(v, o, 64);
        if (lane == 0) sh.fbin[w][b] = v;
      }
      __syncthreads();
      if (tid == 0) {
        float tot[16];
        for (int b = 0; b < 16; ++b) {
          tot[b] = 0.f;
          for (int i = 0; i < NWV; ++i) tot[b] += sh.fbin[i][b];
        }
        int sel = -1;
        for (int b = 15; b >= 0; --b) {
          if (tot[b] > 0.f && above + tot[b] > P) {
            sel = b;
            break;
          }
          above += tot[b];
        }
        if (sel < 0) {  // the mass never exceeds P (rounding): keep everything
          sh.sel_want = -1;
        } else {
          sh.sel_key = (uint32_t)sel;
          sh.sel_want = 0;
          sh.fred[0] = above;
        }
      }
      __syncthreads();
      if (sh.sel_want < 0) {
        crossed = false;
        __syncthreads();
        break;
      }
      prefix |= sh.sel_key << d;
      mask |= 15u << d;
      above = sh.fred[0];
      __syncthreads();
    }
    if (crossed) {
      kp = prefix;
      // every token with key kp has the same weight q: keep the first c of them,
      // c the smallest count with above + c * q > P
      const float q = weight(kp);
      const float c = floorf((P - above) / q) + 1.f;
      n_tie = c < 1.f ? 1 : (c > 2.0e9f ? 0x7fffffff : (int)c);
    } else {
      kp = kth;
    }
  }
  const uint32_t klo = top_p < 1.0f ? kp : kth;  // keys > klo stay; keys == klo: the first n_tie
                                                  // (kp >= kth, so top-k holds for them too)

  // ---- inverse CDF in vocabulary order. Every wave sums the kept mass of its range
  // (lane by lane, then a shuffle tree); the wave whose range holds the target walks
  // it again in index order (64-element steps, a lane scan each).
  int nt = 0;
  float wsum = 0.f;
  {
    // ties of key klo in this lane's elements, then per wave; a tie's rank is its
    // order by index, known only after the wave counts are in
    for (int k = 0; k < n; ++k) nt += (rk.valid(k) && rk.key(k) == klo) ? 1 : 0;
  }
  int wt = nt;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) wt += __shfl_down(wt, o, 64);
  if (lane == 0) sh.wave_ties[w] = wt;
  __syncthreads();
  int tie0 = 0, all_ties = 0;
  for (int i = 0; i < NWV; ++i) {
    if (i < w) tie0 += sh.wave_ties[i];
    all_ties += sh.wave_ties[i];
  }
  if (all_ties <= n_tie) n_tie = 0x7fffffff;  // every tie stays (the usual case: one token)
  // the kept weight of element k, given the ties before it in index order (the wave
  // steps are in index order; within a step, the lanes below)
  auto kept_weight = [&](int k, int ties_before, bool &is_tie, int &ti) {
    const uint32_t key = rk.key(k);
    is_tie = rk.valid(k) && key == klo;
    ti = wave_incl_scan<int>(is_tie ? 1 : 0);
    const bool keep = rk.valid(k) && (key > klo || (is_tie && ties_before + ti - 1 < n_tie));
    return keep ? weight(key) : 0.f;
  };
  if (n_tie == 0x7fffffff) {  // every tie stays: no ranks needed
    for (int k = 0; k < n; ++k) {
      const uint32_t key = rk.key(k);
      if (rk.valid(k) && key >= klo) wsum += weight(key);
    }
  } else {
    int ties = tie0;
    for (int k = 0; k < n; ++k) {
      bool is_tie;
      int ti;
      wsum += kept_weight(k, ties, is_tie, ti);
      ties += __shfl(ti, 63, 64);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) wsum += __shfl_down(wsum, o, 64);
  if (lane == 0) sh.wave_total[w] = wsum;
  if (tid == 0) sh.answer = -1;
  __syncthreads();
  float total = 0.f;
  for (int i = 0; i < NWV; ++i) total += sh.wave_total[i];
  const float target = uniforms[blockIdx.x] * total;
  // owner: the first wave whose range ends above the target; else the last with mass
  int owner = -1;
  float pre = 0.f, owner_pre = 0.f;
  for (int i = 0; i < NWV; ++i) {
    if (sh.wave_total[i] > 0.f) {
      if (pre + sh.wave_total[i] > target) {
        owner = i;
        owner_pre = pre;
        break;
      }
      owner = i;
      owner_pre = pre;
    }
    pre += sh.wave_total[i];
  }
  if (w == owner) {  // the first crossing in index order wins; else the last kept token
    float r = owner_pre;
    int t = tie0;
    int found = -1, last = -1;
    for (int k = 0; k < n && found < 0; ++k) {
      bool is_tie;
      int ti;
      const float e = kept_weight(k, t, is_tie, ti);
      const float incl = wave_incl_scan<float>(e);
      const unsigned long long hit = __ballot(e > 0.f && r + incl > target);
      const unsigned long long any = __ballot(e > 0.f);
      if (hit) found = rk.idx(k) - lane + __ffsll((long long)hit) - 1;
      if (any) last = rk.idx(k) - lane + 63 - __clzll((long long)any);
      r += __shfl(incl, 63, 64);
      t += __shfl(ti, 63, 64);
    }
    if (lane == 0) sh.answer = found >= 0 ? found : last;
  }
  __syncthreads();
  if (tid == 0) next_ids[blockIdx.x] = sh.answer;
}

// Rows that fit 128 KB of LDS (64 K bfloat16 or 32 K float elements) are copied there
// once; longer rows are read again in every pass.
template <typename T>
hipError_t sample_next(const T *logits, long row_stride, int B, int V, float temperature, int top_k, float top_p,
                       const float *uniforms, int32_t *next_ids, hipStream_t s) {
  const dim3 g(B), b(NT);
  if ((long)V * (long)sizeof(T) <= CACHE_BYTES)
    return launch(sample_kernel<T, true>, g, b, s, logits, row_stride, V, temperature, top_k, top_p, uniforms,
                  next_ids);
  return launch(sample_kernel<T, false>, g, b, s, logits, row_stride, V, temperature, top_k, top_p, uniforms,
                next_ids);
}

template hipError_t sample_next<float>(const float *, long, int, int, float, int, float, const float *, int32_t *,
                                       hipStream_t);
template hipError_t sample_next<bf16>(const bf16 *, long, int, int, float, int, float, const float *, int32_t *,
                                      hipStream_t);

}  // namespace smol
