// Shared device helpers for the gfx950 kernels: element types, MFMA wrappers,
// wavefront reductions. Wave size is 64 on CDNA4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define SMOL_WAVE 64

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(f16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE
template <> __device__ __forceinline__ f16 from_f32<f16>(float x) { return (f16)x; }     // RNE

// ---------------------------------------------------------------- element types
// W: how weights, the embedding, the KV cache and the logits are stored (the
// model's dtype). Act<W>: the MFMA operand type of the activations. For bfloat16
// models the activations are float16: every bfloat16 value whose magnitude lies in
// float16's normal range converts to float16 exactly (8 significant bits fit in
// 11), and float16 keeps 3 more bits of each activation at the same MFMA rate.
template <typename W> struct OperandOf { using type = W; };
template <> struct OperandOf<bf16> { using type = f16; };
template <typename W> using Act = typename OperandOf<W>::type;

// ---------------------------------------------------------------- deferred-norm operand scale
// The deferred RMSNorm operand xs (kernels.h, NormIn / NormOut) is stored times
// SMOL_XS_SCALE = 2^-8, and the GEMM that reads it multiplies its output rows by
// 2^8 (exact power-of-two scalings). A normalised row has |value| <= sqrt(H) * max|w|
// (<= 45 |w| at H = 2048); a residual epilogue stores w * x_new * r_old, which grows
// with the row's rms growth g over one update, so an unscaled float16 xs overflows
// (65504) once g passes about 1500 / max|w|. At 2^-8 the limit is 256 times higher
// (g up to ~4e5 / max|w| at H = 2048), while typical values (~2^-8) stay normal in
// float16 (down to 2^-14) and the elements that become subnormal keep the absolute
// spacing (2^-24) of the bottom of the normal range, far below the rounding error of
// the row's typical elements: the products do not lose accuracy. A row whose rms
// shrinks by more than ~2^-6 in one update starts to lose float16 precision
// gradually (no overflow, no NaN).
constexpr float SMOL_XS_SCALE = 0.00390625f;  // 2^-8
constexpr float SMOL_XS_UNSCALE = 256.0f;     // 2^8

// ---------------------------------------------------------------- fragments
// A 32x32x16 MFMA step takes, per lane, 8 consecutive K values of one row of A
// (row = lane % 32, K chunk = lane / 32) and likewise of one column of B. Frag<T>
// holds those 8 values. The same register layout feeds both element types: for
// float the step is issued as eight 32x32x2 MFMAs, instruction j taking element j
// of every lane. A and B are always loaded the same way, so the order in which K
// is summed inside a step does not change the contraction.

template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<f16> { f16x8 v; };
template <> struct Frag<float> { f32x8 v; };

__device__ __forceinline__ void mma_32x32x16(f32x16 &acc, const Frag<bf16> &a, const Frag<bf16> &b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_32x32x16(f32x16 &acc, const Frag<f16> &a, const Frag<f16> &b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a.v, b.v, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma_32x32x16(f32x16 &acc, const Frag<float> &a, const Frag<float> &b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[j], b.v[j], acc, 0, 0, 0);
}

// Load 8 consecutive elements (16 B for bf16, 32 B for float).
__device__ __forceinline__ void load_frag(Frag<bf16> &f, const bf16 *p) {
  f.v = *reinterpret_cast<const bf16x8 *>(p);
}
__device__ __forceinline__ void load_frag(Frag<f16> &f, const f16 *p) {
  f.v = *reinterpret_cast<const f16x8 *>(p);
}
__device__ __forceinline__ void load_frag(Frag<float> &f, const float *p) {
  const f32x4 lo = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 hi = *reinterpret_cast<const f32x4 *>(p + 4);
  f.v = (f32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Row of the 32x32 accumulator held in register r of a lane (column = lane % 32).
__device__ __forceinline__ int acc_row(int r, int lane) { return ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3); }

// ---------------------------------------------------------------- XCD row ownership
// Workgroup i of a launch runs on XCD i % 8, and each XCD has its own L2. The
// prefill's GEMMs give XCD x the row range [x * rows_per_xcd, (x + 1) * rows_per_xcd)
// of the activations, so each row of A is fetched into one L2 only and shared there
// by the workgroups of that row (the weights are read once per XCD). Keeping the
// same ranges from one kernel to the next was measured to buy nothing more: across
// a kernel boundary the rows come back from MALL either way. Only for M >= 1024:
// below that, every XCD must get work.
constexpr int SMOL_XCDS = 8;
__host__ __device__ inline bool xcd_rows(int M) { return M >= 1024; }
// An eighth of M rounded up to whole tiles of max(128, BM) rows, so that every XCD's
// range is made of whole BM-row tiles.
__host__ __device__ inline int rows_per_xcd(int M, int BM) {
  const int g = BM > 128 ? BM : 128;
  return ((M + SMOL_XCDS - 1) / SMOL_XCDS + g - 1) / g * g;
}

// ---------------------------------------------------------------- RoPE angles
// (cos, sin) of p * omega, accurate at any position up to float rounding of the
// result: the angle is formed and reduced modulo 2 pi in double (Cody-Waite, with
// 2 pi split into the double nearest to it plus the remainder), and only the reduced
// angle, |r| <= pi, goes to float sincosf. A float product p * omega alone is off by
// up to 1.4e-4 rad at p = 8191; this is within ~2e-7 everywhere (and much cheaper
// than a double sincos).
__device__ __forceinline__ float2 rope_cos_sin(int pos, double omega) {
  const double x = (double)pos * omega;
  const double k = rint(x * 0.15915494309189535);  // round(x / (2 pi))
  const double r = fma(-k, 6.283185307179586, x) - k * 2.4492935982947064e-16;
  float s, c;
  sincosf((float)r, &s, &c);
  return make_float2(c, s);
}

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, SMOL_WAVE);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, SMOL_WAVE));
  return v;
}

// 16-byte vector (8 two-byte or 4 four-byte elements) for global <-> LDS staging.
// A native vector type, so that arrays of chunks stay in registers.
typedef uint32_t Chunk16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ Chunk16 ld16(const void *p) { return *reinterpret_cast<const Chunk16 *>(p); }
__device__ __forceinline__ void st16(void *p, Chunk16 v) { *reinterpret_cast<Chunk16 *>(p) = v; }

// Element e of a chunk viewed as T.
template <typename T> __device__ __forceinline__ T chunk_elem(const Chunk16 &c, int e);
template <> __device__ __forceinline__ float chunk_elem<float>(const Chunk16 &c, int e) { return __uint_as_float(c[e]); }
template <> __device__ __forceinline__ bf16 chunk_elem<bf16>(const Chunk16 &c, int e) {
  return __builtin_bit_cast(bf16, (uint16_t)(c[e >> 1] >> ((e & 1) * 16)));
}
template <> __device__ __forceinline__ f16 chunk_elem<f16>(const Chunk16 &c, int e) {
  return __builtin_bit_cast(f16, (uint16_t)(c[e >> 1] >> ((e & 1) * 16)));
}

// Direct global -> LDS copy of 16 bytes per lane (gfx950 global_load_lds_dwordx4):
// lane l's 16 bytes land at LDS byte address lds_base + 16 * l, lds_base wave-uniform.
// Issued through inline asm so the compiler adds no waits of its own: the caller
// waits with wait_vmcnt<N>() and a barrier before anyone reads the data.
__device__ __forceinline__ void lds_dma16(const void *g, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds_base) : "memory");
}
template <int N> __device__ __forceinline__ void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)p; }

// Convert a staged chunk from storage type W to operand type Act<W> (same size).
template <typename W> __device__ __forceinline__ Chunk16 to_operand(const Chunk16 &c) { return c; }
// Two bfloat16 in one dword -> two float16 (exact in float16's normal range; one
// v_cvt_pk_f16_f32, round to nearest even, per pair).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t x) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f32x2 f = {__uint_as_float(x << 16), __uint_as_float(x & 0xffff0000u)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}
template <> __device__ __forceinline__ Chunk16 to_operand<bf16>(const Chunk16 &c) {
  Chunk16 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = bf16x2_to_f16x2(c[i]);
  return r;
}
