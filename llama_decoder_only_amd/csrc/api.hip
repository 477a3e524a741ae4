// The C ABI (include/smol.h): host-side argument checks, workspace layout and
// the sequence of kernel launches for a block, a prefill and a decode step.
//
// Order of one block (nnterp "SmolLM3", "The block, in order"; tohio block.py):
//   u = RMSNorm(x; attn_norm); q, k, v = u W^T     gemm_qkv_rope: RoPE on q, k; k, v
//                                                  land in the cache
//   o = causal GQA attention                       attention_prefill / attention_decode
//   x += o W_o^T                                   gemm_residual
//   u = RMSNorm(x; mlp_norm); y = silu(u W_g^T) * (u W_u^T)        gemm_swiglu
//   x += y W_d^T                                   gemm_residual
// The model gathers the embedding before the blocks and applies the final RMSNorm
// and the tied head after them (abi96062 model.py, SmolLM2Model.forward). Every
// RMSNorm is deferred (kernels.h, NormIn / NormOut): the kernel that last wrote x
// leaves xs = w * x * r_old * 2^-8 and the new row sums of squares, and the GEMM that reads
// xs rescales its output rows. Five launches per block, no separate norm kernels.
#include <algorithm>
#include <cmath>
#include <map>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "common.h"
#include "kernels.h"
#include "decode_xcd.h"
#include "smol.h"

namespace {

thread_local std::string g_err;

smol_status fail(smol_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

struct Dims {
  int H, nq, nkv, d, I, L, V, max_pos, G;
  int nope_every, window;  // SmolLM3 variants (smol_config)
  float eps, theta;
  bool bf16;
  size_t esz;
};

smol_status check_config(const smol_config *c, Dims *o) {
  if (!c) return fail(SMOL_ERR_INVALID_ARG, "cfg is NULL");
  if (c->dtype != SMOL_F32 && c->dtype != SMOL_BF16) return fail(SMOL_ERR_INVALID_ARG, "dtype %d unknown", c->dtype);
  if (c->hidden < 1 || c->n_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 1 || c->intermediate < 1 ||
      c->n_layers < 1 || c->vocab < 1 || c->max_pos < 1)
    return fail(SMOL_ERR_INVALID_ARG, "config sizes must be >= 1");
  if (c->hidden != c->n_heads * c->head_dim)
    return fail(SMOL_ERR_INVALID_ARG, "hidden %d != n_heads %d * head_dim %d", c->hidden, c->n_heads, c->head_dim);
  if (c->n_heads % c->n_kv_heads != 0)
    return fail(SMOL_ERR_INVALID_ARG, "n_heads %d not divisible by n_kv_heads %d", c->n_heads, c->n_kv_heads);
  if (!(std::isfinite(c->rms_eps) && c->rms_eps >= 0.f)) return fail(SMOL_ERR_INVALID_ARG, "rms_eps must be finite, >= 0");
  if (!(std::isfinite(c->rope_theta) && c->rope_theta > 0.f)) return fail(SMOL_ERR_INVALID_ARG, "rope_theta must be > 0");
  const int G = c->n_heads / c->n_kv_heads;
  if (G > 4) return fail(SMOL_ERR_UNSUPPORTED, "%d query heads per kv head (supported: 1..4)", G);
  if (c->head_dim != 64 && c->head_dim != 128) return fail(SMOL_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", c->head_dim);
  if (c->hidden % 64 || c->intermediate % 64 || c->vocab % 64)
    return fail(SMOL_ERR_UNSUPPORTED, "hidden, intermediate and vocab must be multiples of 64");
  if (c->hidden > 4096) return fail(SMOL_ERR_UNSUPPORTED, "hidden %d (supported: up to 4096)", c->hidden);
  if (c->no_rope_interval < 0 || c->sliding_window < 0)
    return fail(SMOL_ERR_INVALID_ARG, "no_rope_interval and sliding_window must be >= 0");
  o->nope_every = c->no_rope_interval;
  o->window = c->sliding_window;
  o->H = c->hidden;
  o->nq = c->n_heads;
  o->nkv = c->n_kv_heads;
  o->d = c->head_dim;
  o->I = c->intermediate;
  o->L = c->n_layers;
  o->V = c->vocab;
  o->max_pos = c->max_pos;
  o->G = G;
  o->eps = c->rms_eps;
  o->theta = c->rope_theta;
  o->bf16 = c->dtype == SMOL_BF16;
  o->esz = o->bf16 ? 2 : 4;
  return SMOL_OK;
}

// The kernels move rows in 16-byte vectors and 16-byte copies into LDS, so every
// buffer of rows (weights, embedding, hidden states, caches, logits) starts on a
// 16-byte boundary; a null pointer passes here (the callers check those).
struct Named {
  const void *p;
  const char *name;
};
smol_status check_aligned(std::initializer_list<Named> bufs) {
  for (const Named &b : bufs)
    if ((uintptr_t)b.p % 16) return fail(SMOL_ERR_INVALID_ARG, "%s must be 16-byte aligned", b.name);
  return SMOL_OK;
}

smol_status check_layer(const smol_layer_weights *w, int idx) {
  if (!w) return fail(SMOL_ERR_INVALID_ARG, "layer weights %d: NULL", idx);
  const void *p[9] = {w->attn_norm, w->wq, w->wk, w->wv, w->wo, w->mlp_norm, w->w_gate, w->w_up, w->w_down};
  static const char *names[9] = {"attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"};
  for (int i = 0; i < 9; ++i) {
    if (!p[i]) return fail(SMOL_ERR_INVALID_ARG, "layer %d: %s is NULL", idx, names[i]);
    if ((uintptr_t)p[i] % 16) return fail(SMOL_ERR_INVALID_ARG, "layer %d: %s must be 16-byte aligned", idx, names[i]);
  }
  return SMOL_OK;
}

constexpr size_t ALIGN = 256;
size_t up(size_t n) { return (n + ALIGN - 1) / ALIGN * ALIGN; }

// Workspace carve-up. Offsets in bytes from ws.
struct Ws {
  size_t x, xs, q, k, v, o, y, ss_p, ss_q, rope, part, gpart, dxpart, dxctrl, total;
};

Ws layout(const Dims &D, int op, int B, int T) {
  Ws w{};
  const size_t M = (op == SMOL_OP_DECODE) ? (size_t)B : (size_t)B * T;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += up(bytes); return at; };
  w.x = take(M * D.H * 4);
  w.xs = take(M * D.H * D.esz);
  w.q = take(M * D.nq * D.d * D.esz);
  w.o = take(M * D.nq * D.d * D.esz);
  w.y = take(M * D.I * D.esz);
  w.ss_p = take((size_t)(D.H / 64) * M * 4);  // row sums of squares of x per 64 columns,
  w.ss_q = take((size_t)(D.H / 64) * M * 4);  // two buffers: new and old alternate
  w.rope = take(M * (D.d / 2) * 8);             // (cos, sin) of each row's RoPE angles
  {  // K-split partial sums of the GEMMs that split (few tiles: small M), shared in turn
    const int m = (int)M, e = (int)D.esz;
    const size_t f = std::max({smol::gemm_part_floats(m, D.nq * D.d + 2 * D.nkv * D.d, D.H, e),
                               smol::gemm_part_floats(m, D.H, D.nq * D.d, e), smol::gemm_part_floats(m, 2 * D.I, D.H, e),
                               smol::gemm_part_floats(m, D.H, D.I, e), smol::gemm_part_floats(m, D.V, D.H, e)});
    w.gpart = take(f * 4);
  }
  if (op == SMOL_OP_DECODE) {
    int chunk;
    const int cap = std::min(T, D.max_pos);
    const int splits = smol::decode_splits(cap, D.d, D.esz, &chunk);
    w.part = take((size_t)B * D.nq * splits * (D.d + 2) * 4);
    // the one-launch step (decode_xcd): its attention partials and barrier flags
    w.dxpart = take(smol::decode_xcd_part_floats(B, D.nq, D.nkv) * 4);
    w.dxctrl = take(smol::decode_xcd_ctrl_words(64) * 4);
  } else {
    w.k = take((size_t)B * D.nkv * T * D.d * D.esz);
    w.v = take((size_t)B * D.nkv * T * D.d * D.esz);
  }
  w.total = off;
  return w;
}

// ------------------------------------------------------------------ timing

struct Timing {
  std::mutex mu;
  int kernel = -1, max = 0, count = 0;
  bool armed = false, used = false;  // a pair is offered to / taken by the next launch
  std::vector<hipEvent_t> ev;        // start/stop pairs
} g_timing;

}  // namespace

namespace smol {

void timing_before(int kernel, hipStream_t) {
  g_timing.armed = g_timing.kernel == kernel && g_timing.count < g_timing.max;
  g_timing.used = false;
}

bool timing_take(hipEvent_t *start, hipEvent_t *stop) {
  if (!g_timing.armed) return false;
  g_timing.armed = false;
  g_timing.used = true;
  *start = g_timing.ev[2 * g_timing.count];
  *stop = g_timing.ev[2 * g_timing.count + 1];
  return true;
}

void timing_after(int, hipStream_t) {
  if (g_timing.used) ++g_timing.count;
  g_timing.armed = g_timing.used = false;
}

}  // namespace smol

namespace {

#define SMOL_LAUNCH(kind, call)                                                                        \
  do {                                                                                                 \
    smol::timing_before(kind, s);                                                                      \
    hipError_t e_ = (call);                                                                            \
    smol::timing_after(kind, s);                                                                       \
    if (e_ != hipSuccess) return fail(SMOL_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_));         \
  } while (0)

struct LayerCtx {
  const Dims *D;
  char *ws;
  Ws lay;
  int B, T, pos0;
  void *kc, *vc;
  int cap, kv_off, q_key_off;
  int layer;             // block index: decides the rotary and the window
  const int *cache_len;  // decode only
  const uint8_t *key_mask;  // [B, mask_ld] over key indices, or nullptr
  int mask_ld;
  double inv_freq[64];
  hipStream_t s;
};

// One block. On entry xs = attn_norm * x * r_old, ss_p holds the row sums of squares
// of x and ss_q those r_old came from. On exit the same holds for next_norm (the
// next block's attn_norm or the final norm; nullptr: nothing is left for a norm).
template <typename T>
smol_status run_layer(const LayerCtx &c, const smol_layer_weights *w, float *x, const void *next_norm) {
  const Dims &D = *c.D;
  const hipStream_t s = c.s;
  const bool decode = c.cache_len != nullptr;
  const int M = decode ? c.B : c.B * c.T;
  using A = Act<T>;  // activations: MFMA operand type
  A *xs = (A *)(c.ws + c.lay.xs);
  A *q = (A *)(c.ws + c.lay.q);
  A *o = (A *)(c.ws + c.lay.o);
  A *y = (A *)(c.ws + c.lay.y);
  float *ss_p = (float *)(c.ws + c.lay.ss_p), *ss_q = (float *)(c.ws + c.lay.ss_q);
  float *gpart = (float *)(c.ws + c.lay.gpart);

  // SmolLM3 variants: no rotary on every nope_every-th block, the window on those
  const bool rope_on = !(D.nope_every > 0 && (c.layer + 1) % D.nope_every == 0);
  const int window = (!rope_on && D.window > 0) ? D.window : 0;
  smol::QkvOut qo{M, D.H, D.nq * D.d, D.nkv * D.d, D.d, q, c.kc, c.vc,
                  decode ? 1 : c.T, c.cap, D.nkv, c.pos0, c.kv_off, D.max_pos, c.cache_len,
                  (const float2 *)(c.ws + c.lay.rope), rope_on ? 1 : 0};
  SMOL_LAUNCH(SMOL_K_QKV_ROPE, smol::gemm_qkv_rope<T>(xs, smol::NormIn{ss_p, ss_q, D.eps}, (const T *)w->wq,
                                                      (const T *)w->wk, (const T *)w->wv, qo, gpart, s));
  if (decode) {
    int chunk;
    const int splits = smol::decode_splits(std::min(c.cap, D.max_pos), D.d, D.esz, &chunk);
    smol::DecodeAttnArgs da{q, c.kc, c.vc, o, c.cache_len, c.B, D.nq, D.nkv, D.d, c.cap, D.max_pos, splits, chunk,
                            (float *)(c.ws + c.lay.part), c.key_mask, c.mask_ld, window};
    hipError_t e = smol::attention_decode<T>(da, s);
    if (e != hipSuccess) return fail(SMOL_ERR_HIP, "attention_decode: %s", hipGetErrorString(e));
  } else {
    smol::AttnArgs aa{q, c.kc, c.vc, o, c.B, c.T, D.nq, D.nkv, D.d, c.cap, c.q_key_off, c.key_mask, c.mask_ld,
                      window};
    SMOL_LAUNCH(SMOL_K_ATTENTION, smol::attention_prefill<T>(aa, s));
  }
  // x += o W_o^T; leaves xs for mlp_norm, the new sums in ss_q (ss_p: the old ones)
  SMOL_LAUNCH(SMOL_K_O_PROJ, smol::gemm_residual<T>(o, (const T *)w->wo, M, D.H, D.nq * D.d, x,
                                                    smol::NormOut{ss_p, ss_q, w->mlp_norm, xs, D.eps}, gpart, s));
  SMOL_LAUNCH(SMOL_K_GATE_UP, smol::gemm_swiglu<T>(xs, smol::NormIn{ss_q, ss_p, D.eps}, (const T *)w->w_gate,
                                                   (const T *)w->w_up, M, D.I, D.H, y, gpart, s));
  // x += y W_d^T; leaves xs for next_norm, the new sums in ss_p (ss_q: the old ones)
  const smol::NormOut nxt{ss_q, next_norm ? ss_p : nullptr, next_norm, next_norm ? (void *)xs : nullptr, D.eps};
  SMOL_LAUNCH(SMOL_K_DOWN, smol::gemm_residual<T>(y, (const T *)w->w_down, M, D.H, D.I, x, nxt, gpart, s));
  return SMOL_OK;
}

void fill_inv_freq(const Dims &D, double *f) {
  // omega_i = theta^(-2i/d) (abi96062 components.py, RotaryEmbedding), in double
  for (int i = 0; i < D.d / 2; ++i) f[i] = std::pow((double)D.theta, -2.0 * i / D.d);
}

smol_status check_ws(const Dims &D, int op, int B, int T, void *ws, size_t ws_bytes, Ws *lay) {
  *lay = layout(D, op, B, T);
  if (!ws) return fail(SMOL_ERR_INVALID_ARG, "ws is NULL");
  if (ws_bytes < lay->total)
    return fail(SMOL_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, lay->total);
  if ((uintptr_t)ws % ALIGN) return fail(SMOL_ERR_INVALID_ARG, "ws must be 256-byte aligned");
  return SMOL_OK;
}

// The tied head on the final RMSNorm: logits = u E^T, from the xs the last block left.
template <typename T>
smol_status head(const Dims &D, const smol_model_weights *w, int M, void *logits, char *ws, const Ws &lay,
                 hipStream_t s) {
  const smol::NormIn fin{(const float *)(ws + lay.ss_p), (const float *)(ws + lay.ss_q), D.eps};
  SMOL_LAUNCH(SMOL_K_LM_HEAD, smol::gemm_store<T>((const Act<T> *)(ws + lay.xs), fin, (const T *)w->embed, M, D.V, D.H,
                                                  logits, 0, (float *)(ws + lay.gpart), s));
  return SMOL_OK;
}

// x = E[ids] or x = src, with what the first block's deferred RMSNorm reads and the
// RoPE table of the call's rows (positions as LayerCtx c defines them).
template <typename T>
smol_status prologue(const LayerCtx &c, const int32_t *ids, const T *E, const float *src, float *x,
                     const T *attn_norm, int M) {
  const Dims &D = *c.D;
  const hipStream_t s = c.s;
  smol::RopeIn rope{(float2 *)(c.ws + c.lay.rope), D.d / 2, c.pos0, c.T, c.cache_len, {}};
  for (int i = 0; i < D.d / 2; ++i) rope.inv_freq[i] = c.inv_freq[i];
  SMOL_LAUNCH(SMOL_K_EMBED, smol::rows_ss<T>(ids, E, src, x, (float *)(c.ws + c.lay.ss_p),
                                             (float *)(c.ws + c.lay.ss_q), attn_norm, (Act<T> *)(c.ws + c.lay.xs),
                                             D.eps, M, D.H, D.V, rope, s));
  return SMOL_OK;
}

template <typename T>
smol_status block_impl(const Dims &D, const smol_layer_weights *w, const float *x_in, float *x_out, int B, int T_,
                       int pos0, void *kc, void *vc, int cap, char *ws, const Ws &lay, hipStream_t s) {
  LayerCtx c{};
  c.D = &D;
  c.ws = ws;
  c.lay = lay;
  c.B = B;
  c.T = T_;
  c.pos0 = pos0;
  c.s = s;
  if (kc) {
    c.kc = kc; c.vc = vc; c.cap = cap; c.kv_off = 0; c.q_key_off = pos0;
  } else {
    c.kc = ws + lay.k; c.vc = ws + lay.v; c.cap = T_; c.kv_off = pos0; c.q_key_off = 0;
  }
  fill_inv_freq(D, c.inv_freq);
  smol_status st = prologue<T>(c, nullptr, nullptr, x_in, x_out, (const T *)w->attn_norm, B * T_);
  if (st != SMOL_OK) return st;
  return run_layer<T>(c, w, x_out, nullptr);
}

// Tokens at positions pos0 .. pos0 + T_ - 1 (pos0 > 0 needs the caches, which then
// hold positions 0 .. pos0 - 1 already: a chunk of a longer prefill).
template <typename T>
smol_status prefill_impl(const Dims &D, const smol_model_weights *w, const int32_t *ids, int B, int T_, void *logits,
                         void *kc, void *vc, int cap, char *ws, const Ws &lay, hipStream_t s, int pos0 = 0,
                         const uint8_t *key_mask = nullptr) {
  float *x = (float *)(ws + lay.x);
  const int M = B * T_;
  LayerCtx c{};
  c.D = &D;
  c.ws = ws;
  c.lay = lay;
  c.B = B;
  c.T = T_;
  c.pos0 = pos0;
  c.key_mask = key_mask;
  c.mask_ld = kc ? cap : T_;
  c.s = s;
  fill_inv_freq(D, c.inv_freq);
  smol_status st0 = prologue<T>(c, ids, (const T *)w->embed, x, x, (const T *)w->layers[0].attn_norm, M);
  if (st0 != SMOL_OK) return st0;
  const size_t layer_elems = (size_t)B * D.nkv * cap * D.d;
  for (int l = 0; l < D.L; ++l) {
    if (kc) {
      c.kc = (char *)kc + l * layer_elems * D.esz;
      c.vc = (char *)vc + l * layer_elems * D.esz;
      c.cap = cap; c.kv_off = 0; c.q_key_off = pos0;
    } else {
      c.kc = ws + lay.k; c.vc = ws + lay.v; c.cap = T_; c.kv_off = 0; c.q_key_off = 0;
    }
    const void *next = l + 1 < D.L ? w->layers[l + 1].attn_norm : w->final_norm;
    c.layer = l;
    smol_status st = run_layer<T>(c, &w->layers[l], x, next);
    if (st != SMOL_OK) return st;
  }
  if (!logits) return SMOL_OK;  // generation: the head runs on the last positions only
  return head<T>(D, w, M, logits, ws, lay, s);
}

template <typename T>
smol_status decode_impl(const Dims &D, const smol_model_weights *w, const int32_t *ids, const int32_t *cache_len,
                        int B, void *kc, void *vc, int cap, void *logits, char *ws, const Ws &lay, hipStream_t s,
                        const uint8_t *key_mask = nullptr) {
  float *x = (float *)(ws + lay.x);
  if constexpr (std::is_same<T, bf16>::value) {
    // the whole step but the head in one persistent launch, where the shape fits it
    const int nwx = smol::decode_xcd_groups_per_xcd();
    if (smol::decode_xcd_fits(B, D.H, D.nq, D.nkv, D.d, D.I, D.L, cap, nwx)) {
      smol::DecodeXcdArgs a{};
      a.B = B; a.H = D.H; a.nq = D.nq; a.nkv = D.nkv; a.I = D.I; a.L = D.L; a.V = D.V;
      a.cap = cap; a.max_pos = D.max_pos; a.nope_every = D.nope_every; a.window = D.window;
      a.nwx = nwx; a.sp = smol::decode_xcd_splits(B, D.nkv, nwx); a.mask_ld = cap; a.eps = D.eps;
      a.ids = ids; a.cache_len = cache_len; a.key_mask = key_mask;
      a.embed = (const bf16 *)w->embed; a.final_norm = (const bf16 *)w->final_norm;
      a.kc = (bf16 *)kc; a.vc = (bf16 *)vc;
      a.x = x; a.q = (f16 *)(ws + lay.q); a.o = (f16 *)(ws + lay.o); a.y = (f16 *)(ws + lay.y);
      a.part = (float *)(ws + lay.dxpart); a.xs = (f16 *)(ws + lay.xs);
      a.ss_p = (float *)(ws + lay.ss_p); a.ss_q = (float *)(ws + lay.ss_q);
      a.ctrl = (uint32_t *)(ws + lay.dxctrl);
      a.deadline = smol::decode_xcd_deadline_ticks();
      double f[64];
      fill_inv_freq(D, f);
      for (int i = 0; i < D.d / 2; ++i) a.inv_freq[i] = f[i];
      for (int l = 0; l < D.L; ++l) {
        const smol_layer_weights &Lw = w->layers[l];
        a.layer[l] = smol::DxLayer{(const bf16 *)Lw.wq, (const bf16 *)Lw.wk, (const bf16 *)Lw.wv,
                                   (const bf16 *)Lw.wo, (const bf16 *)Lw.w_gate, (const bf16 *)Lw.w_up,
                                   (const bf16 *)Lw.w_down, (const bf16 *)Lw.attn_norm, (const bf16 *)Lw.mlp_norm};
      }
      SMOL_LAUNCH(SMOL_K_DECODE_STEP, smol::decode_xcd(a, s));
      return head<T>(D, w, B, logits, ws, lay, s);
    }
  }
  LayerCtx c{};
  c.D = &D;
  c.ws = ws;
  c.lay = lay;
  c.B = B;
  c.T = 1;
  c.cap = cap;
  c.cache_len = cache_len;
  c.key_mask = key_mask;
  c.mask_ld = cap;
  c.s = s;
  fill_inv_freq(D, c.inv_freq);
  smol_status st0 = prologue<T>(c, ids, (const T *)w->embed, x, x, (const T *)w->layers[0].attn_norm, B);
  if (st0 != SMOL_OK) return st0;
  const size_t layer_elems = (size_t)B * D.nkv * cap * D.d;
  for (int l = 0; l < D.L; ++l) {
    c.kc = (char *)kc + l * layer_elems * D.esz;
    c.vc = (char *)vc + l * layer_elems * D.esz;
    const void *next = l + 1 < D.L ? w->layers[l + 1].attn_norm : w->final_norm;
    c.layer = l;
    smol_status st = run_layer<T>(c, &w->layers[l], x, next);
    if (st != SMOL_OK) return st;
  }
  return head<T>(D, w, B, logits, ws, lay, s);
}

// Generation workspace: one region that the prefill and then the decode steps use in
// turn (same stream, never at once), then the last-position state, the logits of one
// step and the per-step positions.
struct GenWs {
  Ws pre, dec;
  size_t xs_last, ssp_last, ssq_last, logits, pos, total;
};

GenWs gen_layout(const Dims &D, int B, int T, int max_new, int cap) {
  GenWs g{};
  g.pre = layout(D, SMOL_OP_PREFILL, B, T);
  g.dec = layout(D, SMOL_OP_DECODE, B, cap);
  size_t off = std::max(g.pre.total, g.dec.total);
  auto take = [&](size_t bytes) { size_t at = off; off += up(bytes); return at; };
  g.xs_last = take((size_t)B * D.H * D.esz);
  g.ssp_last = take((size_t)(D.H / 64) * B * 4);
  g.ssq_last = take((size_t)(D.H / 64) * B * 4);
  g.logits = take((size_t)B * D.V * D.esz);
  g.pos = take((size_t)std::max(1, max_new - 1) * B * 4);
  g.total = off;
  return g;
}

template <typename T>
smol_status generate_impl(const Dims &D, const smol_model_weights *w, const int32_t *prompt, const int32_t *lens,
                          int B, int T_, int max_new, float temperature, int top_k, float top_p,
                          const float *uniforms, int32_t *out_ids, void *kc, void *vc, int cap, char *ws,
                          const GenWs &g, hipStream_t s) {
  smol_status st = prefill_impl<T>(D, w, prompt, B, T_, nullptr, kc, vc, cap, ws, g.pre, s);
  if (st != SMOL_OK) return st;
  using A = Act<T>;
  A *xs_last = (A *)(ws + g.xs_last);
  float *ssp = (float *)(ws + g.ssp_last), *ssq = (float *)(ws + g.ssq_last);
  T *logits = (T *)(ws + g.logits);
  int32_t *pos = (int32_t *)(ws + g.pos);
  hipError_t e = smol::gather_last<T>((const A *)(ws + g.pre.xs), (const float *)(ws + g.pre.ss_p),
                                      (const float *)(ws + g.pre.ss_q), B, T_, D.H, lens, xs_last, ssp, ssq, s);
  if (e != hipSuccess) return fail(SMOL_ERR_HIP, "gather_last: %s", hipGetErrorString(e));
  SMOL_LAUNCH(SMOL_K_LM_HEAD, smol::gemm_store<T>(xs_last, smol::NormIn{ssp, ssq, D.eps}, (const T *)w->embed, B, D.V,
                                                  D.H, logits, 0, nullptr, s));
  auto sample = [&](int step) -> smol_status {
    SMOL_LAUNCH(SMOL_K_SAMPLE, smol::sample_next<T>(logits, D.V, B, D.V, temperature, top_k, top_p,
                                                    uniforms ? uniforms + (size_t)step * B : nullptr,
                                                    out_ids + (size_t)step * B, s));
    return SMOL_OK;
  };
  if ((st = sample(0)) != SMOL_OK) return st;
  if (max_new > 1) {
    e = smol::fill_positions(pos, B, max_new - 1, T_, lens, s);
    if (e != hipSuccess) return fail(SMOL_ERR_HIP, "fill_positions: %s", hipGetErrorString(e));
  }
  for (int step = 1; step < max_new; ++step) {
    st = decode_impl<T>(D, w, out_ids + (size_t)(step - 1) * B, pos + (size_t)(step - 1) * B, B, kc, vc, cap, logits,
                        ws, g.dec, s);
    if (st != SMOL_OK) return st;
    if ((st = sample(step)) != SMOL_OK) return st;
  }
  return SMOL_OK;
}

smol_status check_model(const Dims &D, const smol_model_weights *w) {
  if (!w) return fail(SMOL_ERR_INVALID_ARG, "model weights NULL");
  if (!w->embed) return fail(SMOL_ERR_INVALID_ARG, "embed is NULL");
  if (!w->final_norm) return fail(SMOL_ERR_INVALID_ARG, "final_norm is NULL");
  if (!w->layers) return fail(SMOL_ERR_INVALID_ARG, "layers is NULL");
  if (smol_status st = check_aligned({{w->embed, "embed"}, {w->final_norm, "final_norm"}}); st != SMOL_OK) return st;
  for (int l = 0; l < D.L; ++l) {
    smol_status st = check_layer(&w->layers[l], l);
    if (st != SMOL_OK) return st;
  }
  return SMOL_OK;
}


// ------------------------------------------------------------------ backward
// smol_block_backward: the forward recomputed with its activations kept, then the
// chain rule in reverse (backward.hip). M = B*T rows; C3 = (nq + 2 nkv) d.
struct BwWs {
  size_t u, r1, qkv, o, lse, h, wn, r2, gu, dgu, y, dwn, dh, dO, dsum, dqkv, part, du, npart, gpart, rope;
  size_t wf32[9];  // a bf16 model's weights widened to float32 (unused for float32 models)
  size_t total;
};

// The GEMMs of one block backward: (M, N, K, epilogue) of each launch, in order.
struct BwShape {
  int M, N, K, epi;
};
std::vector<BwShape> bw_shapes(const Dims &D, int M) {
  const int H = D.H, I = D.I, QD = D.nq * D.d, C3 = QD + 2 * D.nkv * D.d;
  using namespace smol;
  return {{M, C3, H, BW_STORE},  {M, H, QD, BW_RESID},  {M, 2 * I, H, BW_STORE}, {M, I, H, BW_SWIGLU},
          {H, I, M, BW_ACCUM},   {M, H, 2 * I, BW_STORE}, {2 * I, H, M, BW_ACCUM}, {H, QD, M, BW_ACCUM},
          {M, QD, H, BW_STORE},  {C3, H, M, BW_ACCUM},  {M, H, C3, BW_STORE}};
}

BwWs bw_layout(const Dims &D, int B, int T) {
  BwWs w{};
  const size_t M = (size_t)B * T, H = D.H, C3 = (size_t)(D.nq + 2 * D.nkv) * D.d, QD = (size_t)D.nq * D.d;
  size_t off = 0;
  auto take = [&](size_t floats) { size_t at = off; off += up(floats * 4); return at; };
  w.u = take(M * H);
  w.r1 = take(M);
  w.qkv = take(M * C3);
  w.o = take(M * QD);
  w.lse = take((size_t)B * D.nq * T);
  w.h = take(M * H);
  w.wn = take(M * H);
  w.r2 = take(M);
  w.gu = take(M * 2 * D.I);
  w.dgu = take(M * 2 * D.I);
  w.y = take(M * D.I);
  w.dwn = take(M * H);
  w.dh = take(M * H);
  w.dO = take(M * QD);
  w.dsum = take((size_t)B * D.nq * T);
  w.dqkv = take(M * C3);
  w.part = take(2 * (size_t)D.nq * M * D.d);
  w.du = take(M * H);
  w.npart = take((size_t)smol::bw_rms_part_rows((int)M) * H);
  size_t gp = 0;
  for (const BwShape &g : bw_shapes(D, (int)M)) gp = std::max(gp, smol::bw_gemm_part_floats(g.M, g.N, g.K, g.epi));
  w.gpart = take(std::max<size_t>(gp, 1));
  w.rope = take(M * (D.d / 2) * 2);  // (cos, sin) per row and frequency
  const size_t KD = (size_t)D.nkv * D.d;
  const size_t wsz[9] = {H, QD * H, KD * H, KD * H, H * QD, H, (size_t)D.I * H, (size_t)D.I * H, H * D.I};
  for (int i = 0; i < 9; ++i) w.wf32[i] = D.bf16 ? take(wsz[i]) : 0;
  w.total = off;
  return w;
}

smol::BwOperand operand(const float *p0, int ld, const float *p1 = nullptr, int seg0 = 1 << 30,
                        const float *p2 = nullptr, int seg1 = 1 << 30) {
  return smol::BwOperand{p0, p1, p2, seg0, seg1, ld};
}

smol::BwGemm gemm_args(const smol::BwOperand &a, const smol::BwOperand &b, int M, int N, int K, float *C, int ldc) {
  smol::BwGemm g{};
  g.a = a;
  g.b = b;
  g.M = M;
  g.N = N;
  g.K = K;
  g.C = C;
  g.cseg0 = g.cseg1 = 1 << 30;
  g.ldc = ldc;
  g.ksplit = 1;
  return g;
}

// Output rows split over up to three matrices (fused weight gradients).
smol::BwGemm with_c_segments(smol::BwGemm g, float *C1, int cseg0, float *C2 = nullptr, int cseg1 = 1 << 30) {
  g.C1 = C1;
  g.cseg0 = cseg0;
  g.C2 = C2;
  g.cseg1 = cseg1;
  return g;
}

smol_status backward_impl(const Dims &D, const smol_layer_weights *w, int layer, const float *x, const float *dy,
                          int B, int T, int pos0, const uint8_t *key_mask, float *dx, const smol_layer_grads *gr,
                          int accumulate, char *ws, const BwWs &L, hipStream_t s) {
  const int M = B * T, H = D.H, I = D.I, d = D.d, QD = D.nq * d, KD = D.nkv * d, C3 = QD + 2 * KD;
  const bool rope_on = !(D.nope_every > 0 && (layer + 1) % D.nope_every == 0);
  const int window = (!rope_on && D.window > 0) ? D.window : 0;
  auto F = [&](size_t off) { return (float *)(ws + off); };
  float *u = F(L.u), *r1 = F(L.r1), *qkv = F(L.qkv), *o = F(L.o), *h = F(L.h), *wn = F(L.wn), *r2 = F(L.r2);
  float *gu = F(L.gu), *dgu = F(L.dgu), *y = F(L.y), *dwn = F(L.dwn), *dh = F(L.dh), *dO = F(L.dO);
  float *dqkv = F(L.dqkv), *du = F(L.du), *npart = F(L.npart), *gpart = F(L.gpart);
  const float *Wq = (const float *)w->wq, *Wk = (const float *)w->wk, *Wv = (const float *)w->wv;
  const float *Wo = (const float *)w->wo, *Wg = (const float *)w->w_gate, *Wu = (const float *)w->w_up;
  const float *Wd = (const float *)w->w_down;
  const float *an = (const float *)w->attn_norm, *mn = (const float *)w->mlp_norm;
  const int wgrad = accumulate ? smol::BW_ACCUM : smol::BW_STORE;
  using smol::BW_NN;
  using smol::BW_NT;
  using smol::BW_TN;
  using smol::BW_STORE;
  // every GEMM goes through here: the K split its shape calls for, over gpart
  auto gemm = [&](int layout, int epi, smol::BwGemm g) -> hipError_t {
    g.ksplit = smol::bw_gemm_ksplit(g.M, g.N, g.K, epi);
    g.part = gpart;
    return smol::bw_gemm(layout, epi, g, s);
  };

  // ---- forward, keeping what the backward reads
  SMOL_LAUNCH(SMOL_K_BW_ROWS, smol::bw_rms_fwd(x, an, u, r1, M, H, D.eps, s));
  SMOL_LAUNCH(SMOL_K_BW_GEMM, gemm(BW_NT, BW_STORE, gemm_args(operand(u, H), operand(Wq, H, Wk, QD, Wv, QD + KD),
                                                              M, C3, H, qkv, C3)));
  float2 *rope_cs = (float2 *)F(L.rope);
  if (rope_on) {
    smol::InvFreq inv{};
    fill_inv_freq(D, inv.v);
    SMOL_LAUNCH(SMOL_K_BW_ROWS, smol::bw_rope_table(rope_cs, M, T, d, pos0, inv, s));
    SMOL_LAUNCH(SMOL_K_BW_ROWS, smol::bw_rope(qkv, M, C3, D.nq + D.nkv, d, rope_cs, s));
  }
  smol::BwAttn at{};
  at.qkv = qkv;
  at.ld = C3;
  at.B = B;
  at.T = T;
  at.nq = D.nq;
  at.nkv = D.nkv;
  at.G = D.G;
  at.D = d;
  at.key_mask = key_mask;
  at.window = window;
  at.scale = 1.0f / std::sqrt((float)d);
  at.scale2 = (float)(1.4426950408889634 / std::sqrt((double)d));
  at.o = o;
  at.lse = F(L.lse);
  at.dO = dO;
  at.dsum = F(L.dsum);
  at.dqkv = dqkv;
  at.part = F(L.part);
  at.rope_on = rope_on ? 1 : 0;
  at.rope_cs = rope_cs;
  SMOL_LAUNCH(SMOL_K_BW_ATTN_FWD, smol::bw_attention(0, at, s));
  {  // h = x + o W_o^T
    smol::BwGemm g = gemm_args(operand(o, QD), operand(Wo, QD), M, H, QD, h, H);
    g.R = x;
    g.ldr = H;
    SMOL_LAUNCH(SMOL_K_BW_GEMM, gemm(BW_NT, smol::BW_RESID, g));
  }
  SMOL_LAUNCH(SMOL_K_BW_ROWS, smol::bw_rms_fwd(h, mn, wn, r2, M, H, D.eps, s));
  SMOL_LAUNCH(SMOL_K_BW_GEMM, gemm(BW_NT, BW_STORE, gemm_args(operand(wn, H), operand(Wg, H, Wu, I), M, 2 * I, H,
                                                              gu, 2 * I)));

  // ---- MLP: dy_mlp = dy W_d, through SwiGLU into d(gate | up), and y = silu(g) u
  {
    smol::BwGemm g = gemm_args(operand(dy, H), operand(Wd, I), M, I, H, dgu, 2 * I);
    g.G = gu;
    g.ldg = 2 * I;
    g.half = I;
    g.Y = y;
    g.ldy = I;
    SMOL_LAUNCH(SMOL_K_BW_GEMM, gemm(BW_NN, smol::BW_SWIGLU, g));
  }
  SMOL_LAUNCH(SMOL_K_BW_GEMM, gemm(BW_TN, wgrad, gemm_args(operand(dy, H), operand(y, I), H, I, M, gr->w_down, I)));
  SMOL_LAUNCH(SMOL_K_BW_GEMM, gemm(BW_NN, BW_STORE, gemm_args(operand(dgu, 2 * I), operand(Wg, H, Wu, I), M, H,
                                                              2 * I, dwn, H)));
  // dW_gate | dW_up in one launch: rows [0, I) of d(gate | up)^T w to W_gate's gradient
  SMOL_LAUNCH(SMOL_K_BW_GEMM, gemm(BW_TN, wgrad, with_c_segments(gemm_args(operand(dgu, 2 * I), operand(wn, H), 2 * I,
                                                                           H, M, gr->w_gate, H),
                                                                 gr->w_up, I)));
  // dh = dy + RMSNorm_m backward
  SMOL_LAUNCH(SMOL_K_BW_ROWS, smol::bw_rms_bwd(dwn, h, r2, mn, dy, dh, npart, M, H, s));
  SMOL_LAUNCH(SMOL_K_BW_ROWS, smol::bw_colsum(npart, smol::bw_rms_part_rows(M), H, gr->mlp_norm, accumulate, s));

  // ---- attention
  SMOL_LAUNCH(SMOL_K_BW_GEMM, gemm(BW_TN, wgrad, gemm_args(operand(dh, H), operand(o, QD), H, QD, M, gr->wo, QD)));
  SMOL_LAUNCH(SMOL_K_BW_GEMM, gemm(BW_NN, BW_STORE, gemm_args(operand(dh, H), operand(Wo, QD), M, QD, H, dO, QD)));
  SMOL_LAUNCH(SMOL_K_BW_ROWS, smol::bw_rowdot(dO, o, F(L.dsum), M, T, D.nq, d, s));
  SMOL_LAUNCH(SMOL_K_BW_ATTN_DQ, smol::bw_attention(1, at, s));
  SMOL_LAUNCH(SMOL_K_BW_ATTN_DKDV, smol::bw_attention(2, at, s));
  SMOL_LAUNCH(SMOL_K_BW_ROWS, smol::bw_kv_reduce(F(L.part), dqkv, M, D.nq, D.nkv, D.G, d, C3, s));
  // dW_q | dW_k | dW_v in one launch
  SMOL_LAUNCH(SMOL_K_BW_GEMM, gemm(BW_TN, wgrad, with_c_segments(gemm_args(operand(dqkv, C3), operand(u, H), C3, H, M,
                                                                           gr->wq, H),
                                                                 gr->wk, QD, gr->wv, QD + KD)));
  SMOL_LAUNCH(SMOL_K_BW_GEMM, gemm(BW_NN, BW_STORE, gemm_args(operand(dqkv, C3), operand(Wq, H, Wk, QD, Wv, QD + KD),
                                                              M, H, C3, du, H)));
  // dx = dh + RMSNorm_a backward
  SMOL_LAUNCH(SMOL_K_BW_ROWS, smol::bw_rms_bwd(du, x, r1, an, dh, dx, npart, M, H, s));
  SMOL_LAUNCH(SMOL_K_BW_ROWS, smol::bw_colsum(npart, smol::bw_rms_part_rows(M), H, gr->attn_norm, accumulate, s));
  return SMOL_OK;
}

// ------------------------------------------------------------------ fixed scratch
// smol_decode_step_static runs the decode step on a file-scope device array instead
// of a caller's workspace, for callers that cannot allocate. In host code `scratch`
// names a host-side stand-in, not device memory: its device address is taken once
// per device with hipGetSymbolAddress (with that device current) and only that
// address is ever handed to kernels.
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)SMOL_STATIC_SCRATCH_MIB << 20;
__device__ __attribute__((aligned(256))) char scratch[STATIC_SCRATCH_BYTES];

struct ScratchPtrs {
  std::mutex mu;
  std::map<int, char *> ptr;  // device -> address of that device's copy of `scratch`
} g_scratch;

smol_status static_scratch(char **out) {
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return fail(SMOL_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_scratch.mu);
  auto it = g_scratch.ptr.find(device);
  if (it == g_scratch.ptr.end()) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(SMOL_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    if ((uintptr_t)p % ALIGN) return fail(SMOL_ERR_HIP, "scratch is not 256-byte aligned");
    it = g_scratch.ptr.emplace(device, (char *)p).first;
  }
  *out = it->second;
  return SMOL_OK;
}

}  // namespace

extern "C" {

smol_status smol_workspace_size(const smol_config *cfg, int op, int batch, int seq, size_t *bytes) {
  g_err.clear();
  Dims D;
  smol_status st = check_config(cfg, &D);
  if (st != SMOL_OK) return st;
  if (!bytes) return fail(SMOL_ERR_INVALID_ARG, "bytes is NULL");
  if (op != SMOL_OP_BLOCK && op != SMOL_OP_PREFILL && op != SMOL_OP_DECODE) return fail(SMOL_ERR_INVALID_ARG, "op %d", op);
  if (batch < 1 || seq < 1) return fail(SMOL_ERR_INVALID_ARG, "batch and seq must be >= 1");
  *bytes = layout(D, op, batch, seq).total;
  return SMOL_OK;
}

smol_status smol_block_forward(const smol_config *cfg, const smol_layer_weights *w, const float *x_in, float *x_out,
                               int batch, int seq, int pos0, void *k_cache, void *v_cache, int cache_cap, void *ws,
                               size_t ws_bytes, void *stream) {
  g_err.clear();
  Dims D;
  smol_status st = check_config(cfg, &D);
  if (st != SMOL_OK) return st;
  if ((st = check_layer(w, 0)) != SMOL_OK) return st;
  if (!x_in || !x_out) return fail(SMOL_ERR_INVALID_ARG, "x_in / x_out is NULL");
  if ((st = check_aligned({{x_in, "x_in"}, {x_out, "x_out"}, {k_cache, "k_cache"}, {v_cache, "v_cache"}})) != SMOL_OK)
    return st;
  if (batch < 1 || seq < 1) return fail(SMOL_ERR_INVALID_ARG, "batch %d, seq %d must be >= 1", batch, seq);
  if (pos0 < 0) return fail(SMOL_ERR_INVALID_ARG, "pos0 %d < 0", pos0);
  if ((long)pos0 + seq > D.max_pos)
    return fail(SMOL_ERR_INVALID_ARG, "pos0 + seq = %ld exceeds max_pos %d", (long)pos0 + seq, D.max_pos);
  if (!k_cache != !v_cache) return fail(SMOL_ERR_INVALID_ARG, "k_cache and v_cache must both be set or both NULL");
  if (k_cache && cache_cap < pos0 + seq)
    return fail(SMOL_ERR_INVALID_ARG, "cache_cap %d < pos0 + seq = %d", cache_cap, pos0 + seq);
  Ws lay;
  if ((st = check_ws(D, SMOL_OP_BLOCK, batch, seq, ws, ws_bytes, &lay)) != SMOL_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  return D.bf16 ? block_impl<bf16>(D, w, x_in, x_out, batch, seq, pos0, k_cache, v_cache, cache_cap, (char *)ws, lay, s)
                : block_impl<float>(D, w, x_in, x_out, batch, seq, pos0, k_cache, v_cache, cache_cap, (char *)ws, lay, s);
}

smol_status smol_model_prefill_ex(const smol_config *cfg, const smol_model_weights *w, const int32_t *ids, int batch,
                                  int seq, int pos0, const uint8_t *key_mask, void *logits, void *k_cache,
                                  void *v_cache, int cache_cap, void *ws, size_t ws_bytes, void *stream) {
  g_err.clear();
  Dims D;
  smol_status st = check_config(cfg, &D);
  if (st != SMOL_OK) return st;
  if ((st = check_model(D, w)) != SMOL_OK) return st;
  if (!ids || !logits) return fail(SMOL_ERR_INVALID_ARG, "ids / logits is NULL");
  if ((st = check_aligned({{logits, "logits"}, {k_cache, "k_cache"}, {v_cache, "v_cache"}})) != SMOL_OK) return st;
  if (batch < 1 || seq < 1) return fail(SMOL_ERR_INVALID_ARG, "batch %d, seq %d must be >= 1", batch, seq);
  if (pos0 < 0) return fail(SMOL_ERR_INVALID_ARG, "pos0 %d < 0", pos0);
  if ((long)pos0 + seq > D.max_pos)
    return fail(SMOL_ERR_INVALID_ARG, "pos0 + seq = %ld exceeds max_pos %d", (long)pos0 + seq, D.max_pos);
  if (!k_cache != !v_cache) return fail(SMOL_ERR_INVALID_ARG, "k_cache and v_cache must both be set or both NULL");
  if (pos0 > 0 && !k_cache) return fail(SMOL_ERR_INVALID_ARG, "pos0 %d > 0 needs the caches of positions before it", pos0);
  if (k_cache && cache_cap < pos0 + seq)
    return fail(SMOL_ERR_INVALID_ARG, "cache_cap %d < pos0 + seq = %d", cache_cap, pos0 + seq);
  Ws lay;
  if ((st = check_ws(D, SMOL_OP_PREFILL, batch, seq, ws, ws_bytes, &lay)) != SMOL_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  return D.bf16 ? prefill_impl<bf16>(D, w, ids, batch, seq, logits, k_cache, v_cache, cache_cap, (char *)ws, lay, s,
                                     pos0, key_mask)
                : prefill_impl<float>(D, w, ids, batch, seq, logits, k_cache, v_cache, cache_cap, (char *)ws, lay, s,
                                      pos0, key_mask);
}

smol_status smol_model_prefill(const smol_config *cfg, const smol_model_weights *w, const int32_t *ids, int batch,
                               int seq, void *logits, void *k_cache, void *v_cache, int cache_cap, void *ws,
                               size_t ws_bytes, void *stream) {
  return smol_model_prefill_ex(cfg, w, ids, batch, seq, 0, nullptr, logits, k_cache, v_cache, cache_cap, ws, ws_bytes,
                               stream);
}

smol_status smol_decode_step(const smol_config *cfg, const smol_model_weights *w, const int32_t *ids,
                             const int32_t *cache_len, int batch, void *k_cache, void *v_cache, int cache_cap,
                             void *logits, void *ws, size_t ws_bytes, void *stream) {
  return smol_decode_step_ex(cfg, w, ids, cache_len, batch, nullptr, k_cache, v_cache, cache_cap, logits, ws, ws_bytes,
                             stream);
}

smol_status smol_decode_step_ex(const smol_config *cfg, const smol_model_weights *w, const int32_t *ids,
                                const int32_t *cache_len, int batch, const uint8_t *key_mask, void *k_cache,
                                void *v_cache, int cache_cap, void *logits, void *ws, size_t ws_bytes, void *stream) {
  g_err.clear();
  Dims D;
  smol_status st = check_config(cfg, &D);
  if (st != SMOL_OK) return st;
  if ((st = check_model(D, w)) != SMOL_OK) return st;
  if (!ids || !cache_len || !logits) return fail(SMOL_ERR_INVALID_ARG, "ids / cache_len / logits is NULL");
  if (!k_cache || !v_cache) return fail(SMOL_ERR_INVALID_ARG, "decode needs k_cache and v_cache");
  if ((st = check_aligned({{logits, "logits"}, {k_cache, "k_cache"}, {v_cache, "v_cache"}})) != SMOL_OK) return st;
  if (batch < 1) return fail(SMOL_ERR_INVALID_ARG, "batch %d must be >= 1", batch);
  if (cache_cap < 1) return fail(SMOL_ERR_INVALID_ARG, "cache_cap %d must be >= 1", cache_cap);
  Ws lay;
  if ((st = check_ws(D, SMOL_OP_DECODE, batch, cache_cap, ws, ws_bytes, &lay)) != SMOL_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  return D.bf16 ? decode_impl<bf16>(D, w, ids, cache_len, batch, k_cache, v_cache, cache_cap, logits, (char *)ws, lay, s,
                                    key_mask)
                : decode_impl<float>(D, w, ids, cache_len, batch, k_cache, v_cache, cache_cap, logits, (char *)ws, lay,
                                     s, key_mask);
}

smol_status smol_decode_step_static(const smol_config *cfg, const smol_model_weights *w, const int32_t *ids,
                                    const int32_t *cache_len, int batch, void *k_cache, void *v_cache, int cache_cap,
                                    void *logits, void *stream) {
  g_err.clear();
  Dims D;
  smol_status st = check_config(cfg, &D);
  if (st != SMOL_OK) return st;
  if ((st = check_model(D, w)) != SMOL_OK) return st;
  if (!ids || !cache_len || !logits) return fail(SMOL_ERR_INVALID_ARG, "ids / cache_len / logits is NULL");
  if (!k_cache || !v_cache) return fail(SMOL_ERR_INVALID_ARG, "decode needs k_cache and v_cache");
  if ((st = check_aligned({{logits, "logits"}, {k_cache, "k_cache"}, {v_cache, "v_cache"}})) != SMOL_OK) return st;
  if (batch < 1) return fail(SMOL_ERR_INVALID_ARG, "batch %d must be >= 1", batch);
  if (cache_cap < 1) return fail(SMOL_ERR_INVALID_ARG, "cache_cap %d must be >= 1", cache_cap);
  const Ws lay = layout(D, SMOL_OP_DECODE, batch, cache_cap);
  if (lay.total > STATIC_SCRATCH_BYTES)
    return fail(SMOL_ERR_WORKSPACE, "decode step needs %zu bytes of scratch, more than the fixed %zu (%d MiB)",
                lay.total, STATIC_SCRATCH_BYTES, SMOL_STATIC_SCRATCH_MIB);
  char *ws = nullptr;
  if ((st = static_scratch(&ws)) != SMOL_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  return D.bf16 ? decode_impl<bf16>(D, w, ids, cache_len, batch, k_cache, v_cache, cache_cap, logits, ws, lay, s)
                : decode_impl<float>(D, w, ids, cache_len, batch, k_cache, v_cache, cache_cap, logits, ws, lay, s);
}

smol_status smol_generate_workspace_size(const smol_config *cfg, int batch, int prompt_len, int max_new,
                                         int cache_cap, size_t *bytes) {
  g_err.clear();
  Dims D;
  smol_status st = check_config(cfg, &D);
  if (st != SMOL_OK) return st;
  if (!bytes) return fail(SMOL_ERR_INVALID_ARG, "bytes is NULL");
  if (batch < 1 || prompt_len < 1 || max_new < 1 || cache_cap < 1)
    return fail(SMOL_ERR_INVALID_ARG, "batch, prompt_len, max_new and cache_cap must be >= 1");
  *bytes = gen_layout(D, batch, prompt_len, max_new, cache_cap).total;
  return SMOL_OK;
}

smol_status smol_generate(const smol_config *cfg, const smol_model_weights *w, const int32_t *prompt_ids,
                          const int32_t *prompt_lens, int batch, int prompt_len, int max_new, float temperature,
                          int top_k, float top_p,
                          const float *uniforms, int32_t *out_ids, void *k_cache, void *v_cache, int cache_cap,
                          void *ws, size_t ws_bytes, void *stream) {
  g_err.clear();
  Dims D;
  smol_status st = check_config(cfg, &D);
  if (st != SMOL_OK) return st;
  if ((st = check_model(D, w)) != SMOL_OK) return st;
  if (!prompt_ids || !out_ids) return fail(SMOL_ERR_INVALID_ARG, "prompt_ids / out_ids is NULL");
  if (!k_cache || !v_cache) return fail(SMOL_ERR_INVALID_ARG, "generation needs k_cache and v_cache");
  if ((st = check_aligned({{k_cache, "k_cache"}, {v_cache, "v_cache"}})) != SMOL_OK) return st;
  if (batch < 1 || prompt_len < 1 || max_new < 1)
    return fail(SMOL_ERR_INVALID_ARG, "batch %d, prompt_len %d, max_new %d must be >= 1", batch, prompt_len, max_new);
  const long last = (long)prompt_len + max_new - 1;  // positions fed: 0 .. last - 1
  if (last > D.max_pos) return fail(SMOL_ERR_INVALID_ARG, "prompt_len + max_new - 1 = %ld exceeds max_pos %d", last, D.max_pos);
  if (last > cache_cap) return fail(SMOL_ERR_INVALID_ARG, "prompt_len + max_new - 1 = %ld exceeds cache_cap %d", last, cache_cap);
  if (!(temperature >= 0.f) || !std::isfinite(temperature))
    return fail(SMOL_ERR_INVALID_ARG, "temperature must be finite and >= 0");
  if (!(top_p >= 0.f)) return fail(SMOL_ERR_INVALID_ARG, "top_p must be >= 0");
  if (top_k < 0) return fail(SMOL_ERR_INVALID_ARG, "top_k %d < 0", top_k);
  if (temperature > 0.f && !uniforms) return fail(SMOL_ERR_INVALID_ARG, "uniforms is NULL");
  if (!ws) return fail(SMOL_ERR_INVALID_ARG, "ws is NULL");
  if ((uintptr_t)ws % ALIGN) return fail(SMOL_ERR_INVALID_ARG, "ws must be 256-byte aligned");
  const GenWs g = gen_layout(D, batch, prompt_len, max_new, cache_cap);
  if (ws_bytes < g.total) return fail(SMOL_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, g.total);
  hipStream_t s = (hipStream_t)stream;
  return D.bf16 ? generate_impl<bf16>(D, w, prompt_ids, prompt_lens, batch, prompt_len, max_new, temperature, top_k,
                                      top_p, uniforms, out_ids, k_cache, v_cache, cache_cap, (char *)ws, g, s)
                : generate_impl<float>(D, w, prompt_ids, prompt_lens, batch, prompt_len, max_new, temperature, top_k,
                                       top_p, uniforms, out_ids, k_cache, v_cache, cache_cap, (char *)ws, g, s);
}

smol_status smol_sample(const void *logits, int dtype, int batch, int vocab, int64_t row_stride, float temperature,
                        int top_k, float top_p, const float *uniforms, int32_t *next_ids, void *stream) {
  g_err.clear();
  if (!logits || !next_ids) return fail(SMOL_ERR_INVALID_ARG, "logits / next_ids is NULL");
  if (dtype != SMOL_F32 && dtype != SMOL_BF16) return fail(SMOL_ERR_INVALID_ARG, "dtype %d unknown", dtype);
  if (batch < 1 || vocab < 1) return fail(SMOL_ERR_INVALID_ARG, "batch %d, vocab %d must be >= 1", batch, vocab);
  if (batch > 1 && row_stride < vocab)
    return fail(SMOL_ERR_INVALID_ARG, "row_stride %lld < vocab %d", (long long)row_stride, vocab);
  if (!(temperature >= 0.f) || !std::isfinite(temperature))
    return fail(SMOL_ERR_INVALID_ARG, "temperature must be finite and >= 0");
  if (!(top_p >= 0.f)) return fail(SMOL_ERR_INVALID_ARG, "top_p must be >= 0");
  if (top_k < 0) return fail(SMOL_ERR_INVALID_ARG, "top_k %d < 0", top_k);
  if (temperature > 0.f && !uniforms) return fail(SMOL_ERR_INVALID_ARG, "uniforms is NULL");
  hipStream_t s = (hipStream_t)stream;
  SMOL_LAUNCH(SMOL_K_SAMPLE, dtype == SMOL_BF16
                                 ? smol::sample_next<bf16>((const bf16 *)logits, (long)row_stride, batch, vocab,
                                                           temperature, top_k, top_p, uniforms, next_ids, s)
                                 : smol::sample_next<float>((const float *)logits, (long)row_stride, batch, vocab,
                                                            temperature, top_k, top_p, uniforms, next_ids, s));
  return SMOL_OK;
}


smol_status smol_block_backward_workspace_size(const smol_config *cfg, int batch, int seq, size_t *bytes) {
  g_err.clear();
  Dims D;
  smol_status st = check_config(cfg, &D);
  if (st != SMOL_OK) return st;
  if (!bytes) return fail(SMOL_ERR_INVALID_ARG, "bytes is NULL");
  if (batch < 1 || seq < 1) return fail(SMOL_ERR_INVALID_ARG, "batch and seq must be >= 1");
  *bytes = bw_layout(D, batch, seq).total;
  return SMOL_OK;
}

smol_status smol_block_backward(const smol_config *cfg, const smol_layer_weights *w, int layer, const float *x,
                                const float *dy, int batch, int seq, int pos0, const uint8_t *key_mask, float *dx,
                                const smol_layer_grads *grads, int accumulate, void *ws, size_t ws_bytes,
                                void *stream) {
  g_err.clear();
  Dims D;
  smol_status st = check_config(cfg, &D);
  if (st != SMOL_OK) return st;
  if ((st = check_layer(w, layer)) != SMOL_OK) return st;
  if (layer < 0 || layer >= D.L) return fail(SMOL_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, D.L);
  if (!x || !dy || !dx) return fail(SMOL_ERR_INVALID_ARG, "x / dy / dx is NULL");
  if (dx == x || dx == dy) return fail(SMOL_ERR_INVALID_ARG, "dx may not alias x or dy");
  if (!grads) return fail(SMOL_ERR_INVALID_ARG, "grads is NULL");
  {
    float *const g[9] = {grads->attn_norm, grads->wq, grads->wk, grads->wv, grads->wo,
                         grads->mlp_norm, grads->w_gate, grads->w_up, grads->w_down};
    for (int i = 0; i < 9; ++i)
      if (!g[i]) return fail(SMOL_ERR_INVALID_ARG, "grads: gradient %d is NULL", i);
  }
  if (accumulate != 0 && accumulate != 1) return fail(SMOL_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  if (batch < 1 || seq < 1) return fail(SMOL_ERR_INVALID_ARG, "batch %d, seq %d must be >= 1", batch, seq);
  if (pos0 < 0) return fail(SMOL_ERR_INVALID_ARG, "pos0 %d < 0", pos0);
  if ((long)pos0 + seq > D.max_pos)
    return fail(SMOL_ERR_INVALID_ARG, "pos0 + seq = %ld exceeds max_pos %d", (long)pos0 + seq, D.max_pos);
  if ((long)batch * seq * std::max(2 * D.I, (D.nq + 2 * D.nkv) * D.d) > INT32_MAX)
    return fail(SMOL_ERR_UNSUPPORTED, "batch * seq too large");
  const void *aligned[3] = {x, dy, dx};
  for (const void *p : aligned)
    if ((uintptr_t)p % 16) return fail(SMOL_ERR_INVALID_ARG, "x, dy and dx must be 16-byte aligned");
  const BwWs lay = bw_layout(D, batch, seq);
  if (!ws) return fail(SMOL_ERR_INVALID_ARG, "ws is NULL");
  if (ws_bytes < lay.total) return fail(SMOL_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, lay.total);
  if ((uintptr_t)ws % ALIGN) return fail(SMOL_ERR_INVALID_ARG, "ws must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  smol_layer_weights wf = *w;
  if (D.bf16) {  // widen the weights to float32 once (exact) and differentiate in float32
    const void *src[9] = {w->attn_norm, w->wq, w->wk, w->wv, w->wo, w->mlp_norm, w->w_gate, w->w_up, w->w_down};
    const void **dst[9] = {&wf.attn_norm, &wf.wq, &wf.wk, &wf.wv, &wf.wo, &wf.mlp_norm, &wf.w_gate, &wf.w_up, &wf.w_down};
    const size_t QD = (size_t)D.nq * D.d, KD = (size_t)D.nkv * D.d, H = D.H;
    const size_t n[9] = {H, QD * H, KD * H, KD * H, H * QD, H, (size_t)D.I * H, (size_t)D.I * H, H * D.I};
    for (int i = 0; i < 9; ++i) {
      float *to = (float *)((char *)ws + lay.wf32[i]);
      SMOL_LAUNCH(SMOL_K_BW_ROWS, smol::bw_widen((const bf16 *)src[i], to, n[i], s));
      *dst[i] = to;
    }
  }
  return backward_impl(D, &wf, layer, x, dy, batch, seq, pos0, key_mask, dx, grads, accumulate, (char *)ws, lay, s);
}

const char *smol_status_string(smol_status s) {
  // A C caller may pass any int; in C++ an enum object outside the enumerators' range
  // is undefined, so the value is read as the int it is.
  int v;
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case SMOL_OK: return "ok";
    case SMOL_ERR_INVALID_ARG: return "invalid argument";
    case SMOL_ERR_UNSUPPORTED: return "unsupported shape";
    case SMOL_ERR_WORKSPACE: return "workspace too small";
    case SMOL_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char *smol_last_error(void) { return g_err.c_str(); }

smol_status smol_timing_begin(int kernel, int max_launches) {
  g_err.clear();
  if (kernel < 0 || kernel >= SMOL_K_COUNT) return fail(SMOL_ERR_INVALID_ARG, "kernel class %d", kernel);
  if (max_launches < 1 || max_launches > 1 << 16) return fail(SMOL_ERR_INVALID_ARG, "max_launches %d", max_launches);
  std::lock_guard<std::mutex> lk(g_timing.mu);
  while ((int)g_timing.ev.size() < 2 * max_launches) {
    hipEvent_t e;
    hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) return fail(SMOL_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(err));
    g_timing.ev.push_back(e);
  }
  g_timing.kernel = kernel;
  g_timing.max = max_launches;
  g_timing.count = 0;
  return SMOL_OK;
}

smol_status smol_timing_end(float *total_ms, int *launches) {
  g_err.clear();
  if (!total_ms || !launches) return fail(SMOL_ERR_INVALID_ARG, "total_ms / launches is NULL");
  std::lock_guard<std::mutex> lk(g_timing.mu);
  float sum = 0.f;
  for (int i = 0; i < g_timing.count; ++i) {
    hipError_t err = hipEventSynchronize(g_timing.ev[2 * i + 1]);
    if (err != hipSuccess) return fail(SMOL_ERR_HIP, "hipEventSynchronize: %s", hipGetErrorString(err));
    float ms = 0.f;
    err = hipEventElapsedTime(&ms, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]);
    if (err != hipSuccess) return fail(SMOL_ERR_HIP, "hipEventElapsedTime: %s", hipGetErrorString(err));
    sum += ms;
  }
  *total_ms = sum;
  *launches = g_timing.count;
  g_timing.kernel = -1;
  g_timing.count = 0;
  return SMOL_OK;
}

}  // extern "C"
