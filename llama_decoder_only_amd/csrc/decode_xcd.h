// Host-side declarations of the one-launch decode step (decode_xcd.hip).
#pragma once

#include "kernels.h"

namespace smol {

// The whole decode step of a bfloat16 model with head_dim 64 as one persistent
// launch partitioned by XCD (decode_xcd.hip), up to the final norm: it leaves the
// head's operand in xs, ss_p and ss_q as the last block of the multi-kernel path
// does, and the lm_head GEMM follows as its own launch. Limits: decode_xcd_fits.
constexpr int DX_UMAX = 3;      // 16-column units per workgroup of the gate/up phase (weights in LDS)
constexpr int DX_UREG = 2;      // the same for QKV, o_proj and down (weights in registers)
constexpr int DX_HMAX = 576;    // hidden size (the gate/up weights of a workgroup then fit in LDS)
constexpr int DX_KMAX = 1536;   // longest contraction (the intermediate size)
constexpr int DX_LMAX = 40;     // layers (their weight pointers travel as kernel arguments)
constexpr int DX_SPMAX = 32;    // attention splits per (row, kv head)
// Control block: abort word, error word, then one flag per workgroup (16 words apart).
constexpr int DX_CTRL_ABORT = 0, DX_CTRL_ERR = 16, DX_CTRL_WORDS = 32;
struct DxLayer {
  const bf16 *wq, *wk, *wv, *wo, *wg, *wu, *wd, *an, *mn;
};
struct DecodeXcdArgs {
  int B, H, nq, nkv, I, L, V, cap, max_pos, nope_every, window, nwx, sp, mask_ld;
  float eps;
  const int32_t *ids, *cache_len;
  const uint8_t *key_mask;  // [B, mask_ld] over key indices, or nullptr
  const bf16 *embed, *final_norm;
  bf16 *kc, *vc;            // [L, B, nkv, cap, 64]
  float *x;                 // [B, H] residual stream
  f16 *q, *o, *y;           // [B, H], [B, H], [B, I]
  float *part;              // [B, nq, sp, 66] attention partials
  f16 *xs;                  // [B, H] head operand
  float *ss_p, *ss_q;       // [H / 64, B]
  uint32_t *ctrl;           // decode_xcd_ctrl_words(nwx), zeroed by decode_xcd before the step
  unsigned long long deadline;  // barrier wait limit after the step starts, shader-clock ticks
  double inv_freq[32];
  DxLayer layer[DX_LMAX];
};
unsigned long long decode_xcd_deadline_ticks();
int decode_xcd_groups_per_xcd();  // workgroups per XCD group on the current device (CUs / 8)
bool decode_xcd_fits(int B, int H, int nq, int nkv, int d, int I, int L, int cap, int nwx);
int decode_xcd_splits(int B, int nkv, int nwx);
size_t decode_xcd_part_floats(int B, int nq, int nkv);  // attention partials, any admitted nwx
size_t decode_xcd_ctrl_words(int nwx);
hipError_t decode_xcd(const DecodeXcdArgs &a, hipStream_t s);

}  // namespace smol
