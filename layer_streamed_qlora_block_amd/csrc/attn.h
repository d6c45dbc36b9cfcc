// Causal GQA attention launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// q, k, v live in one bf16 buffer qkv [B*S, ld] at column offsets q_off,
// k_off, v_off (heads back to back, hd each).  Head h reads kv head
// h / (H / KV).  out bf16 [B*S, ldo]; lse float [B, H, S] (natural log).
struct AttnArgs {
  const uint16_t* qkv; int64_t ld; int q_off, k_off, v_off;
  int S, H, KV, hd;
  float scale;                 // 1/sqrt(hd)
  uint16_t* out; int64_t ldo;
  float* lse;
};
int attn_fwd(const AttnArgs& a, int B, hipStream_t st);

// Backward: dO and O bf16 [B*S, lddo] (o is the forward output); D float
// [B, H, S] scratch; dq float [B*S, lddq]; dk, dv float [B*S, lddkv] hold one
// partial per QUERY head (lddkv >= H*hd): the kv head's gradient is the sum
// of the partials of its H/KV query heads.
struct AttnBwdArgs {
  const uint16_t* qkv; int64_t ld; int q_off, k_off, v_off;
  int S, H, KV, hd;
  float scale;
  const uint16_t* dO; const uint16_t* O; int64_t lddo;
  const float* lse; float* D;
  float* dq; int64_t lddq;
  float* dk; float* dv; int64_t lddkv;
};
int attn_bwd(const AttnBwdArgs& a, int B, hipStream_t st);
// dK / dV of each kv head from the per-query-head partials of attn_bwd:
// out [T, KV*hd] = the sum, in head order, of the H/KV partials in part [T, H*hd].
void attn_group_sum(const float* part, float* out, int T, int H, int KV, int hd, hipStream_t st);

// The whole attention backward of the C ABI (argument checks, D, dQ, the
// per-query-head dK / dV partials and their group sums) over caller scratch
// ws: qls_attention_ws_bytes(B, S, H, hd) bytes.  ws_cap >= 0 is ws's size,
// checked (QLS_EINVAL when too small); -1 skips the check.  Returns a QLS_*
// code with the message set.
int attention_bwd_run(const uint16_t* qkv, const uint16_t* out, const uint16_t* dout, const float* lse, int B,
                      int S, int H, int KV, int hd, float* dq, float* dk, float* dv, void* ws, int64_t ws_cap,
                      hipStream_t st);
