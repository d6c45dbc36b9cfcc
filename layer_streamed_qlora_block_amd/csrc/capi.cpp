// C ABI: error plumbing, the NF4 dequant hook, the one-linear and the
// attention entry points.
#include <algorithm>
#include <cmath>
#include <initializer_list>
#include <string>

#include "attn.h"
#include "gemm.h"
#include "internal.h"
#include "ops.h"

static thread_local std::string t_err;

void set_error(const std::string& msg) { t_err = msg; }
int fail(int code, const std::string& msg) {
  t_err = msg;
  return code;
}
int hip_fail(hipError_t e, const char* what) {
  t_err = std::string(what) + ": " + hipGetErrorString(e);
  return QLS_EHIP;
}

extern "C" {

int qls_abi_version(void) { return QLS_ABI_VERSION; }
const char* qls_last_error(void) { return t_err.c_str(); }

int qls_nf4_dequant_dev(const uint8_t* d_codes, const float* d_absmax, int64_t n, uint16_t* d_out,
                        void* stream) {
  if (!d_codes || !d_absmax || !d_out) return fail(QLS_EINVAL, "NULL buffer");
  if (n < 0 || n % 64) return fail(QLS_EINVAL, "n must be a non-negative multiple of 64");
  if (nf4_dequant_launch(d_codes, d_absmax, n, d_out, (hipStream_t)stream))
    return fail(QLS_EHIP, "codebook upload failed");
  QLS_HIP(hipGetLastError());
  return QLS_OK;
}

int qls_nf4_absmax_expand_dev(const uint8_t* d_q8, const float* d_scales, int64_t nblocks, float* d_out,
                              void* stream) {
  if (!d_q8 || !d_scales || !d_out) return fail(QLS_EINVAL, "NULL buffer");
  if (nblocks < 0) return fail(QLS_EINVAL, "nblocks must be non-negative");
  absmax_expand_flat_launch(d_q8, d_scales, nblocks, d_out, (hipStream_t)stream);
  QLS_HIP(hipGetLastError());
  return QLS_OK;
}

int qls_adamw_step(float* d_params, const float* d_grads, float* d_m, float* d_v, int64_t n, int step,
                   double lr, double beta1, double beta2, double eps, double weight_decay, void* stream) {
  if (!d_params || !d_grads || !d_m || !d_v) return fail(QLS_EINVAL, "NULL buffer");
  if (n < 0 || step < 1) return fail(QLS_EINVAL, "n must be >= 0 and step >= 1");
  if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0) || !(eps > 0.0))
    return fail(QLS_EINVAL, "betas must be in [0, 1) and eps positive");
  adamw_update(d_params, d_grads, d_m, d_v, n, step, lr, beta1, beta2, eps, weight_decay, (hipStream_t)stream);
  QLS_HIP(hipGetLastError());
  return QLS_OK;
}

int64_t qls_linear_ws_bytes(int T, int N, int K, int r) {
  if (T <= 0 || N <= 0 || K <= 0 || r <= 0) return fail(QLS_EINVAL, "sizes must be positive");
  return linear_ws_bytes(T, N, K, r);
}

int qls_linear_fwd(const uint8_t* codes, const float* absmax, int N, int K, const uint16_t* x, int T,
                   const uint16_t* A, const uint16_t* B, int r, float alpha, uint16_t* y,
                   uint16_t* u, void* ws, void* stream) {
  if (!codes || !absmax || !x || !y) return fail(QLS_EINVAL, "NULL buffer");
  if (T <= 0 || N <= 0 || K <= 0) return fail(QLS_EINVAL, "sizes must be positive");
  if (N % 16 || K % 16) return fail(QLS_EUNSUPPORTED, "N and K must be multiples of 16");
  const bool lora = A && B;
  if (lora && (r <= 0 || r % 8 || r > 128 || !u || !ws))
    return fail(QLS_EINVAL, "LoRA needs r in [8,128] (multiple of 8), u and ws");
  LinearFwd f{};
  f.T = T; f.N = N; f.K = K; f.r = lora ? r : 0;
  f.x = x; f.codes = codes; f.absmax = absmax;
  f.A = lora ? A : nullptr; f.nmod = 1; f.mod_end[0] = N; f.Bm[0] = lora ? B : nullptr;
  f.s = lora ? alpha / (float)r : 0.f;
  f.y = y; f.ldy = N; f.u = lora ? u : nullptr;
  f.ws = reinterpret_cast<float*>(ws);
  int rc = linear_fwd(f, (hipStream_t)stream);
  if (rc) return fail(QLS_EHIP, "kernel combination not built");
  QLS_HIP(hipGetLastError());
  return QLS_OK;
}

int64_t qls_attention_ws_bytes(int B, int S, int H, int hd) {
  if (B <= 0 || S <= 0 || H <= 0 || hd <= 0) return fail(QLS_EINVAL, "sizes must be positive");
  const int64_t T = (int64_t)B * S;
  return align_up((int64_t)B * H * S * 4, 256) + 2 * align_up(T * H * hd * 4, 256);
}

static int attn_check(int B, int S, int H, int KV, int hd) {
  if (B <= 0 || S <= 0 || H <= 0 || KV <= 0) return fail(QLS_EINVAL, "sizes must be positive");
  if (hd != 64 && hd != 128) return fail(QLS_EUNSUPPORTED, "head_dim must be 64 or 128");
  if (H % KV || H / KV > 8) return fail(QLS_EUNSUPPORTED, "n_heads must be a multiple of n_kv_heads, at most 8 times it");
  return QLS_OK;
}

// True when every pointer is 16-byte aligned (the kernels load 8 bf16 at a time).
static bool aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (reinterpret_cast<uintptr_t>(p) % 16) return false;
  return true;
}

int qls_attention_fwd(const uint16_t* qkv, int B, int S, int H, int KV, int hd, uint16_t* out, float* lse,
                      void* stream) {
  if (!qkv || !out || !lse) return fail(QLS_EINVAL, "NULL buffer");
  if (!aligned16({qkv, out, lse})) return fail(QLS_EINVAL, "attention buffers must be 16-byte aligned");
  int rc = attn_check(B, S, H, KV, hd);
  if (rc) return rc;
  AttnArgs a{};
  a.qkv = qkv; a.ld = (int64_t)(H + 2 * KV) * hd; a.q_off = 0; a.k_off = H * hd; a.v_off = (H + KV) * hd;
  a.S = S; a.H = H; a.KV = KV; a.hd = hd; a.scale = 1.f / std::sqrt((float)hd);
  a.out = out; a.ldo = (int64_t)H * hd; a.lse = lse;
  if (attn_fwd(a, B, (hipStream_t)stream)) return fail(QLS_EUNSUPPORTED, "attention shape not supported");
  QLS_HIP(hipGetLastError());
  return QLS_OK;
}

int qls_attention_bwd(const uint16_t* qkv, const uint16_t* out, const uint16_t* dout, const float* lse, int B,
                      int S, int H, int KV, int hd, float* dq, float* dk, float* dv, void* ws, void* stream) {
  return attention_bwd_run(qkv, out, dout, lse, B, S, H, KV, hd, dq, dk, dv, ws, -1, (hipStream_t)stream);
}

}  // extern "C"

// Attention backward over caller scratch ws (ws_cap >= 0: its size in bytes,
// checked; -1: the caller sized it with qls_attention_ws_bytes).
int attention_bwd_run(const uint16_t* qkv, const uint16_t* out, const uint16_t* dout, const float* lse, int B,
                      int S, int H, int KV, int hd, float* dq, float* dk, float* dv, void* ws, int64_t ws_cap,
                      hipStream_t st) {
  if (!qkv || !out || !dout || !lse || !dq || !dk || !dv || !ws) return fail(QLS_EINVAL, "NULL buffer");
  if (!aligned16({qkv, out, dout, lse, dq, dk, dv, ws}))
    return fail(QLS_EINVAL, "attention buffers must be 16-byte aligned");
  int rc = attn_check(B, S, H, KV, hd);
  if (rc) return rc;
  if (ws_cap >= 0 && qls_attention_ws_bytes(B, S, H, hd) > ws_cap)
    return fail(QLS_EINVAL, "attention scratch of " + std::to_string(qls_attention_ws_bytes(B, S, H, hd)) +
                                " bytes exceeds the " + std::to_string(ws_cap) + " available");

  const int64_t T = (int64_t)B * S;
  char* w = reinterpret_cast<char*>(ws);
  float* D = reinterpret_cast<float*>(w);
  float* pk = reinterpret_cast<float*>(w + align_up((int64_t)B * H * S * 4, 256));
  float* pv = reinterpret_cast<float*>(w + align_up((int64_t)B * H * S * 4, 256) + align_up(T * H * hd * 4, 256));
  AttnBwdArgs a{};
  a.qkv = qkv; a.ld = (int64_t)(H + 2 * KV) * hd; a.q_off = 0; a.k_off = H * hd; a.v_off = (H + KV) * hd;
  a.S = S; a.H = H; a.KV = KV; a.hd = hd; a.scale = 1.f / std::sqrt((float)hd);
  a.dO = dout; a.O = out; a.lddo = (int64_t)H * hd; a.lse = lse; a.D = D;
  a.dq = dq; a.lddq = (int64_t)H * hd; a.dk = pk; a.dv = pv; a.lddkv = (int64_t)H * hd;
  if (attn_bwd(a, B, st)) return fail(QLS_EUNSUPPORTED, "attention shape not supported");
  attn_group_sum(pk, dk, (int)T, H, KV, hd, st);
  attn_group_sum(pv, dv, (int)T, H, KV, hd, st);
  QLS_HIP(hipGetLastError());
  return QLS_OK;
}

extern "C" {

int qls_linear_bwd(const uint8_t* codes, const float* absmax, int N, int K, const uint16_t* x,
                   const uint16_t* u, const uint16_t* dy, int T, const uint16_t* A,
                   const uint16_t* B, int r, float alpha, float* dx, float* dA, float* dB, void* ws,
                   void* stream) {
  if (!codes || !absmax || !x || !u || !dy || !A || !B || !dx || !dA || !dB || !ws)
    return fail(QLS_EINVAL, "NULL buffer");
  if (T <= 0 || N <= 0 || K <= 0) return fail(QLS_EINVAL, "sizes must be positive");
  if (N % 16 || K % 16) return fail(QLS_EUNSUPPORTED, "N and K must be multiples of 16");
  if (r <= 0 || r % 8 || r > 128) return fail(QLS_EUNSUPPORTED, "r must be a multiple of 8 in [8,128]");
  hipStream_t st = (hipStream_t)stream;
  const float s = alpha / (float)r;
  uint16_t* du = reinterpret_cast<uint16_t*>(ws);
  float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + align_up((int64_t)T * r * 2, 256));
  int rc = 0;
  rc |= skinny_du(dy, N, T, N, B, r, s, du, r, part, st);
  rc |= skinny_dB(dy, N, T, N, u, r, s, dB, part, st);
  rc |= skinny_dA(du, r, T, r, x, K, K, dA, part, st);
  LinearDx d{};
  d.T = T; d.Kc = N; d.Nout = K;
  d.dy = dy; d.lddy = N; d.codes = codes; d.absmax = absmax; d.ldq = K;
  d.du = du; d.lddu = r; d.Acat = A; d.rc = r;
  d.out = dx; d.ldo = K; d.epi = EPI_F32; d.ws = part;
  rc |= linear_dx(d, st);
  if (rc) return fail(QLS_EHIP, "kernel combination not built");
  QLS_HIP(hipGetLastError());
  return QLS_OK;
}

}  // extern "C"
