// Host-side launch helpers built on the GEMM family and the layer kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// ---------------------------------------------------------------- QLoRA linear
// Y = bf16( X W^T + s U_g B_g^T (+ res) ), U = bf16( X A_cat^T ), where the N
// output columns are split into nmod modules (cumulative ends mod_end[]), each
// with its own LoRA B_g [N_g, r]; A_cat [nmod*r, K] stacks the modules' A.
struct LinearFwd {
  int T, N, K, r;
  const uint16_t* x; int64_t ldx;
  const uint8_t* codes; const float* absmax;
  const uint16_t* A;            // nullptr: adapters disabled
  int nmod; int mod_end[4]; const uint16_t* Bm[4];
  float s;
  const uint16_t* res; int64_t ldres;
  uint16_t* y; int64_t ldy;
  uint16_t* u;                  // U_cat [T, nmod*r]
  float* ws;                    // split-K partials
  hipEvent_t ev0, ev1;          // optional: recorded around the dequant-GEMM kernel
  hipEvent_t ev2;               // optional: recorded after its split-K reduce (only if split)
  int tile;                     // out: 256 or 128, the output tile of the kernel taken
  int ksplit;                   // out: contraction slices of that kernel (1: no reduce)
};
int linear_fwd(LinearFwd& f, hipStream_t st);

// out = dY W + du_cat A_cat, contraction over W's Kc rows (dY [T, Kc]) and the
// rc concatenated LoRA ranks; W NF4 with Nout columns.
struct LinearDx {
  int T, Kc, Nout;
  const uint16_t* dy; int64_t lddy;
  const uint8_t* codes; const float* absmax; int64_t ldq;
  const uint16_t* du; int64_t lddu; const uint16_t* Acat; int rc;   // Acat [rc, Nout]
  void* out; int64_t ldo; int epi;    // EPI_F32 / EPI_BF16 / EPI_SWIGLU_BWD
  const uint16_t* gu; int64_t ldgu; int I;
  float* ws;                    // split-K partials (nullptr: no split)
  hipEvent_t ev0, ev1;          // optional: recorded around the dequant-GEMM kernel
  hipEvent_t ev2;               // optional: recorded after its split-K reduce (only if split)
  int tile;                     // out: 256 or 128, the output tile of the kernel taken
  int ksplit;                   // out: contraction slices of that kernel (1: no reduce)
};
int linear_dx(LinearDx& d, hipStream_t st);
// Split-K factor for a 128 x 128-tiled GEMM of M x N x K (partials fit in
// skinny_partial_floats()).
int big_split(int M, int N, int K);
// Kernel choice for an M x N x K dequant-GEMM: the 256 x 256 kernels (big)
// with ksplit contraction slices, or the 128 x 128 ones.
struct GemmPlan { bool big; int ksplit; };
GemmPlan plan_nf4(int M, int N, int K, bool can_split);

// Skinny LoRA products (split-K over the long dimension, deterministic reduce).
// U = bf16(x A^T)                   x [T, K] (ldx), A [n, K]          -> U [T, n] (ldu)
int skinny_U(const uint16_t* x, int64_t ldx, int T, int K, const uint16_t* A, int n, uint16_t* U,
             int64_t ldu, float* part, hipStream_t st);
// du = bf16(s dY B)                 dY [T, N] (lddy), B [N, r]        -> du [T, r] (lddu)
int skinny_du(const uint16_t* dy, int64_t lddy, int T, int N, const uint16_t* B, int r, float s,
              uint16_t* du, int64_t lddu, float* part, hipStream_t st);
// dB = s dY^T u  (float32)          dY [T, N], u [T, r] (ldu)         -> dB [N, r]
int skinny_dB(const uint16_t* dy, int64_t lddy, int T, int N, const uint16_t* u, int64_t ldu,
              float s, float* dB, float* part, hipStream_t st, int r = -1);
// dA = du^T x    (float32)          du [T, r] (lddu), x [T, K] (ldx)  -> dA [r, K]
int skinny_dA(const uint16_t* du, int64_t lddu, int T, int r, const uint16_t* x, int64_t ldx,
              int K, float* dA, float* part, hipStream_t st);
// dA_i = du_i^T x for nmod (<= 4) modules sharing x, as one product:
// du = [du_0 | du_1 | ...] [T, nmod r] (lddu), x [T, K] (ldx) -> dA[i] [r, K].
// Always goes through float partials (nmod r x K per slice) in part, which
// holds part_floats floats; -1 when they would not fit.
int skinny_dA_multi(const uint16_t* du, int64_t lddu, int T, int r, int nmod, const uint16_t* x, int64_t ldx,
                    int K, float* const* dA, float* part, int64_t part_floats, hipStream_t st);
// Several skinny products in as few launches as their loaders allow: one
// grouped GEMM launch per loader combination (A_ROW / B_BF16_NN: du-like,
// A_COL / B_BF16_NN: dA- and dB-like, A_ROW / B_BF16_NT: U-like), then one
// launch that sums every product's split-K partials in split order (the same
// arithmetic as the one-product calls).  C: bf16 (mode 0) or float (mode 1)
// alpha * product, or with rows > 0 row block i of the float product to
// Crows[i] (ldc).  Partials are laid out back to back in part (part_floats
// floats); -1 when they do not fit or more than kMaxGroup products are given.
struct SkinnyProd {
  int aload, bload;
  const uint16_t* A; int64_t lda;
  const uint16_t* B; int64_t ldb;
  int M, N, K;
  float alpha; int mode;
  void* C; int64_t ldc;
  int rows; float* Crows[4];
};
int skinny_group(const SkinnyProd* p, int n, float* part, int64_t part_floats, hipStream_t st);
// Floats of partials skinny_group lays out for these products.
int64_t skinny_group_floats(const SkinnyProd* p, int n);
// The product descriptions of the one-product calls above.
SkinnyProd sk_du(const uint16_t* dy, int64_t lddy, int T, int N, const uint16_t* B, int r, float s, uint16_t* du,
                 int64_t lddu);
SkinnyProd sk_dB(const uint16_t* dy, int64_t lddy, int T, int N, const uint16_t* u, int64_t ldu, float s, float* dB,
                 int r);
SkinnyProd sk_dA_multi(const uint16_t* du, int64_t lddu, int T, int r, int nmod, const uint16_t* x, int64_t ldx,
                       int K, float* const* dA);
// Largest split-K partial buffer (floats) any skinny product of these sizes needs.
int64_t skinny_partial_floats(int64_t max_mn);

int64_t linear_ws_bytes(int T, int N, int K, int r);

// ---------------------------------------------------------------- layer kernels (elem.hip)
void rmsnorm_fwd(const uint16_t* x, const uint16_t* w, float eps, uint16_t* y, int T, int d,
                 hipStream_t st);
// out = gres + dRMSNorm(x, w; dy); optional bf16 copy of out.  Needs d % 8 ==
// 0, d <= 8192 and 16-byte aligned pointers; -1 (nothing launched) otherwise.
int rmsnorm_bwd(const uint16_t* x, const uint16_t* w, float eps, const float* dy, const float* gres,
                float* out, uint16_t* out_bf16, int T, int d, hipStream_t st);
// In-place rotate-half RoPE on the q and k column blocks of qkv [T, ld].
// Needs hd % 8 == 0, ld % 4 == 0, qkv 8-byte and cs 16-byte aligned; -1
// (nothing launched) otherwise.
int rope_fwd(uint16_t* qkv, int64_t ld, int T, int S, int H, int KV, int hd, const float* cs,
             hipStream_t st);
// dq = bf16(R^-1 dq'), dk = bf16(R^-1 dk'), dv = bf16(dv) into dqkv [T, ld] (q | k | v).
// dq [T, H*hd]; dk and dv [T, H*hd] hold per-query-head partials that are
// summed over each kv head's group in head order.  Alignment as rope_fwd,
// dq / dk / dv 16-byte aligned; -1 (nothing launched) otherwise.
int rope_bwd(const float* dq, const float* dk, const float* dv, uint16_t* dqkv, int64_t ld, int T,
             int S, int H, int KV, int hd, const float* cs, hipStream_t st);
void swiglu_fwd(const uint16_t* gu, uint16_t* a, int T, int I, hipStream_t st);
// x[t] = E[ids[t]]; ids outside [0, V) give a zero row and set *bad (device int) to 1.
void embed_gather(const int32_t* ids, const uint16_t* E, uint16_t* x, int T, int d, int V, int* bad,
                  hipStream_t st);
void f32_to_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t st);
void bf16_to_f32(const uint16_t* x, float* y, int64_t n, hipStream_t st);
// Copy-cast segments of the packed float32 LoRA vector into the bf16 working
// copy: for each layer l and segment j, n[j] elements from src + l*ss + so[j]
// to dst + l*ds + dof[j].
struct CastSeg { int64_t so[14], dof[14], n[14]; int nseg; };
void lora_cast(const float* src, int64_t ss, uint16_t* dst, int64_t ds, int L, const CastSeg& seg,
               hipStream_t st);
// Cross-entropy helpers.
void ce_finalize(const float* stats, int ntiles, const float* tgt_logit, const int32_t* tgt, int T,
                 float* lse, float* logp, hipStream_t st);
void ce_targets(const int32_t* ids, int B, int S, int32_t* tgt, hipStream_t st);
// w_t = 1/N where row t has a target, else 0; loss = -sum_t w_t logp_t.
void sft_weights_loss(const float* logp, const int32_t* tgt, int T, int N, float* w, float* loss,
                      hipStream_t st);
void seq_logp(const float* logp, int B, int S, int prompt_len, float* seq, float* tok, hipStream_t st);
// Preference heads (the qls_pref_kind values).
enum PrefKind { PREF_DPO = 0, PREF_SIMPO = 1, PREF_ORPO = 2, PREF_KTO = 3 };
struct PrefArgs { int kind; float beta, gamma, lam, lam_d, lam_u; };
// Loss of head a on the pair's response log-likelihoods (logp_ref NULL for
// the reference-free heads), row weights w [2S] = -dL/dpi per response row,
// aux (optional) [4] = pi_c, pi_r, rho_c, rho_r.
void pref_loss(const PrefArgs& a, const float* logp_pol, const float* logp_ref, int S, int prompt_len,
               float* w, float* loss, float* aux, hipStream_t st);
// AdamW update of n float32 parameters at step t (1-based), in place.
void adamw_update(float* p, const float* g, float* m, float* v, int64_t n, int t, double lr, double b1,
                  double b2, double eps, double wd, hipStream_t st);
// Bounded spin of `ticks` wall-clock ticks (test hook).
void spin_delay(int64_t ticks, hipStream_t st);
