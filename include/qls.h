/*
 * qls.h -- C ABI of the layer-streamed QLoRA step for AMD Instinct MI355X (gfx950).
 *
 * One LoRA fine-tuning step in which the frozen NF4-quantised decoder stack
 * lives in pinned host memory and streams into a two-slot device pool one
 * layer at a time, prefetched one layer ahead.  Each resident layer runs the
 * forward pass; the backward sweep reloads the layers, recomputes each
 * forward from its checkpointed input and back-propagates to the LoRA A/B
 * matrices only.
 *
 * Sources (web pages on the "layer streaming" feature of the Soup fine-tuning
 * tool; cited by title and section):
 *   [P1] "Can You Fine-Tune Llama 3.1 8B on a 4GB GPU? Soup's Layer Streaming
 *        Explained": "How Soup's layer streaming actually works" (frozen base
 *        off the GPU, page-locked host memory, reusable device buffers,
 *        prefetch of the next layer, layers read again for the recomputed
 *        backward); "Why NF4 matters so much" (NF4 host store, asynchronous
 *        copies need page-locked memory); "Did a correctness bug invalidate the
 *        Llama 3.1 8B result?" (size-dependent silent wrong gradients).
 *   [P2] "Fine tune an 8B model on a 4GB laptop GPU (Soup setup)": "The
 *        number, and exactly what it means" (embeddings and LM head stay
 *        resident; streamed run bit-exact against the resident run); "Step 2,
 *        train" (32 layers, two device buffers, base store pinned in RAM).
 *   [P4] "Soup ... fine-tune 8B on a 4 GB laptop GPU" radar note: "In detail"
 *        (DPO reference = the same base stream with the adapters disabled).
 *   [P5] "How Layer Streaming Enables Fine-Tuning an 8B Model on a 4 GB GPU":
 *        "Runtime Execution Flow" (per-layer load / release, runtime stats).
 *
 * Conventions
 *   - Every function returns QLS_OK (0) or a negative QLS_E* code; the
 *     thread-local text of the last failure is returned by qls_last_error().
 *   - "d_" pointers are device pointers (HIP), "h_" pointers host pointers.
 *     Device buffers are borrowed: the caller (normally PyTorch) owns them and
 *     must keep them alive while work that uses them is in flight.
 *   - Streams are hipStream_t passed as void*.  Entry points taking a session
 *     enqueue asynchronously on the session's compute stream and return before
 *     the GPU finishes, unless a host output (h_*) is requested.
 *   - bf16 tensors are passed as uint16_t (raw bfloat16 bits), row-major.
 *   - A session is used by one host thread at a time.
 */
#ifndef QLS_H
#define QLS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QLS_ABI_VERSION 3

enum {
  QLS_OK = 0,
  QLS_EINVAL = -1,       /* bad argument or shape */
  QLS_ENOMEM = -2,       /* host allocation failed or workspace too small */
  QLS_ENOPIN = -3,       /* pinned host allocation failed or exceeds the cap */
  QLS_EHIP = -4,         /* a HIP runtime call failed (message has hipGetErrorString) */
  QLS_ESTATE = -5,       /* object not ready (e.g. a store layer never set) */
  QLS_EUNSUPPORTED = -6, /* shape outside what the kernels support */
  QLS_EIO = -7           /* disk-tier file create / read / write failed */
};

enum { QLS_STREAMED = 0, QLS_RESIDENT = 1 };

/* Absmax format of a store (see qls_store_create_fmt). */
enum { QLS_ABSMAX_F32 = 0, QLS_ABSMAX_DQ8 = 1 };

/* Module order used everywhere (records, LoRA packing): */
enum { QLS_Q = 0, QLS_K, QLS_V, QLS_O, QLS_GATE, QLS_UP, QLS_DOWN, QLS_NMOD };

/* Llama-style decoder shape plus LoRA hyper-parameters.
 * Linears as (out x in): q (H*hd x d), k and v (KV*hd x d), o (d x H*hd),
 * gate and up (I x d), down (d x I).  LoRA scale s = alpha / r.
 * Supported: head_dim in {64, 128}; n_heads % n_kv_heads == 0 with at most 8
 * query heads per kv head; hidden at most 8192; hidden, intermediate and
 * every linear's in/out multiples of 16; lora_r a multiple of 8 in [8, 128];
 * vocab a multiple of 8. */
typedef struct qls_model_cfg {
  int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, intermediate, vocab;
  float rms_eps, rope_theta;
  int32_t lora_r;
  float lora_alpha;
} qls_model_cfg;

/* Per-session run configuration.
 *   mode        QLS_STREAMED: two device slots, layers copied host->device
 *               on a copy stream one layer ahead, each copy after the slot's
 *               previous layer has released it (the first copy of a sweep
 *               part by part, each code blob after its last reader);
 *               QLS_RESIDENT: the whole store is copied to the device once
 *               at session creation.
 *   max_tokens  upper bound on B*S of any call (DPO uses 2*S).
 *   max_seq     upper bound on S.
 *   ce_chunk    vocabulary columns per cross-entropy chunk (0 = 32768;
 *               rounded up to a multiple of 128).
 *   timing      non-zero: record hipEvents around every copy and layer so
 *               qls_session_stats can report copy / compute / overlap time. */
typedef struct qls_run_cfg {
  int32_t mode;
  int32_t max_tokens;
  int32_t max_seq;
  int32_t ce_chunk;
  int32_t timing;
} qls_run_cfg;

/* Resident (never streamed) tensors, bf16, device pointers, borrowed:
 * embedding [vocab x hidden], LM head [vocab x hidden], final norm [hidden]. */
typedef struct qls_resident {
  const uint16_t* d_embed;
  const uint16_t* d_lm_head;
  const uint16_t* d_final_norm;
} qls_resident;

/* Read-only view of one layer record in the pinned host store.
 * codes[m]: NF4 codes of module m, numel/2 bytes, element 2k in the high
 * nibble of byte k; norms: bf16 [hidden].  QLS_ABSMAX_F32 stores: absmax[m]
 * numel/64 float32 (absmax_q8 / absmax_scale NULL).  QLS_ABSMAX_DQ8 stores:
 * absmax_q8[m] numel/64 uint8 and absmax_scale[m] ceil(numel/64/256) float32
 * (absmax NULL). */
typedef struct qls_layer_view {
  const uint8_t* codes[QLS_NMOD];
  const float* absmax[QLS_NMOD];
  const uint16_t* norm_attn;
  const uint16_t* norm_mlp;
  const void* record;
  int64_t record_bytes;
  int32_t absmax_format;
  const uint8_t* absmax_q8[QLS_NMOD];
  const float* absmax_scale[QLS_NMOD];
} qls_layer_view;

typedef struct qls_stats {
  int64_t steps;          /* step-like calls since the last reset */
  int64_t layer_loads;    /* host->device layer copies issued */
  int64_t h2d_bytes;      /* bytes of those copies */
  double copy_ms;         /* sum of copy durations (timing on) */
  double compute_ms;      /* sum of per-layer compute spans (timing on) */
  double overlap_ms;      /* copy time overlapped by layer compute (timing on) */
  double step_ms;         /* wall time of the last step on the GPU (timing on) */
  int64_t ws_bytes;       /* workspace bytes the session uses */
  /* Dequant-GEMM launches of the steps since the last reset (timing on):
   * forward Y = X W^T (+ LoRA) and transposed dX = dY W (+ LoRA), each with
   * the summed duration of the GEMM kernel itself (hipEvents on the compute
   * stream around that launch; a split-K reduce that follows it is not
   * included) and the summed algorithmic work 2*T*N*K (+ 2*T*N*r for the LoRA
   * term) in GFLOP. */
  double dq_fwd_ms, dq_fwd_gflop;
  int64_t dq_fwd_launches;
  double dq_dx_ms, dq_dx_gflop;
  int64_t dq_dx_launches;
  /* The part of the above taken by the 256 x 256-tile kernels (the rest ran
   * the 128 x 128-tile kernels), and the summed duration of the split-K
   * reduce kernels that followed any of the launches (timing on). */
  double dq_fwd_big_ms, dq_fwd_big_gflop;
  int64_t dq_fwd_big_launches;
  double dq_dx_big_ms, dq_dx_big_gflop;
  int64_t dq_dx_big_launches;
  double dq_fwd_reduce_ms, dq_dx_reduce_ms;
  /* Disk tier (streamed sessions over a tiered store): records read from the
   * file (read-aheads included), their bytes, the summed read time on the
   * reader thread and the time the step's host thread waited for a record. */
  int64_t disk_reads, disk_bytes;
  double disk_read_ms, disk_wait_ms;
  /* Copy time not covered by any layer's compute span (copy_ms - overlap_ms;
   * timing on): the part of the layer stream that sits on the step's
   * critical path ([P1] "How Soup's layer streaming actually works").  */
  double exposed_copy_ms;
  /* Largest workspace any call since the last reset needed: the
   * qls_workspace_bytes of this session's run configuration with max_tokens
   * and max_seq set to that call's token count and sequence length (ws_bytes
   * is the size for the configured maxima). */
  int64_t peak_ws_bytes;
  /* The part of dq_fwd_reduce_ms / dq_dx_reduce_ms that followed the
   * 256 x 256-tile launches (timing on). */
  double dq_fwd_big_reduce_ms, dq_dx_big_reduce_ms;
} qls_stats;

typedef struct qls_store qls_store;
typedef struct qls_session qls_session;

/* ---------------------------------------------------------------- basics */
int qls_abi_version(void);
/* Message for the last non-zero return on this thread; valid until the next
 * qls_* call on the same thread. */
const char* qls_last_error(void);

/* ---------------------------------------------------------------- NF4
 * [P1] "Why NF4 matters so much": the frozen store is NF4, about a quarter of
 * bf16.  Levels: QLoRA's NormalFloat construction (7 negative quantiles of
 * N(0,1), 8 positive, an exact 0, scaled so the ends are -1 and +1), float32,
 * ascending.  Blocks of 64 consecutive elements of the row-major flattened
 * tensor share one float32 absmax. */
int qls_nf4_codebook(float out[16]);

/* Host quantiser.  w: n float32 (n % 64 == 0).  codes: n/2 bytes (element 2k
 * high nibble); absmax: n/64 float32.  code = argmin_j |w/a - cb[j]| taken in
 * float32, ties to the lower index; an all-zero block gets code 7 and absmax
 * 0.  n_threads <= 0 uses all hardware threads.  Errors: QLS_EINVAL. */
int qls_nf4_quantize(const float* h_w, int64_t n, uint8_t* h_codes, float* h_absmax,
                     int n_threads);

/* Device dequantiser: d_out[i] = bf16_rne(float32(cb[code_i] * absmax[i/64])).
 * Bit-exact reference of the in-GEMM dequantisation.  Asynchronous on stream. */
int qls_nf4_dequant_dev(const uint8_t* d_codes, const float* d_absmax, int64_t n,
                        uint16_t* d_out, void* stream);

/* Double quantisation of an absmax array ([P2] "Step 2, train": a 3.60 GB
 * pinned store for 32 layers and 113 MB device buffers, i.e. NF4 codes plus
 * 8-bit absmax; the format is this library's reading).  Per group of 256
 * consecutive entries (the last may be shorter): s = float32(max / 255),
 * q = clamp(rint(float32(a / s)), 0, 255) with ties to even, s = 0 gives q = 0.
 * h_q8: nblocks bytes; h_scales: ceil(nblocks / 256) float32.  Host only. */
int qls_nf4_double_quant(const float* h_absmax, int64_t nblocks, uint8_t* h_q8, float* h_scales);
/* Device decode: d_out[i] = float32(float32(q8[i]) * scales[i / 256]), the
 * absmax the kernels use for a QLS_ABSMAX_DQ8 store.  Asynchronous on stream. */
int qls_nf4_absmax_expand_dev(const uint8_t* d_q8, const float* d_scales, int64_t nblocks,
                              float* d_out, void* stream);

/* ---------------------------------------------------------------- one QLoRA linear
 * y = bf16( x W^T + s * u B^T ),  u = bf16( x A^T ),  s = alpha / r,
 * with W the dequantised NF4 weight [N x K].  x bf16 [T x K]; A bf16 [r x K];
 * B bf16 [N x r]; outputs y bf16 [T x N] and u bf16 [T x r].  d_A/d_B NULL
 * runs the base product only (u untouched).  K, N multiples of 16; r multiple
 * of 8.  d_ws: scratch of qls_linear_ws_bytes(T, N, K, r) bytes; required with
 * adapters, optional without (NULL: the base GEMM runs without split-K, so its
 * fp32 sums may round differently from a run with the workspace). */
int64_t qls_linear_ws_bytes(int T, int N, int K, int r);
int qls_linear_fwd(const uint8_t* d_codes, const float* d_absmax, int N, int K,
                   const uint16_t* d_x, int T, const uint16_t* d_A, const uint16_t* d_B,
                   int r, float alpha, uint16_t* d_y, uint16_t* d_u, void* d_ws,
                   void* stream);
/* Backward of the same linear for upstream dY bf16 [T x N]:
 *   du = bf16(s dY B);  dA = du^T x  [r x K] fp32;  dB = s dY^T u [N x r] fp32;
 *   dX = dY W + du A    [T x K] fp32. */
int qls_linear_bwd(const uint8_t* d_codes, const float* d_absmax, int N, int K,
                   const uint16_t* d_x, const uint16_t* d_u, const uint16_t* d_dy, int T,
                   const uint16_t* d_A, const uint16_t* d_B, int r, float alpha,
                   float* d_dx, float* d_dA, float* d_dB, void* d_ws, void* stream);

/* Causal grouped-query attention of one decoder layer on its own (the
 * attention inside qls_sft_step; [P2] "The number, and exactly what it means"
 * fixes the Llama-3.1-8B attention shape).  qkv bf16 [B*S x (H + 2 KV) hd]:
 * per token the H query heads, then the KV key heads, then the KV value heads,
 * hd each; query head h reads kv head h / (H / KV); scores q k^T / sqrt(hd)
 * over keys j <= i of the same sequence.  Forward: out bf16 [B*S x H hd],
 * lse float32 [B x H x S] (natural log-sum-exp of each score row).  Backward
 * from dout bf16 [B*S x H hd] (out and lse from the forward): dq float32
 * [B*S x H hd], dk and dv float32 [B*S x KV hd], each the sum over the query
 * heads of its kv head, in head order.  d_ws: qls_attention_ws_bytes(B, S, H,
 * hd) bytes of scratch.  hd in {64, 128}, H a multiple of KV and at most 8 KV;
 * QLS_EUNSUPPORTED otherwise, QLS_EINVAL for NULL buffers, buffers not
 * 16-byte aligned or sizes <= 0.
 * Asynchronous on `stream`. */
int64_t qls_attention_ws_bytes(int B, int S, int H, int hd);
int qls_attention_fwd(const uint16_t* d_qkv, int B, int S, int H, int KV, int hd, uint16_t* d_out,
                      float* d_lse, void* stream);
int qls_attention_bwd(const uint16_t* d_qkv, const uint16_t* d_out, const uint16_t* d_dout,
                      const float* d_lse, int B, int S, int H, int KV, int hd, float* d_dq,
                      float* d_dk, float* d_dv, void* d_ws, void* stream);

/* Attention backward that allocates nothing: for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Arguments, layouts, results and errors
 * as qls_attention_bwd, without d_ws: the scratch (qls_attention_ws_bytes(B,
 * S, H, hd) bytes) lives in a fixed device array of the library,
 * QLS_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends (at the 8B
 * shape, H = 32 and hd = 128, up to 1275 tokens).  A larger problem is
 * refused with QLS_EINVAL before any launch.  All calls on one GPU share its
 * array, so calls that overlap on one GPU (on different streams, or from
 * different threads) race; calls ordered on one stream do not.  Calls no
 * allocating routine. */
#define QLS_NOALLOC_SCRATCH_BYTES (40 * 1024 * 1024)
int qls_attention_bwd_noalloc(const uint16_t* d_qkv, const uint16_t* d_out, const uint16_t* d_dout,
                              const float* d_lse, int B, int S, int H, int KV, int hd, float* d_dq,
                              float* d_dk, float* d_dv, void* stream);

/* ---------------------------------------------------------------- optimizer
 * AdamW (decoupled weight decay) on n float32 parameters, in place, at step
 * `step` (1-based): the training loop around qls_sft_step / qls_dpo_step.  The
 * pages train at lr 2e-5 ([P2] "Step 1, the config") and compare 20 streamed
 * with 20 resident steps ([P3] "The gotchas nobody's mentioning yet"); they
 * name no optimizer.  With b1 = beta1, b2 = beta2, float32 arithmetic, each
 * operation rounded on its own:
 *   p <- p * (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2;
 *   p <- p - (lr / (1 - b1^step)) * m / (sqrt(v) / sqrt(1 - b2^step) + eps)
 * with every constant (1 - lr wd, b1, 1 - b1, b2, 1 - b2, lr / (1 - b1^step),
 * 1 / sqrt(1 - b2^step), eps) formed in double on the host from the double
 * hyper-parameters and rounded once to float32.  m and
 * v start at zero (caller-owned, same length as the parameters).  Errors:
 * QLS_EINVAL (NULL, n < 0, step < 1, betas outside [0, 1), eps <= 0).
 * Asynchronous on stream. */
int qls_adamw_step(float* d_params, const float* d_grads, float* d_m, float* d_v, int64_t n, int step,
                   double lr, double beta1, double beta2, double eps, double weight_decay, void* stream);

/* ---------------------------------------------------------------- sizes */
/* Bytes of one layer record: the 7 code blobs, the absmax data (QLS_ABSMAX_F32:
 * 7 float32 arrays; QLS_ABSMAX_DQ8: 7 uint8 arrays then 7 float32 scale
 * arrays), 2 bf16 norms, each region 256-byte aligned.  The _fmt form takes the
 * format; the plain form is QLS_ABSMAX_F32.  At the 8B shape: 122,699,776 B
 * (F32) and 112,529,408 B (DQ8). */
int64_t qls_layer_record_bytes(const qls_model_cfg* cfg);
int64_t qls_layer_record_bytes_fmt(const qls_model_cfg* cfg, int absmax_format);
/* Length of the packed LoRA vector: layer-major, modules q,k,v,o,gate,up,down,
 * each A [r x in] row-major then B [out x r] row-major. */
int64_t qls_lora_numel(const qls_model_cfg* cfg);

/* ---------------------------------------------------------------- host store
 * [P1] "How Soup's layer streaming actually works", item 2 and [P2] "Step 2,
 * train": the frozen decoder stack lives in page-locked host memory, one
 * record per layer.  Records are allocated with hipHostMalloc; if pinning
 * fails, or n_layers * record bytes exceeds max_pinned_bytes (0 = no cap),
 * creation fails with QLS_ENOPIN.  The store owns its host memory and must
 * outlive every session created over it. */
int qls_store_create(const qls_model_cfg* cfg, uint64_t max_pinned_bytes, qls_store** out);
/* Same, with the absmax format: QLS_ABSMAX_F32 (qls_store_create) or
 * QLS_ABSMAX_DQ8 (absmax double-quantised when a layer is set; the session
 * decodes it on the device when a record arrives, before the layer's first
 * kernel).  Errors as qls_store_create, plus QLS_EINVAL for an unknown format. */
int qls_store_create_fmt(const qls_model_cfg* cfg, int absmax_format, uint64_t max_pinned_bytes,
                         qls_store** out);
/* Quantise and pack one layer.  w[m]: float32 [out x in] of module m; norms
 * bf16 [hidden].  Inputs are borrowed for the call.  n_threads as for
 * qls_nf4_quantize.  Errors: QLS_EINVAL (layer out of range / NULL). */
int qls_store_set_layer_fp32(qls_store* st, int layer, const float* const h_w[QLS_NMOD],
                             const uint16_t* h_norm_attn, const uint16_t* h_norm_mlp,
                             int n_threads);
/* Pack a layer that is already quantised (codes / absmax as in qls_nf4_quantize;
 * a QLS_ABSMAX_DQ8 store double-quantises the absmax as it packs). */
int qls_store_set_layer_nf4(qls_store* st, int layer, const uint8_t* const h_codes[QLS_NMOD],
                            const float* const h_absmax[QLS_NMOD],
                            const uint16_t* h_norm_attn, const uint16_t* h_norm_mlp);
/* Read-only pointers into one record.  For a disk-tier layer the record is
 * first read into a store-owned host buffer: the pointers stay valid until
 * the next view of a disk-tier layer or the store's destruction.  Errors:
 * QLS_EINVAL, QLS_ESTATE (disk layer never set), QLS_EIO. */
int qls_store_layer_view(const qls_store* st, int layer, qls_layer_view* out);
void qls_store_destroy(qls_store* st);   /* NULL-safe; removes a disk tier's file */

/* Two-tier store ([P1] "How Soup's layer streaming actually works", item 2,
 * and its FAQ on an SSD instead of enough RAM: records that do not fit in
 * pinned host memory spill to an NVMe-backed file, which adds the storage
 * read rate as a further bound).  Layers [0, ram_layers) are pinned host
 * records as in qls_store_create_fmt; layers [ram_layers, n_layers) live in
 * the file `path` (created or truncated, owned by the store, deleted by
 * qls_store_destroy), one record per 4096-byte-aligned slot, written when the
 * layer is set.  A streamed session reads a disk layer with one buffered
 * sequential pread of the whole record into one of three pinned staging
 * buffers, then drops the record's pages from the page cache
 * (POSIX_FADV_DONTNEED) so that the next read comes from the device again; a
 * reader thread reads the next disk layer of the sweep ahead of its request,
 * and the copy to the device slot starts from the staging buffer.  A resident
 * session reads every disk layer once at creation.  Errors: QLS_EINVAL (format, ram_layers
 * outside [0, n_layers], no path with disk layers), QLS_ENOPIN, QLS_EIO. */
enum { QLS_TIER_PINNED = 0, QLS_TIER_DISK = 1 };
int qls_store_create_tiered(const qls_model_cfg* cfg, int absmax_format, int ram_layers,
                            const char* path, qls_store** out);
/* QLS_TIER_PINNED or QLS_TIER_DISK for one layer; QLS_EINVAL if out of range. */
int qls_store_layer_tier(const qls_store* st, int layer);

/* ---------------------------------------------------------------- session
 * Token ids: the embedding gather turns an id outside [0, vocab) into a zero
 * row and raises a per-session device flag, which stays raised until it is
 * reported: by the next step-like call given a host loss pointer (h_loss), or
 * by qls_session_stats, which return QLS_EINVAL and clear it (the step
 * itself has run, AdamW included, on the zero rows).
 *
 * Device bytes a session needs: the two slots (or the whole store when
 * RESIDENT), layer-input checkpoints, one layer's activations and gradients,
 * the bf16 LoRA working copy, the cross-entropy chunk and split-K scratch. */
int qls_workspace_bytes(const qls_store* st, const qls_run_cfg* run, int64_t* out);

/* Bind a store, a device workspace, two streams (compute and copy, both at
 * default priority) and the resident tensors.  Everything is borrowed and must
 * outlive the session; the session owns only its hipEvents.  d_ws and the
 * resident tensors must be 256-byte aligned (torch's allocations are).
 * RESIDENT mode copies the whole store to the workspace before returning.
 * Errors: QLS_ENOMEM (ws_bytes too small, checked before any launch),
 * QLS_ESTATE (a store layer never set), QLS_EINVAL, QLS_EHIP. */
int qls_session_create(const qls_store* st, const qls_run_cfg* run, void* d_ws, int64_t ws_bytes,
                       void* compute_stream, void* copy_stream, const qls_resident* res,
                       qls_session** out);
void qls_session_destroy(qls_session* s);  /* NULL-safe; synchronises its streams */

/* One streamed SFT step (page [P1] "How Soup's layer streaming actually
 * works"): forward sweep over the layers as they stream in, final RMSNorm and
 * vocabulary-chunked next-token cross-entropy against the resident LM head
 * (mean over B*(S-1) targets), then the backward sweep in reverse layer order
 * that recomputes each layer from its checkpoint.  d_ids int32 [B x S] in
 * [0, vocab); d_lora float32 packed (qls_lora_numel); d_grads float32, same
 * packing, overwritten with dL/dA, dL/dB; d_loss float32 [1].  h_loss non-NULL
 * blocks until the step is done and copies the loss there. */
int qls_sft_step(qls_session* s, const int32_t* d_ids, int B, int S, const float* d_lora,
                 float* d_grads, float* d_loss, float* h_loss);

/* qls_sft_step followed by qls_adamw_step(d_lora, d_grads, d_m, d_v, n, step,
 * ...) over the whole LoRA vector, with each layer's slice updated as soon as
 * that layer's backward has made its gradients final, so the optimizer runs
 * while the remaining layers stream.  d_lora is read (before any update of
 * this step) and updated in place; d_grads holds the step's gradients as in
 * qls_sft_step.  Results equal the two separate calls bit for bit.  Errors as
 * qls_sft_step and qls_adamw_step. */
int qls_sft_step_adamw(qls_session* s, const int32_t* d_ids, int B, int S, float* d_lora,
                       float* d_grads, float* d_m, float* d_v, int step, double lr, double beta1,
                       double beta2, double eps, double weight_decay, float* d_loss, float* h_loss);

/* Forward-only sweep returning per-sequence sums of next-token log-probs over
 * positions [prompt_len, S): d_seq_logp float32 [B]; d_tok_logp (optional)
 * float32 [B x S] with entry t = log p(ids_{t+1} | ids_{<=t}) (0 at t = S-1).
 * d_lora == NULL disables the adapters: the DPO reference pass of [P4]. */
int qls_logprobs(qls_session* s, const int32_t* d_ids, int B, int S, int prompt_len,
                 const float* d_lora, float* d_seq_logp, float* d_tok_logp);

/* One DPO step on a (chosen, rejected) pair of length S sharing a prompt of
 * prompt_len tokens.  The reference (adapters disabled, [P4]) is computed on
 * each resident layer inside the same forward sweep as the policy, so the
 * step streams the stack exactly as an SFT step does.  Loss = softplus(-z),
 * z = beta((pi_c - ref_c) - (pi_r - ref_r)), log-probs summed over the
 * response positions.  d_aux (optional) float32 [4] = pi_c, pi_r, ref_c, ref_r.
 * Same as qls_pref_step with kind QLS_PREF_DPO. */
int qls_dpo_step(qls_session* s, const int32_t* d_chosen, const int32_t* d_rejected, int S,
                 int prompt_len, float beta, const float* d_lora, float* d_grads,
                 float* d_loss, float* h_loss, float* d_aux);

/* Preference heads on a (chosen, rejected) pair, after the papers that
 * define them (the pages name the four methods as running on the layer stream
 * and give KTO the same adapters-disabled reference as DPO: page "Soup ...
 * radar note", section "In detail").  With pi_x the response log-likelihood
 * of sequence x, rho_x the same with the adapters disabled and n = S -
 * prompt_len response tokens:
 *   QLS_PREF_DPO    z = beta((pi_c - rho_c) - (pi_r - rho_r)), L = softplus(-z)
 *   QLS_PREF_SIMPO  z = beta pi_c / n - beta pi_r / n - gamma,  L = softplus(-z)
 *                   (reference-free)
 *   QLS_PREF_ORPO   l_x = pi_x / n, lo_x = l_x - log(1 - e^l_x),
 *                   L = -l_c + lambda softplus(lo_r - lo_c) (reference-free)
 *   QLS_PREF_KTO    r_x = pi_x - rho_x, z0 = max(0, (r_c + r_r) / 2) held
 *                   constant, chosen desirable and rejected undesirable:
 *                   L = (lambda_d (1 - sigmoid(beta (r_c - z0)))
 *                        + lambda_u (1 - sigmoid(beta (z0 - r_r)))) / 2
 * Unused fields are ignored; beta > 0 except for ORPO, the lambdas >= 0. */
enum qls_pref_kind { QLS_PREF_DPO = 0, QLS_PREF_SIMPO = 1, QLS_PREF_ORPO = 2, QLS_PREF_KTO = 3 };
typedef struct qls_pref_cfg {
  int32_t kind;     /* qls_pref_kind */
  float beta;       /* DPO, SimPO, KTO */
  float gamma;      /* SimPO target margin */
  float lambda;     /* ORPO odds-ratio weight */
  float lambda_d;   /* KTO desirable weight */
  float lambda_u;   /* KTO undesirable weight */
} qls_pref_cfg;

/* One preference step of head cfg->kind, otherwise as qls_dpo_step: heads
 * with a reference compute it on each resident layer inside the policy's
 * forward sweep; the reference-free heads skip it.  Either way the step
 * streams the stack exactly as an SFT step does.  d_aux (optional) float32
 * [4] = pi_c, pi_r, rho_c, rho_r (rho = 0 without a reference).  Errors:
 * QLS_EINVAL for an unknown kind, non-finite parameters, beta <= 0 where beta
 * is used, a negative weight, or the conditions of qls_dpo_step. */
int qls_pref_step(qls_session* s, const qls_pref_cfg* cfg, const int32_t* d_chosen,
                  const int32_t* d_rejected, int S, int prompt_len, const float* d_lora,
                  float* d_grads, float* d_loss, float* h_loss, float* d_aux);

/* One streamed decoder layer on its own: forward, recomputed forward and
 * backward of layer `layer` for input d_x bf16 [B*S x hidden] and upstream
 * gradient d_gout bf16 [B*S x hidden].  Writes d_out bf16 [B*S x hidden]
 * (layer output), d_gin float32 [B*S x hidden] (dL/dx) and that layer's
 * slice of d_grads (packed LoRA layout, other layers untouched). */
int qls_layer_fwd_bwd(qls_session* s, int layer, const uint16_t* d_x, const uint16_t* d_gout,
                      int B, int S, const float* d_lora, uint16_t* d_out, float* d_gin,
                      float* d_grads);

/* Device pointer to the layer-input checkpoints of the last step: bf16
 * [(n_layers + 1) x tokens x hidden] (entry n_layers = final hidden state). */
int qls_session_checkpoints(qls_session* s, const uint16_t** d_ptr, int64_t* tokens);

/* Synchronises the session and fills *out; then reports a raised token-id
 * flag (QLS_EINVAL, *out still filled). */
int qls_session_stats(qls_session* s, qls_stats* out);
int qls_session_reset_stats(qls_session* s);

/* Test hooks; they add operations and never switch kernels.
 *   QLS_DBG_POISON_ON_RELEASE  fill a slot with 0xFF bytes (NaN bf16/fp32) on
 *                              the copy stream right after it is released
 *   QLS_DBG_COPY_DELAY         a host callback sleeping delay_us on the copy
 *                              stream before each layer copy
 *   QLS_DBG_COMPUTE_DELAY      a bounded spin kernel of about delay_us on the
 *                              compute stream before each slot release and
 *                              after each release of a code part (q|k|v, o,
 *                              gate|up, down) of a slot
 *   QLS_DBG_NO_REUSE           reload every layer even when a slot still holds it
 *   QLS_DBG_STREAM_FENCE       the copy stream waits on a slot's release on the
 *                              device; by default the host waits for the
 *                              release before it enqueues the copy
 *   QLS_DBG_RECOMPUTE_ALL      the backward sweep recomputes every layer's
 *                              forward from its checkpoint, also at the two
 *                              ends of the sweep, where it otherwise reuses
 *                              the last layer's forward intermediates and
 *                              restores layer 0's saved ones */
enum {
  QLS_DBG_POISON_ON_RELEASE = 1u,
  QLS_DBG_COPY_DELAY = 2u,
  QLS_DBG_COMPUTE_DELAY = 4u,
  QLS_DBG_NO_REUSE = 8u,
  QLS_DBG_STREAM_FENCE = 16u,
  QLS_DBG_RECOMPUTE_ALL = 32u
};
int qls_debug_set(qls_session* s, uint32_t flags, int delay_us);

/* Test hook for checking gradients layer by layer on a real step ([P1] "The
 * gradient bug also reveals something important about AI benchmarks": a loss
 * can look right while the gradients are wrong).  While d_buf is non-NULL,
 * every backward sweep (qls_sft_step, qls_sft_step_adamw, qls_pref_step,
 * qls_dpo_step) copies the float32 residual gradient at each layer boundary
 * into d_buf, float32 [(n_layers + 1) x B*S x hidden]: entry l = dL/dx_l, the
 * gradient with respect to layer l's input checkpoint (entry n_layers: the
 * gradient the final norm and LM head hand to the last layer).  The copies
 * run on the compute stream; they add operations and never switch kernels.
 * A step fails with QLS_EINVAL before any launch when n_floats is smaller
 * than (n_layers + 1) * B*S * hidden.  d_buf NULL turns the hook off; the
 * buffer is borrowed. */
int qls_debug_capture_grads(qls_session* s, float* d_buf, int64_t n_floats);

#ifdef __cplusplus
}
#endif
#endif /* QLS_H */
