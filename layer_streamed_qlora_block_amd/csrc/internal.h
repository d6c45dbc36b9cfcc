// Host-side internals shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/qls.h"

static inline int64_t align_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }
static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- errors
void set_error(const std::string& msg);
int fail(int code, const std::string& msg);
int hip_fail(hipError_t e, const char* what);
#define QLS_HIP(call)                                        \
  do {                                                       \
    hipError_t e_ = (call);                                  \
    if (e_ != hipSuccess) return hip_fail(e_, #call);        \
  } while (0)

// ---------------------------------------------------------------- NF4
void nf4_codebook_host(float out[16]);
const float* nf4_codebook_dev();
int nf4_dequant_launch(const uint8_t* codes, const float* absmax, int64_t n, uint16_t* out,
                       hipStream_t st);
void nf4_quantize_host(const float* w, int64_t n, uint8_t* codes, float* absmax, int n_threads);

// ---------------------------------------------------------------- model shape
struct ModuleShape { int out, in; };
struct Shape {
  qls_model_cfg c;
  ModuleShape mod[QLS_NMOD];
  int64_t numel[QLS_NMOD];
  int qd, kvd;       // H*hd, KV*hd
  int nqkv;          // qd + 2*kvd
  float s;           // alpha / r
};
bool make_shape(const qls_model_cfg* c, Shape* out, std::string* why);

// One layer record: all code blobs back to back (module order), then the
// absmax data, then the two bf16 norms; regions 256-B aligned.  Back-to-back
// blobs make q|k|v and gate|up single row-major NF4 matrices.
//   QLS_ABSMAX_F32: all float32 absmax arrays back to back (absmax_off).
//   QLS_ABSMAX_DQ8: all 8-bit absmax codes back to back (q8_off), then all
//   float32 group scales back to back (scale_off, one per 256 blocks of a
//   module).  The session expands them into float32 arrays laid out as
//   exp_off (back to back, the F32 layout shifted to 0) before a layer's use.
struct RecordLayout {
  int fmt;
  int64_t code_off[QLS_NMOD];
  int64_t absmax_off[QLS_NMOD];            // F32 only
  int64_t q8_off[QLS_NMOD], scale_off[QLS_NMOD];   // DQ8 only
  int64_t exp_off[QLS_NMOD];               // float32 absmax, relative (both formats)
  int64_t nblocks;                          // absmax entries of the layer
  int64_t block_start[QLS_NMOD + 1];        // first absmax index of each module
  int64_t scale_start[QLS_NMOD];            // first group scale of each module
  int64_t norm_attn_off, norm_mlp_off;
  int64_t bytes;
};
RecordLayout record_layout(const Shape& sh, int fmt);
// Second-level absmax quantisation (host, float32 IEEE, no contraction).
void nf4_double_quant_host(const float* absmax, int64_t nb, uint8_t* q8, float* scales);
// Device expansion of one layer's DQ8 absmax into float32 (layout exp_off).
int absmax_expand_launch(const uint8_t* rec, const RecordLayout& lay, float* out, hipStream_t st);
// Device expansion of one array: out[i] = float32(q8[i] * scales[i / 256]).
int absmax_expand_flat_launch(const uint8_t* q8, const float* scales, int64_t nb, float* out,
                              hipStream_t st);

// Offsets (elements) of each module's A and B in the packed float32 LoRA
// vector, per layer, plus the per-layer stride.
struct LoraLayout {
  int64_t a_off[QLS_NMOD], b_off[QLS_NMOD];
  int64_t per_layer;
};
LoraLayout lora_layout(const Shape& sh);

// Store accessors (store.cpp).
const Shape& store_shape(const qls_store* st);
const RecordLayout& store_layout(const qls_store* st);
// Host record of a pinned layer (nullptr for a disk-tier layer).
const uint8_t* store_record(const qls_store* st, int layer);
// Layers [0, store_ram_layers) are pinned; the rest are read from store_disk.
int store_ram_layers(const qls_store* st);
class DiskFile;
const DiskFile* store_disk(const qls_store* st);
bool store_complete(const qls_store* st, int* missing);
