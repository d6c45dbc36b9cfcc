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

// One layer record: all code blobs back to back (module order), then all
// absmax arrays back to back, then the two bf16 norms; regions 256-B aligned.
// Back-to-back blobs make q|k|v and gate|up single row-major NF4 matrices.
struct RecordLayout {
  int64_t code_off[QLS_NMOD];
  int64_t absmax_off[QLS_NMOD];
  int64_t norm_attn_off, norm_mlp_off;
  int64_t bytes;
};
RecordLayout record_layout(const Shape& sh);

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
const uint8_t* store_record(const qls_store* st, int layer);
bool store_complete(const qls_store* st, int* missing);
