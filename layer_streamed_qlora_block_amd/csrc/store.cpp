// Pinned NF4 host store: one record per decoder layer.
//
// The frozen decoder stack lives in page-locked host memory so the layer
// copies can run asynchronously next to compute (page "Can You Fine-Tune Llama
// 3.1 8B on a 4GB GPU? ...", sections "How Soup's layer streaming actually
// works", item 2, and "Why NF4 matters so much"; page "Fine tune an 8B model on
// a 4GB laptop GPU (Soup setup)", section "Step 2, train": the base store is
// pinned in RAM across 32 layers).
#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>

#include "disk.h"
#include "internal.h"

struct qls_store {
  Shape sh;
  RecordLayout lay;   // lay.fmt: QLS_ABSMAX_F32 or QLS_ABSMAX_DQ8
  uint8_t* host = nullptr;          // ram_layers * lay.bytes, hipHostMalloc
  int ram_layers = 0;               // layers [0, ram_layers) pinned, the rest in `disk`
  DiskFile disk;
  mutable std::vector<uint8_t> view; // last disk record handed out by a layer view
  std::vector<char> ready;
};

bool make_shape(const qls_model_cfg* c, Shape* o, std::string* why) {
  auto bad = [&](const char* m) { if (why) *why = m; return false; };
  if (!c) return bad("cfg is NULL");
  if (c->n_layers <= 0 || c->hidden <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 ||
      c->head_dim <= 0 || c->intermediate <= 0 || c->vocab <= 0 || c->lora_r <= 0)
    return bad("all sizes must be positive");
  if (c->n_heads % c->n_kv_heads) return bad("n_heads must be a multiple of n_kv_heads");
  if (!(c->rms_eps > 0) || !(c->rope_theta > 0) || !(c->lora_alpha > 0))
    return bad("rms_eps, rope_theta and lora_alpha must be positive");
  o->c = *c;
  o->qd = c->n_heads * c->head_dim;
  o->kvd = c->n_kv_heads * c->head_dim;
  o->nqkv = o->qd + 2 * o->kvd;
  const int d = c->hidden, I = c->intermediate;
  o->mod[QLS_Q] = {o->qd, d};
  o->mod[QLS_K] = {o->kvd, d};
  o->mod[QLS_V] = {o->kvd, d};
  o->mod[QLS_O] = {d, o->qd};
  o->mod[QLS_GATE] = {I, d};
  o->mod[QLS_UP] = {I, d};
  o->mod[QLS_DOWN] = {d, I};
  for (int m = 0; m < QLS_NMOD; ++m) {
    o->numel[m] = (int64_t)o->mod[m].out * o->mod[m].in;
    if (o->numel[m] % 64) return bad("every linear's numel must be a multiple of 64");
  }
  o->s = c->lora_alpha / (float)c->lora_r;
  return true;
}

RecordLayout record_layout(const Shape& sh, int fmt) {
  RecordLayout L{};
  L.fmt = fmt;
  int64_t off = 0;
  for (int m = 0; m < QLS_NMOD; ++m) { L.code_off[m] = off; off += sh.numel[m] / 2; }
  off = align_up(off, 256);
  int64_t e = 0, b = 0, g = 0;
  for (int m = 0; m < QLS_NMOD; ++m) {
    L.exp_off[m] = e;
    L.block_start[m] = b;
    L.scale_start[m] = g;
    e += sh.numel[m] / 64 * 4;
    b += sh.numel[m] / 64;
    g += cdiv(sh.numel[m] / 64, 256);
  }
  L.block_start[QLS_NMOD] = b;
  L.nblocks = b;
  if (fmt == QLS_ABSMAX_DQ8) {
    for (int m = 0; m < QLS_NMOD; ++m) L.q8_off[m] = off + L.block_start[m];
    off = align_up(off + b, 256);
    for (int m = 0; m < QLS_NMOD; ++m) L.scale_off[m] = off + 4 * L.scale_start[m];
    off = align_up(off + 4 * g, 256);
  } else {
    for (int m = 0; m < QLS_NMOD; ++m) L.absmax_off[m] = off + L.exp_off[m];
    off = align_up(off + e, 256);
  }
  L.norm_attn_off = off; off = align_up(off + 2LL * sh.c.hidden, 256);
  L.norm_mlp_off = off; off = align_up(off + 2LL * sh.c.hidden, 256);
  L.bytes = off;
  return L;
}

LoraLayout lora_layout(const Shape& sh) {
  LoraLayout L{};
  int64_t off = 0;
  const int r = sh.c.lora_r;
  for (int m = 0; m < QLS_NMOD; ++m) {
    L.a_off[m] = off; off += (int64_t)r * sh.mod[m].in;
    L.b_off[m] = off; off += (int64_t)sh.mod[m].out * r;
  }
  L.per_layer = off;
  return L;
}

// ---------------------------------------------------------------- quantiser
// code = argmin_j |w/a - cb[j]| with the division, subtraction and comparison
// in float32 (ties to the lower index); an all-zero block is code 7, absmax 0.
static void quantize_blocks(const float* w, int64_t b0, int64_t b1, uint8_t* codes, float* absmax,
                            const float* cb) {
  for (int64_t b = b0; b < b1; ++b) {
    const float* x = w + b * 64;
    float a = 0.f;
    for (int e = 0; e < 64; ++e) a = std::max(a, std::fabs(x[e]));
    absmax[b] = a;
    uint8_t* out = codes + b * 32;
    if (a == 0.f) {
      std::memset(out, 0x77, 32);
      continue;
    }
    uint8_t idx[64];
    for (int e = 0; e < 64; ++e) {
      const float n = x[e] / a;   // one IEEE float32 division (no fast-math)
      int best = 0;
      float bd = std::fabs(n - cb[0]);
      for (int j = 1; j < 16; ++j) {
        const float dj = std::fabs(n - cb[j]);
        if (dj < bd) { bd = dj; best = j; }
      }
      idx[e] = (uint8_t)best;
    }
    for (int k = 0; k < 32; ++k) out[k] = (uint8_t)((idx[2 * k] << 4) | idx[2 * k + 1]);
  }
}

// Second level: per group of 256 absmax values s = f32(max / 255), q =
// clamp(rint(f32(a / s)), 0, 255) (round half to even), s = 0 -> q = 0.
void nf4_double_quant_host(const float* a, int64_t nb, uint8_t* q8, float* scales) {
  for (int64_t g0 = 0, gi = 0; g0 < nb; g0 += 256, ++gi) {
    const int64_t g1 = std::min<int64_t>(nb, g0 + 256);
    float c = 0.f;
    for (int64_t i = g0; i < g1; ++i) c = std::max(c, a[i]);
    const float sc = c / 255.0f;
    scales[gi] = sc;
    for (int64_t i = g0; i < g1; ++i) {
      if (!(sc > 0.f)) { q8[i] = 0; continue; }
      const float x = std::nearbyint(a[i] / sc);   // default rounding: nearest, ties to even
      q8[i] = (uint8_t)std::min(255.f, std::max(0.f, x));
    }
  }
}

void nf4_quantize_host(const float* w, int64_t n, uint8_t* codes, float* absmax, int n_threads) {
  float cb[16];
  nf4_codebook_host(cb);
  const int64_t nb = n / 64;
  int nt = n_threads > 0 ? n_threads : (int)std::max(1u, std::thread::hardware_concurrency());
  nt = (int)std::min<int64_t>(nt, std::max<int64_t>(1, nb / 1024));
  if (nt <= 1) { quantize_blocks(w, 0, nb, codes, absmax, cb); return; }
  std::vector<std::thread> th;
  for (int i = 0; i < nt; ++i) {
    const int64_t b0 = nb * i / nt, b1 = nb * (i + 1) / nt;
    th.emplace_back(quantize_blocks, w, b0, b1, codes, absmax, cb);
  }
  for (auto& x : th) x.join();
}

// ---------------------------------------------------------------- C ABI
extern "C" {

int64_t qls_layer_record_bytes_fmt(const qls_model_cfg* cfg, int absmax_format) {
  Shape sh;
  std::string why;
  if (!make_shape(cfg, &sh, &why)) return fail(QLS_EINVAL, why);
  if (absmax_format != QLS_ABSMAX_F32 && absmax_format != QLS_ABSMAX_DQ8)
    return fail(QLS_EINVAL, "absmax_format must be QLS_ABSMAX_F32 or QLS_ABSMAX_DQ8");
  return record_layout(sh, absmax_format).bytes;
}

int64_t qls_layer_record_bytes(const qls_model_cfg* cfg) {
  return qls_layer_record_bytes_fmt(cfg, QLS_ABSMAX_F32);
}

int64_t qls_lora_numel(const qls_model_cfg* cfg) {
  Shape sh;
  std::string why;
  if (!make_shape(cfg, &sh, &why)) return fail(QLS_EINVAL, why);
  return lora_layout(sh).per_layer * cfg->n_layers;
}

int qls_nf4_codebook(float out[16]) {
  if (!out) return fail(QLS_EINVAL, "out is NULL");
  nf4_codebook_host(out);
  return QLS_OK;
}

int qls_nf4_quantize(const float* w, int64_t n, uint8_t* codes, float* absmax, int n_threads) {
  if (!w || !codes || !absmax) return fail(QLS_EINVAL, "NULL buffer");
  if (n < 0 || n % 64) return fail(QLS_EINVAL, "n must be a non-negative multiple of 64");
  nf4_quantize_host(w, n, codes, absmax, n_threads);
  return QLS_OK;
}

int qls_nf4_double_quant(const float* absmax, int64_t nblocks, uint8_t* q8, float* scales) {
  if (!absmax || !q8 || !scales) return fail(QLS_EINVAL, "NULL buffer");
  if (nblocks < 0) return fail(QLS_EINVAL, "nblocks must be non-negative");
  nf4_double_quant_host(absmax, nblocks, q8, scales);
  return QLS_OK;
}

int qls_store_create_fmt(const qls_model_cfg* cfg, int absmax_format, uint64_t max_pinned_bytes,
                         qls_store** out) {
  if (!out) return fail(QLS_EINVAL, "out is NULL");
  *out = nullptr;
  Shape sh;
  std::string why;
  if (!make_shape(cfg, &sh, &why)) return fail(QLS_EINVAL, why);
  if (absmax_format != QLS_ABSMAX_F32 && absmax_format != QLS_ABSMAX_DQ8)
    return fail(QLS_EINVAL, "absmax_format must be QLS_ABSMAX_F32 or QLS_ABSMAX_DQ8");
  auto* st = new (std::nothrow) qls_store;
  if (!st) return fail(QLS_ENOMEM, "host allocation failed");
  st->sh = sh;
  st->lay = record_layout(sh, absmax_format);
  const uint64_t total = (uint64_t)st->lay.bytes * (uint64_t)cfg->n_layers;
  if (max_pinned_bytes && total > max_pinned_bytes) {
    delete st;
    return fail(QLS_ENOPIN, "store of " + std::to_string(total) + " bytes exceeds the pinned cap of " +
                                std::to_string(max_pinned_bytes));
  }
  hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&st->host), total, hipHostMallocDefault);
  if (e != hipSuccess || !st->host) {
    delete st;
    return fail(QLS_ENOPIN, std::string("hipHostMalloc of the store failed: ") + hipGetErrorString(e));
  }
  st->ram_layers = cfg->n_layers;
  st->ready.assign(cfg->n_layers, 0);
  *out = st;
  return QLS_OK;
}

int qls_store_create(const qls_model_cfg* cfg, uint64_t max_pinned_bytes, qls_store** out) {
  return qls_store_create_fmt(cfg, QLS_ABSMAX_F32, max_pinned_bytes, out);
}

int qls_store_create_tiered(const qls_model_cfg* cfg, int absmax_format, int ram_layers, const char* path,
                            qls_store** out) {
  if (!out) return fail(QLS_EINVAL, "out is NULL");
  *out = nullptr;
  Shape sh;
  std::string why;
  if (!make_shape(cfg, &sh, &why)) return fail(QLS_EINVAL, why);
  if (absmax_format != QLS_ABSMAX_F32 && absmax_format != QLS_ABSMAX_DQ8)
    return fail(QLS_EINVAL, "absmax_format must be QLS_ABSMAX_F32 or QLS_ABSMAX_DQ8");
  if (ram_layers < 0 || ram_layers > cfg->n_layers) return fail(QLS_EINVAL, "ram_layers must be in [0, n_layers]");
  if (ram_layers < cfg->n_layers && (!path || !*path)) return fail(QLS_EINVAL, "disk layers need a file path");
  auto* st = new (std::nothrow) qls_store;
  if (!st) return fail(QLS_ENOMEM, "host allocation failed");
  st->sh = sh;
  st->lay = record_layout(sh, absmax_format);
  st->ram_layers = ram_layers;
  if (ram_layers > 0) {
    hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&st->host), (size_t)st->lay.bytes * ram_layers,
                                 hipHostMallocDefault);
    if (e != hipSuccess || !st->host) {
      delete st;
      return fail(QLS_ENOPIN, std::string("hipHostMalloc of the store failed: ") + hipGetErrorString(e));
    }
  }
  if (ram_layers < cfg->n_layers && st->disk.open(path, st->lay.bytes, cfg->n_layers - ram_layers, &why)) {
    qls_store_destroy(st);
    return fail(QLS_EIO, why);
  }
  st->ready.assign(cfg->n_layers, 0);
  *out = st;
  return QLS_OK;
}

int qls_store_layer_tier(const qls_store* st, int layer) {
  if (!st) return fail(QLS_EINVAL, "NULL argument");
  if (layer < 0 || layer >= st->sh.c.n_layers) return fail(QLS_EINVAL, "layer out of range");
  return layer < st->ram_layers ? QLS_TIER_PINNED : QLS_TIER_DISK;
}

// Where set_layer_* builds layer's record: in place for a pinned layer, in
// the caller's buffer (then written to the file) for a disk layer, so layers
// can be set from several threads at once.
static uint8_t* record_dst(qls_store* st, int layer, std::vector<uint8_t>* local) {
  if (layer < st->ram_layers) return st->host + (int64_t)layer * st->lay.bytes;
  local->assign((size_t)st->lay.bytes, 0);
  return local->data();
}

static int record_commit(qls_store* st, int layer, const uint8_t* rec) {
  if (layer < st->ram_layers) return QLS_OK;
  const int rc = st->disk.write(layer - st->ram_layers, rec);
  if (rc) return fail(QLS_EIO, std::string("disk tier write failed: ") + std::strerror(-rc));
  return QLS_OK;
}

// Write module m's absmax into the record in the store's format.
static void put_absmax(qls_store* st, uint8_t* rec, int m, const float* absmax) {
  const int64_t nb = st->sh.numel[m] / 64;
  if (st->lay.fmt == QLS_ABSMAX_DQ8)
    nf4_double_quant_host(absmax, nb, rec + st->lay.q8_off[m],
                          reinterpret_cast<float*>(rec + st->lay.scale_off[m]));
  else
    std::memcpy(rec + st->lay.absmax_off[m], absmax, nb * 4);
}

static int set_norms(qls_store* st, uint8_t* rec, const uint16_t* na, const uint16_t* nm) {
  std::memcpy(rec + st->lay.norm_attn_off, na, 2 * (size_t)st->sh.c.hidden);
  std::memcpy(rec + st->lay.norm_mlp_off, nm, 2 * (size_t)st->sh.c.hidden);
  return QLS_OK;
}

int qls_store_set_layer_fp32(qls_store* st, int layer, const float* const w[QLS_NMOD],
                             const uint16_t* na, const uint16_t* nm, int n_threads) {
  if (!st || !w || !na || !nm) return fail(QLS_EINVAL, "NULL argument");
  if (layer < 0 || layer >= st->sh.c.n_layers) return fail(QLS_EINVAL, "layer out of range");
  for (int m = 0; m < QLS_NMOD; ++m)
    if (!w[m]) return fail(QLS_EINVAL, "NULL weight");
  std::vector<uint8_t> local;
  uint8_t* rec = record_dst(st, layer, &local);
  std::vector<float> amax;
  for (int m = 0; m < QLS_NMOD; ++m) {
    if (st->lay.fmt == QLS_ABSMAX_F32) {
      nf4_quantize_host(w[m], st->sh.numel[m], rec + st->lay.code_off[m],
                        reinterpret_cast<float*>(rec + st->lay.absmax_off[m]), n_threads);
    } else {
      amax.resize(st->sh.numel[m] / 64);
      nf4_quantize_host(w[m], st->sh.numel[m], rec + st->lay.code_off[m], amax.data(), n_threads);
      put_absmax(st, rec, m, amax.data());
    }
  }
  set_norms(st, rec, na, nm);
  const int rc = record_commit(st, layer, rec);
  if (rc) return rc;
  st->ready[layer] = 1;
  return QLS_OK;
}

int qls_store_set_layer_nf4(qls_store* st, int layer, const uint8_t* const codes[QLS_NMOD],
                            const float* const absmax[QLS_NMOD], const uint16_t* na,
                            const uint16_t* nm) {
  if (!st || !codes || !absmax || !na || !nm) return fail(QLS_EINVAL, "NULL argument");
  if (layer < 0 || layer >= st->sh.c.n_layers) return fail(QLS_EINVAL, "layer out of range");
  for (int m = 0; m < QLS_NMOD; ++m)
    if (!codes[m] || !absmax[m]) return fail(QLS_EINVAL, "NULL module buffer");
  std::vector<uint8_t> local;
  uint8_t* rec = record_dst(st, layer, &local);
  for (int m = 0; m < QLS_NMOD; ++m) {
    std::memcpy(rec + st->lay.code_off[m], codes[m], st->sh.numel[m] / 2);
    put_absmax(st, rec, m, absmax[m]);
  }
  set_norms(st, rec, na, nm);
  const int rc = record_commit(st, layer, rec);
  if (rc) return rc;
  st->ready[layer] = 1;
  return QLS_OK;
}

int qls_store_layer_view(const qls_store* st, int layer, qls_layer_view* out) {
  if (!st || !out) return fail(QLS_EINVAL, "NULL argument");
  if (layer < 0 || layer >= st->sh.c.n_layers) return fail(QLS_EINVAL, "layer out of range");
  const uint8_t* rec;
  if (layer < st->ram_layers) {
    rec = st->host + (int64_t)layer * st->lay.bytes;
  } else {
    if (!st->ready[layer]) return fail(QLS_ESTATE, "layer was never set");
    st->view.resize((size_t)st->lay.bytes);
    const int rc = st->disk.read_any(layer - st->ram_layers, st->view.data());
    if (rc) return fail(QLS_EIO, std::string("disk tier read failed: ") + std::strerror(-rc));
    rec = st->view.data();
  }
  const bool dq = st->lay.fmt == QLS_ABSMAX_DQ8;
  out->absmax_format = st->lay.fmt;
  for (int m = 0; m < QLS_NMOD; ++m) {
    out->codes[m] = rec + st->lay.code_off[m];
    out->absmax[m] = dq ? nullptr : reinterpret_cast<const float*>(rec + st->lay.absmax_off[m]);
    out->absmax_q8[m] = dq ? rec + st->lay.q8_off[m] : nullptr;
    out->absmax_scale[m] = dq ? reinterpret_cast<const float*>(rec + st->lay.scale_off[m]) : nullptr;
  }
  out->norm_attn = reinterpret_cast<const uint16_t*>(rec + st->lay.norm_attn_off);
  out->norm_mlp = reinterpret_cast<const uint16_t*>(rec + st->lay.norm_mlp_off);
  out->record = rec;
  out->record_bytes = st->lay.bytes;
  return QLS_OK;
}

void qls_store_destroy(qls_store* st) {
  if (!st) return;
  if (st->host) (void)hipHostFree(st->host);
  delete st;
}

}  // extern "C"

// Accessors for the session code.
const Shape& store_shape(const qls_store* st) { return st->sh; }
const RecordLayout& store_layout(const qls_store* st) { return st->lay; }
const uint8_t* store_record(const qls_store* st, int layer) {
  return layer < st->ram_layers ? st->host + (int64_t)layer * st->lay.bytes : nullptr;
}
int store_ram_layers(const qls_store* st) { return st->ram_layers; }
const DiskFile* store_disk(const qls_store* st) { return st->disk.is_open() ? &st->disk : nullptr; }
bool store_complete(const qls_store* st, int* missing) {
  for (int l = 0; l < (int)st->ready.size(); ++l)
    if (!st->ready[l]) { if (missing) *missing = l; return false; }
  return true;
}
