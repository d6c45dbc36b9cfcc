// Session: workspace plan, two-slot streaming pool and the step schedules.
//
// The frozen decoder stack streams from the pinned store into a small pool of
// device buffers, one layer ahead of compute; a slot is reused once the layer
// it held is finished (page "Can You Fine-Tune Llama 3.1 8B on a 4GB GPU?
// ...", section "How Soup's layer streaming actually works", item 3).  The
// backward sweep reads the layers again because each layer's forward is
// recomputed from its checkpointed input (same section, item 4), except at
// the two ends of the sweep, where the copy engine idles: the last layer's
// forward intermediates are still in the workspace at the turn, and layer 0's
// are saved by the forward sweep for the backward that closes the step.  The last two layers of the forward sweep are still resident at the
// turn, so a step loads 2L - 2 records; a slot that still holds the layer a prefetch asks for is not
// copied again (across steps too).
//
// Ordering is two-sided with events: a slot is overwritten only after
// `released[s]` (recorded on the compute stream after the last kernel that
// reads slot s) has completed, and the compute stream waits on `copied[s]`
// before the first kernel that reads it.  That is the guard against the
// size-dependent silent wrong-gradient class of bug described on the same page
// ("Did a correctness bug invalidate the Llama 3.1 8B result?").
//
// The release is awaited on the host, which then enqueues the copy: a
// device-side wait of the copy stream on the compute stream's event delays
// each copy by 50-80 us on this runtime even when the event completed long
// before, and the copies are the step's critical path when it is link-bound.
// To keep the compute stream fed meanwhile, the sweeps request layer l+1
// after enqueueing layer l (its slot was released by layer l-1), so the host
// blocks while a whole layer of kernels is queued.  QLS_DBG_STREAM_FENCE
// restores the device-side wait.
//
// The first copy of each sweep (layer 2 going forward, layer L-3 going
// backward) would wait for a layer that holds a pinned slot while the copy
// engine idles: layer 0's forward at the start of a step, the last layer's
// backward at the turn.  That copy goes in five parts: the q|k|v, o, gate|up
// and down codes and the rest (absmax data and norms).  The layer's kernels
// stop reading the code parts one after another (in module order going
// forward, in reverse order in the backward), each part has its own release
// event, recorded after the last product that reads it, and the copy takes
// the parts in that order, each after its own event, the rest after
// `released[s]`; it so starts with the layer's first product instead of after
// its last kernel.  Every other copy is one transfer after `released[s]`
// (each extra transfer costs the link some throughput).
#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstring>
#include <memory>
#include <thread>
#include <vector>

#include "attn.h"
#include "disk.h"
#include "gemm.h"
#include "internal.h"
#include "ops.h"

namespace {

constexpr int kTile = 128;

// Parts of a layer record, in the order of its bytes: the q|k|v, o, gate|up
// and down code blobs, then the rest (absmax data, norms).
enum { PART_QKV = 0, PART_O, PART_GU, PART_DOWN, PART_REST };
constexpr unsigned kAllParts = (1u << PART_REST) - 1;

struct Plan {
  int64_t slots, ckpt, n1, qkv, attn, lse, Dv, h, n2, gu, a, uqkv, uo, ugu, udown;
  int64_t g, dh, dn, dyb, dgu, dattn, dqf, dkf, dvf, dqkv, du, xo;
  int64_t lbf, hf, stats, lse_t, tgt_logit, logp, logp_ref, roww, tgt, ids, dlog, dhf, part;
  int64_t xref0, xref1, scal, rope;
  int64_t amax;   // two float32 absmax expansions (double-quantised stores only)
  int64_t acts0;  // layer 0's forward intermediates, kept for its backward (the [n1, g) range)
  int64_t total;
};

struct Sizes {
  int Tm, Smax, Vc, ntiles, nchunks;
};

Sizes sizes_of(const Shape& sh, const qls_run_cfg& run) {
  Sizes z{};
  z.Tm = run.max_tokens;
  z.Smax = run.max_seq;
  int vc = run.ce_chunk > 0 ? run.ce_chunk : 32768;
  vc = (int)align_up(vc, kTile);
  z.Vc = std::min<int>(vc, (int)align_up(sh.c.vocab, kTile));
  z.ntiles = (int)cdiv(sh.c.vocab, kTile);
  z.nchunks = (int)cdiv(sh.c.vocab, z.Vc);
  return z;
}

// The skinny LoRA products of one layer's backward, in the groups that run
// as one launch each (plus one reduce): the du of each linear group, then
// its dB and dA.  Pointers null: sizes only (dA of a single module: rows =
// r, one block).
struct SkGroups { SkinnyProd p[8][4]; int n[8]; };
SkGroups layer_groups(const Shape& sh, int T) {
  SkGroups G{};
  const int d = sh.c.hidden, I = sh.c.intermediate, r = sh.c.lora_r;
  float* nil[4] = {nullptr, nullptr, nullptr, nullptr};
  G.p[0][0] = sk_du(nullptr, d, T, d, nullptr, r, 1.f, nullptr, r); G.n[0] = 1;                  // down
  G.p[1][0] = sk_dB(nullptr, d, T, d, nullptr, r, 1.f, nullptr, r);
  G.p[1][1] = sk_dA_multi(nullptr, r, T, r, 1, nullptr, I, I, nil); G.n[1] = 2;
  for (int k = 0; k < 2; ++k) {                                                                   // gate, up
    G.p[2][k] = sk_du(nullptr, 2 * I, T, I, nullptr, r, 1.f, nullptr, 2 * r);
    G.p[3][k] = sk_dB(nullptr, 2 * I, T, I, nullptr, 2 * r, 1.f, nullptr, r);
  }
  G.n[2] = 2;
  G.p[3][2] = sk_dA_multi(nullptr, 2 * r, T, r, 2, nullptr, d, d, nil); G.n[3] = 3;
  G.p[4][0] = sk_du(nullptr, d, T, d, nullptr, r, 1.f, nullptr, r); G.n[4] = 1;                  // o
  G.p[5][0] = sk_dB(nullptr, d, T, d, nullptr, r, 1.f, nullptr, r);
  G.p[5][1] = sk_dA_multi(nullptr, r, T, r, 1, nullptr, sh.qd, sh.qd, nil); G.n[5] = 2;
  const int nout[3] = {sh.qd, sh.kvd, sh.kvd};
  for (int k = 0; k < 3; ++k) {                                                                   // q, k, v
    G.p[6][k] = sk_du(nullptr, sh.nqkv, T, nout[k], nullptr, r, 1.f, nullptr, 3 * r);
    G.p[7][k] = sk_dB(nullptr, sh.nqkv, T, nout[k], nullptr, 3 * r, 1.f, nullptr, r);
  }
  G.n[6] = 3;
  G.p[7][3] = sk_dA_multi(nullptr, 3 * r, T, r, 3, nullptr, d, d, nil); G.n[7] = 4;
  return G;
}

// Floats of the split-K partial buffer: the largest any skinny product or
// group of them lays out at T tokens (their split factors grow with the
// contraction over T, so the session's largest T bounds every call), with the
// floors of skinny_partial_floats (which cover the dequant-GEMM splits too).
int64_t part_floats(const Shape& sh, int64_t T) {
  const int64_t d = sh.c.hidden, I = sh.c.intermediate, r = sh.c.lora_r;
  const int64_t mx = std::max({T * 3 * r, I * r, (int64_t)sh.qd * r, r * std::max<int64_t>(d, I), 3 * r * d,
                               2 * r * d});
  int64_t need = skinny_partial_floats(mx);
  const SkGroups G = layer_groups(sh, (int)T);
  for (int i = 0; i < 8; ++i) need = std::max(need, skinny_group_floats(G.p[i], G.n[i]));
  return need;
}

Plan make_plan(const Shape& sh, const RecordLayout& lay, const qls_run_cfg& run, int64_t lora_numel) {
  const Sizes z = sizes_of(sh, run);
  const int64_t T = z.Tm, d = sh.c.hidden, I = sh.c.intermediate, r = sh.c.lora_r;
  const int64_t L = sh.c.n_layers, H = sh.c.n_heads;
  Plan p{};
  int64_t off = 0;
  auto take = [&](int64_t bytes) { const int64_t o = off; off = align_up(off + std::max<int64_t>(bytes, 1), 256); return o; };
  p.slots = take((run.mode == QLS_RESIDENT ? L : 2) * lay.bytes);
  p.ckpt = take((L + 1) * T * d * 2);
  p.n1 = take(T * d * 2);
  p.qkv = take(T * sh.nqkv * 2);
  p.attn = take(T * sh.qd * 2);
  p.lse = take(T * H * 4);
  p.Dv = take(T * H * 4);
  p.h = take(T * d * 2);
  p.n2 = take(T * d * 2);
  p.gu = take(T * 2 * I * 2);
  p.a = take(T * I * 2);
  p.uqkv = take(T * 3 * r * 2);
  p.uo = take(T * r * 2);
  p.ugu = take(T * 2 * r * 2);
  p.udown = take(T * r * 2);
  p.g = take(T * d * 4);
  p.dh = take(T * d * 4);
  p.dn = take(T * d * 4);
  p.dyb = take(T * d * 2);
  p.dgu = take(T * 2 * I * 2);
  p.dattn = take(T * sh.qd * 2);
  p.dqf = take(T * sh.qd * 4);
  p.dkf = take(T * sh.qd * 4);    // per-query-head partials of dK and dV
  p.dvf = take(T * sh.qd * 4);
  p.dqkv = take(T * sh.nqkv * 2);
  p.du = take(T * 3 * r * 2);
  p.xo = take(T * d * 2);
  p.lbf = take(lora_numel * 2);
  p.hf = take(T * d * 2);
  p.stats = take(T * z.ntiles * 2 * 4);
  p.lse_t = take(T * 4);
  p.tgt_logit = take(T * 4);
  p.logp = take(T * 4);
  p.logp_ref = take(T * 4);
  p.roww = take(T * 4);
  p.tgt = take(T * 4);
  p.ids = take(T * 4);
  p.dlog = take(T * z.Vc * 2);
  p.dhf = take(T * d * 4);
  p.part = take(part_floats(sh, T) * 4);
  p.xref0 = take(T * d * 2);
  p.xref1 = take(T * d * 2);
  p.scal = take(64);
  p.rope = take((int64_t)z.Smax * (sh.c.head_dim / 2) * 2 * 4);
  p.amax = take(lay.fmt == QLS_ABSMAX_DQ8 ? 2 * lay.nblocks * 4 : 0);
  p.acts0 = take(p.g - p.n1);
  p.total = off;
  return p;
}

bool check_run(const Shape& sh, const qls_run_cfg* run, std::string* why) {
  auto bad = [&](const char* m) { *why = m; return false; };
  if (!run) return bad("run cfg is NULL");
  if (run->mode != QLS_STREAMED && run->mode != QLS_RESIDENT) return bad("mode must be STREAMED or RESIDENT");
  if (run->max_tokens <= 0 || run->max_seq < 2) return bad("max_tokens must be > 0 and max_seq >= 2");
  const qls_model_cfg& c = sh.c;
  if (c.head_dim != 64 && c.head_dim != 128) return bad("head_dim must be 64 or 128");
  if (c.n_heads / c.n_kv_heads > 8) return bad("at most 8 query heads per kv head");
  if (c.hidden % 16 || c.intermediate % 16 || sh.qd % 16 || sh.kvd % 16)
    return bad("hidden, intermediate and head widths must be multiples of 16");
  if (c.hidden > 8192) return bad("hidden must be at most 8192");
  if (c.lora_r % 8 || c.lora_r > 128) return bad("lora_r must be a multiple of 8 up to 128");
  if (c.vocab % 8) return bad("vocab must be a multiple of 8");
  return true;
}

struct TimedEv { hipEvent_t a, b; };
// A timed dequant-GEMM: a..b the kernel, b..c its split-K reduce (c null: none).
struct TimedK { hipEvent_t a, b, c; double gflop; bool big; };

}  // namespace

// AdamW folded into the backward sweep (qls_sft_step_adamw): on while one runs.
struct FusedOpt {
  bool on = false;
  float *p = nullptr, *m = nullptr, *v = nullptr;
  int t = 0;
  double lr = 0, b1 = 0, b2 = 0, eps = 0, wd = 0;
};

struct qls_session {
  const qls_store* st = nullptr;
  FusedOpt opt;
  int ram_layers = 0;                   // layers [ram_layers, L) come from the disk tier
  std::unique_ptr<DiskReader> disk;
  Shape sh;
  RecordLayout lay;
  LoraLayout ll;
  int64_t wa[QLS_NMOD], wb[QLS_NMOD];   // bf16 working-copy offsets (elements, per layer)
  CastSeg seg;
  qls_run_cfg run;
  Sizes z;
  Plan p;
  uint8_t* ws = nullptr;
  hipStream_t cs = nullptr, ps = nullptr;
  qls_resident res;
  hipEvent_t copied[2] = {}, released[2] = {};
  // Release of each code part of a slot (PART_*); `marked[s]` has bit p set
  // once the current use of slot s has recorded part p's event.
  hipEvent_t part_rel[2][PART_REST] = {};
  unsigned marked[2] = {0, 0};
  bool parts_next = false;   // the next copy goes in parts (set at the start of a sweep)
  int slot_layer[2] = {-1, -1};
  // Layer whose forward intermediates (with adapters) the workspace still
  // holds: the last layer of a forward sweep, until the backward reaches it.
  int acts_layer = -1;
  // Layer 0's forward intermediates (with adapters) were saved to p.acts0.
  bool acts0_saved = false;
  // Double-quantised stores: expansion buffer e = layer & 1 holds the float32
  // absmax of exp_layer[e], decoded from copy number exp_gen[e] of its slot.
  int64_t slot_gen[2] = {0, 0};
  int exp_layer[2] = {-1, -1};
  int64_t exp_gen[2] = {-1, -1};
  uint32_t dbg = 0;
  int delay_us = 0;
  // Test hook (qls_debug_capture_grads): residual gradients at every layer
  // boundary of a backward sweep, (n_layers + 1) x T x hidden floats.
  float* cap = nullptr;
  int64_t cap_n = 0;
  int64_t part_n = 0;       // floats of the split-K partial buffer (part_floats at max_tokens)
  int64_t peak_ws = 0;      // largest workspace a call since the last reset needed
  int64_t wall_khz = 100000;
  // stats
  int64_t steps = 0, loads = 0, h2d = 0;
  bool timing = false;
  std::vector<hipEvent_t> ev_pool;
  size_t ev_next = 0;
  // Timing mode: events accumulate over the steps since the last reset and are
  // folded into sums when the stats are read.
  std::vector<TimedEv> copy_ev, comp_ev, step_ev;
  std::vector<TimedK> kf_ev, kd_ev;
  void clear_timing() { ev_next = 0; copy_ev.clear(); comp_ev.clear(); step_ev.clear(); kf_ev.clear(); kd_ev.clear(); }
  int run_fwd(LinearFwd& f, bool lora, hipStream_t st) {
    if (timing) { f.ev0 = next_ev(); f.ev1 = next_ev(); f.ev2 = next_ev(); }
    const int rc = linear_fwd(f, st);
    if (timing && !rc)
      kf_ev.push_back({f.ev0, f.ev1, f.ksplit > 1 ? f.ev2 : nullptr,
                       2e-9 * f.T * (double)f.N * (f.K + (lora ? f.r : 0)), f.tile == 256});
    return rc;
  }
  int run_dx(LinearDx& d, hipStream_t st) {
    if (timing) { d.ev0 = next_ev(); d.ev1 = next_ev(); d.ev2 = next_ev(); }
    const int rc = linear_dx(d, st);
    if (timing && !rc)
      kd_ev.push_back({d.ev0, d.ev1, d.ksplit > 1 ? d.ev2 : nullptr,
                       2e-9 * d.T * (double)d.Nout * (d.Kc + d.rc), d.tile == 256});
    return rc;
  }

  // The product just enqueued on the compute stream was the last reader of
  // code part `part` of layer l's slot in this use of it.
  int mark(int l, int part) {
    if (run.mode == QLS_RESIDENT) return QLS_OK;
    QLS_HIP(hipEventRecord(part_rel[l & 1][part], cs));
    marked[l & 1] |= 1u << part;
    // Test hook: hold back the kernels after the release so that a copy into
    // a part that is still read later would land first.
    if (dbg & QLS_DBG_COMPUTE_DELAY) spin_delay((int64_t)delay_us * wall_khz / 1000, cs);
    return QLS_OK;
  }
  // Byte range [*a, *b) of part `part` of a record.
  void part_range(int part, int64_t* a, int64_t* b) const {
    static const int first[PART_REST + 1] = {QLS_Q, QLS_O, QLS_GATE, QLS_DOWN, -1};
    const int64_t codes_end = lay.code_off[QLS_DOWN] + sh.numel[QLS_DOWN] / 2;
    *a = part == PART_REST ? codes_end : lay.code_off[first[part]];
    *b = part == PART_DOWN ? codes_end : part == PART_REST ? lay.bytes : lay.code_off[first[part + 1]];
  }

  template <class T> T* at(int64_t off) const { return reinterpret_cast<T*>(ws + off); }
  float* amax_buf(int l) const { return at<float>(p.amax) + (int64_t)(l & 1) * lay.nblocks; }
  uint16_t* ck(int l) const { return at<uint16_t>(p.ckpt) + (int64_t)l * z.Tm * sh.c.hidden; }
  uint16_t* lw(int l) const { return at<uint16_t>(p.lbf) + (int64_t)l * ll.per_layer; }

  // Timing events: read only after both streams are synchronized, so they skip
  // the system-scope fence (cache write-back and invalidation) on record.
  hipEvent_t next_ev() {
    if (ev_next >= ev_pool.size()) {
      hipEvent_t e;
      if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
      ev_pool.push_back(e);
    }
    return ev_pool[ev_next++];
  }
};

namespace {

void sleep_cb(void* us) {
  std::this_thread::sleep_for(std::chrono::microseconds((int64_t)(intptr_t)us));
}

// ---------------------------------------------------------------- pool
// Enqueue the copy of `layer` into slot layer & 1 on the copy stream once the
// slot's release has completed, or part by part, each once its own release
// has completed, for the first copy of a sweep (blocking this thread until
// then).  A disk-tier layer is first read into a pinned staging
// buffer (blocking this thread until the read is done); dir = the sweep's
// direction: the order in which its layers free the code parts, and the
// reader's read-ahead.
int prefetch(qls_session* S, int layer, int dir) {
  if (S->run.mode == QLS_RESIDENT) return QLS_OK;
  const int s = layer & 1;
  const bool reuse = !(S->dbg & (QLS_DBG_NO_REUSE | QLS_DBG_POISON_ON_RELEASE));
  if (reuse && S->slot_layer[s] == layer) return QLS_OK;
  const bool parts = S->parts_next;
  S->parts_next = false;
  const uint8_t* src = store_record(S->st, layer);
  int buf = -1;
  if (layer >= S->ram_layers) {
    src = S->disk->take(layer, dir, &buf);
    if (!src) return fail(QLS_EIO, S->disk->error());
  }
  uint8_t* dst = S->at<uint8_t>(S->p.slots) + s * S->lay.bytes;
  static const int fwd_order[PART_REST + 1] = {PART_QKV, PART_O, PART_GU, PART_DOWN, PART_REST};
  static const int bwd_order[PART_REST + 1] = {PART_DOWN, PART_GU, PART_O, PART_QKV, PART_REST};
  // The device-side fence waits once, for the whole slot (`released[s]` is
  // recorded after every part's event).
  if (S->dbg & QLS_DBG_STREAM_FENCE) QLS_HIP(hipStreamWaitEvent(S->ps, S->released[s], 0));
  for (int i = parts ? 0 : PART_REST; i <= PART_REST; ++i) {
    const int part = dir >= 0 ? fwd_order[i] : bwd_order[i];
    if (!(S->dbg & QLS_DBG_STREAM_FENCE))
      QLS_HIP(hipEventSynchronize(part == PART_REST ? S->released[s] : S->part_rel[s][part]));
    if ((i == 0 || !parts) && (S->dbg & QLS_DBG_COPY_DELAY))
      QLS_HIP(hipLaunchHostFunc(S->ps, sleep_cb, (void*)(intptr_t)S->delay_us));
    int64_t a = 0, b = S->lay.bytes;
    if (parts) S->part_range(part, &a, &b);
    if (b <= a) continue;
    TimedEv te{};
    if (S->timing) { te.a = S->next_ev(); te.b = S->next_ev(); QLS_HIP(hipEventRecord(te.a, S->ps)); }
    QLS_HIP(hipMemcpyAsync(dst + a, src + a, (size_t)(b - a), hipMemcpyHostToDevice, S->ps));
    if (S->timing) { QLS_HIP(hipEventRecord(te.b, S->ps)); S->copy_ev.push_back(te); }
  }
  if (buf >= 0 && S->disk->after_copy(buf, S->ps)) return fail(QLS_EHIP, "hipEventRecord failed");
  QLS_HIP(hipEventRecord(S->copied[s], S->ps));
  S->slot_layer[s] = layer;
  S->slot_gen[s] += 1;
  S->loads += 1;
  S->h2d += S->lay.bytes;
  return QLS_OK;
}

int acquire(qls_session* S, int layer, const uint8_t** rec, TimedEv* te) {
  if (S->run.mode == QLS_RESIDENT) {
    *rec = S->at<uint8_t>(S->p.slots) + (int64_t)layer * S->lay.bytes;
  } else {
    const int s = layer & 1;
    if (S->slot_layer[s] != layer) {
      int rc = prefetch(S, layer, 1);
      if (rc) return rc;
    }
    QLS_HIP(hipStreamWaitEvent(S->cs, S->copied[s], 0));
    *rec = S->at<uint8_t>(S->p.slots) + s * S->lay.bytes;
    S->marked[s] = 0;
  }
  if (S->lay.fmt == QLS_ABSMAX_DQ8) {
    // Decode the 8-bit absmax of this record once per arrival, on the compute
    // stream (ordered after the copy fence and before the layer's kernels).
    const int e = layer & 1;
    const int64_t gen = S->run.mode == QLS_RESIDENT ? 0 : S->slot_gen[e];
    if (S->exp_layer[e] != layer || S->exp_gen[e] != gen) {
      if (absmax_expand_launch(*rec, S->lay, S->amax_buf(layer), S->cs))
        return fail(QLS_EHIP, "absmax expansion launch failed");
      S->exp_layer[e] = layer;
      S->exp_gen[e] = gen;
    }
  }
  if (S->timing) { te->a = S->next_ev(); te->b = S->next_ev(); QLS_HIP(hipEventRecord(te->a, S->cs)); }
  return QLS_OK;
}

int release(qls_session* S, int layer, TimedEv* te) {
  if (S->dbg & QLS_DBG_COMPUTE_DELAY) spin_delay((int64_t)S->delay_us * S->wall_khz / 1000, S->cs);
  if (S->timing) { QLS_HIP(hipEventRecord(te->b, S->cs)); S->comp_ev.push_back(*te); }
  if (S->run.mode == QLS_RESIDENT) return QLS_OK;
  const int s = layer & 1;
  // Parts this use did not mark are released with the rest.
  for (int part = 0; part < PART_REST; ++part)
    if (!(S->marked[s] >> part & 1)) QLS_HIP(hipEventRecord(S->part_rel[s][part], S->cs));
  S->marked[s] = kAllParts;
  QLS_HIP(hipEventRecord(S->released[s], S->cs));
  if (S->dbg & QLS_DBG_POISON_ON_RELEASE) {
    QLS_HIP(hipStreamWaitEvent(S->ps, S->released[s], 0));
    QLS_HIP(hipMemsetAsync(S->at<uint8_t>(S->p.slots) + s * S->lay.bytes, 0xFF, S->lay.bytes, S->ps));
    S->slot_layer[s] = -1;
  }
  return QLS_OK;
}

// ---------------------------------------------------------------- layer
struct W {
  const uint8_t* code[QLS_NMOD];
  const float* amax[QLS_NMOD];
  const uint16_t* na;
  const uint16_t* nm;
};

// The layer's codes and norms in its record; its float32 absmax in the record
// (F32 store) or in the expansion buffer acquire() decoded it into (DQ8 store).
W weights(const qls_session* S, const uint8_t* rec, int layer) {
  W w{};
  const bool dq = S->lay.fmt == QLS_ABSMAX_DQ8;
  for (int m = 0; m < QLS_NMOD; ++m) {
    w.code[m] = rec + S->lay.code_off[m];
    w.amax[m] = dq ? S->amax_buf(layer) + S->lay.exp_off[m] / 4
                   : reinterpret_cast<const float*>(rec + S->lay.absmax_off[m]);
  }
  w.na = reinterpret_cast<const uint16_t*>(rec + S->lay.norm_attn_off);
  w.nm = reinterpret_cast<const uint16_t*>(rec + S->lay.norm_mlp_off);
  return w;
}

#define QLS_RC(x) do { if (x) return fail(QLS_EHIP, "kernel launch configuration not built: " #x); } while (0)

int fwd_layer(qls_session* S, int l, const uint8_t* rec, const uint16_t* x, uint16_t* xout, bool lora,
              int T, int B, int Sq) {
  const Shape& sh = S->sh;
  const int d = sh.c.hidden, I = sh.c.intermediate, r = sh.c.lora_r;
  const W w = weights(S, rec, l);
  const uint16_t* lw = S->lw(l);
  hipStream_t st = S->cs;
  uint16_t* n1 = S->at<uint16_t>(S->p.n1);
  uint16_t* qkv = S->at<uint16_t>(S->p.qkv);
  uint16_t* attn = S->at<uint16_t>(S->p.attn);
  uint16_t* h = S->at<uint16_t>(S->p.h);
  uint16_t* n2 = S->at<uint16_t>(S->p.n2);
  uint16_t* gu = S->at<uint16_t>(S->p.gu);
  uint16_t* a = S->at<uint16_t>(S->p.a);
  float* part = S->at<float>(S->p.part);

  rmsnorm_fwd(x, w.na, sh.c.rms_eps, n1, T, d, st);
  LinearFwd f{};
  f.T = T; f.N = sh.nqkv; f.K = d; f.r = r; f.x = n1; f.ldx = d;
  f.codes = w.code[QLS_Q]; f.absmax = w.amax[QLS_Q];
  f.A = lora ? lw + S->wa[QLS_Q] : nullptr;
  f.nmod = 3; f.mod_end[0] = sh.qd; f.mod_end[1] = sh.qd + sh.kvd; f.mod_end[2] = sh.nqkv;
  f.Bm[0] = lw + S->wb[QLS_Q]; f.Bm[1] = lw + S->wb[QLS_K]; f.Bm[2] = lw + S->wb[QLS_V];
  f.s = sh.s; f.y = qkv; f.ldy = sh.nqkv; f.u = S->at<uint16_t>(S->p.uqkv); f.ws = part;
  QLS_RC(S->run_fwd(f, lora, st));
  QLS_RC(S->mark(l, PART_QKV));
  QLS_RC(rope_fwd(qkv, sh.nqkv, T, Sq, sh.c.n_heads, sh.c.n_kv_heads, sh.c.head_dim, S->at<float>(S->p.rope), st));
  AttnArgs aa{};
  aa.qkv = qkv; aa.ld = sh.nqkv; aa.q_off = 0; aa.k_off = sh.qd; aa.v_off = sh.qd + sh.kvd;
  aa.S = Sq; aa.H = sh.c.n_heads; aa.KV = sh.c.n_kv_heads; aa.hd = sh.c.head_dim;
  aa.scale = 1.f / std::sqrt((float)sh.c.head_dim);
  aa.out = attn; aa.ldo = sh.qd; aa.lse = S->at<float>(S->p.lse);
  QLS_RC(attn_fwd(aa, B, st));

  f = LinearFwd{};
  f.T = T; f.N = d; f.K = sh.qd; f.r = r; f.x = attn; f.ldx = sh.qd;
  f.codes = w.code[QLS_O]; f.absmax = w.amax[QLS_O];
  f.A = lora ? lw + S->wa[QLS_O] : nullptr;
  f.nmod = 1; f.mod_end[0] = d; f.Bm[0] = lw + S->wb[QLS_O];
  f.s = sh.s; f.res = x; f.ldres = d; f.y = h; f.ldy = d; f.u = S->at<uint16_t>(S->p.uo); f.ws = part;
  QLS_RC(S->run_fwd(f, lora, st));
  QLS_RC(S->mark(l, PART_O));

  rmsnorm_fwd(h, w.nm, sh.c.rms_eps, n2, T, d, st);
  f = LinearFwd{};
  f.T = T; f.N = 2 * I; f.K = d; f.r = r; f.x = n2; f.ldx = d;
  f.codes = w.code[QLS_GATE]; f.absmax = w.amax[QLS_GATE];
  f.A = lora ? lw + S->wa[QLS_GATE] : nullptr;
  f.nmod = 2; f.mod_end[0] = I; f.mod_end[1] = 2 * I;
  f.Bm[0] = lw + S->wb[QLS_GATE]; f.Bm[1] = lw + S->wb[QLS_UP];
  f.s = sh.s; f.y = gu; f.ldy = 2 * I; f.u = S->at<uint16_t>(S->p.ugu); f.ws = part;
  QLS_RC(S->run_fwd(f, lora, st));
  QLS_RC(S->mark(l, PART_GU));
  swiglu_fwd(gu, a, T, I, st);

  f = LinearFwd{};
  f.T = T; f.N = d; f.K = I; f.r = r; f.x = a; f.ldx = I;
  f.codes = w.code[QLS_DOWN]; f.absmax = w.amax[QLS_DOWN];
  f.A = lora ? lw + S->wa[QLS_DOWN] : nullptr;
  f.nmod = 1; f.mod_end[0] = d; f.Bm[0] = lw + S->wb[QLS_DOWN];
  f.s = sh.s; f.res = h; f.ldres = d; f.y = xout; f.ldy = d; f.u = S->at<uint16_t>(S->p.udown); f.ws = part;
  QLS_RC(S->run_fwd(f, lora, st));
  return S->mark(l, PART_DOWN);
}

// g (float [T, d]) holds dL/d(layer output) on entry and dL/d(layer input) on
// exit; dyb holds bf16(g) on entry and on exit (the kernel that produces g
// writes both).
int bwd_layer(qls_session* S, int l, const uint8_t* rec, const uint16_t* x, float* grads, int T, int B,
              int Sq) {
  const Shape& sh = S->sh;
  const int d = sh.c.hidden, I = sh.c.intermediate, r = sh.c.lora_r;
  const float s = sh.s;
  const W w = weights(S, rec, l);
  const uint16_t* lw = S->lw(l);
  hipStream_t st = S->cs;
  float* gl = grads + (int64_t)l * S->ll.per_layer;
  auto dA = [&](int m) { return gl + S->ll.a_off[m]; };
  auto dB = [&](int m) { return gl + S->ll.b_off[m]; };
  float* g = S->at<float>(S->p.g);
  float* dh = S->at<float>(S->p.dh);
  float* dn = S->at<float>(S->p.dn);
  uint16_t* dyb = S->at<uint16_t>(S->p.dyb);
  uint16_t* dgu = S->at<uint16_t>(S->p.dgu);
  uint16_t* du = S->at<uint16_t>(S->p.du);
  float* part = S->at<float>(S->p.part);
  const uint16_t* n1 = S->at<uint16_t>(S->p.n1);
  const uint16_t* n2 = S->at<uint16_t>(S->p.n2);
  const uint16_t* attn = S->at<uint16_t>(S->p.attn);
  const uint16_t* a = S->at<uint16_t>(S->p.a);
  const uint16_t* h = S->at<uint16_t>(S->p.h);
  const uint16_t* uqkv = S->at<uint16_t>(S->p.uqkv);
  const uint16_t* ugu = S->at<uint16_t>(S->p.ugu);

  const int64_t pf = S->part_n;
  // ---- down projection + SwiGLU (dY = dyb): du, then dB and dA as one group
  {
    const SkinnyProd g1[1] = {sk_du(dyb, d, T, d, lw + S->wb[QLS_DOWN], r, s, du, r)};
    QLS_RC(skinny_group(g1, 1, part, pf, st));
    float* const dAd[1] = {dA(QLS_DOWN)};
    const SkinnyProd g2[2] = {sk_dB(dyb, d, T, d, S->at<uint16_t>(S->p.udown), r, s, dB(QLS_DOWN), r),
                              sk_dA_multi(du, r, T, r, 1, a, I, I, dAd)};
    QLS_RC(skinny_group(g2, 2, part, pf, st));
  }
  LinearDx x1{};
  x1.T = T; x1.Kc = d; x1.Nout = I; x1.dy = dyb; x1.lddy = d;
  x1.codes = w.code[QLS_DOWN]; x1.absmax = w.amax[QLS_DOWN]; x1.ldq = I;
  x1.du = du; x1.lddu = r; x1.Acat = lw + S->wa[QLS_DOWN]; x1.rc = r;
  x1.out = dgu; x1.ldo = 2 * I; x1.epi = EPI_SWIGLU_BWD; x1.ws = part;
  x1.gu = S->at<uint16_t>(S->p.gu); x1.ldgu = 2 * I; x1.I = I;
  QLS_RC(S->run_dx(x1, st));
  QLS_RC(S->mark(l, PART_DOWN));

  // ---- gate / up: both du, then both dB and the dA of both (they contract n2: one product)
  {
    SkinnyProd g1[2], g2[3];
    for (int k = 0; k < 2; ++k) {
      const int m = k == 0 ? QLS_GATE : QLS_UP;
      g1[k] = sk_du(dgu + k * I, 2 * I, T, I, lw + S->wb[m], r, s, du + k * r, 2 * r);
      g2[k] = sk_dB(dgu + k * I, 2 * I, T, I, ugu + k * r, 2 * r, s, dB(m), r);
    }
    float* const dA_gu[2] = {dA(QLS_GATE), dA(QLS_UP)};
    g2[2] = sk_dA_multi(du, 2 * r, T, r, 2, n2, d, d, dA_gu);
    QLS_RC(skinny_group(g1, 2, part, pf, st));
    QLS_RC(skinny_group(g2, 3, part, pf, st));
  }
  LinearDx x2{};
  x2.T = T; x2.Kc = 2 * I; x2.Nout = d; x2.dy = dgu; x2.lddy = 2 * I;
  x2.codes = w.code[QLS_GATE]; x2.absmax = w.amax[QLS_GATE]; x2.ldq = d;
  x2.du = du; x2.lddu = 2 * r; x2.Acat = lw + S->wa[QLS_GATE]; x2.rc = 2 * r;
  x2.out = dn; x2.ldo = d; x2.epi = EPI_F32; x2.ws = part;
  QLS_RC(S->run_dx(x2, st));
  QLS_RC(S->mark(l, PART_GU));
  QLS_RC(rmsnorm_bwd(h, w.nm, sh.c.rms_eps, dn, g, dh, dyb, T, d, st));

  // ---- o projection: du, then dB and dA
  {
    const SkinnyProd g1[1] = {sk_du(dyb, d, T, d, lw + S->wb[QLS_O], r, s, du, r)};
    QLS_RC(skinny_group(g1, 1, part, pf, st));
    float* const dAo[1] = {dA(QLS_O)};
    const SkinnyProd g2[2] = {sk_dB(dyb, d, T, d, S->at<uint16_t>(S->p.uo), r, s, dB(QLS_O), r),
                              sk_dA_multi(du, r, T, r, 1, attn, sh.qd, sh.qd, dAo)};
    QLS_RC(skinny_group(g2, 2, part, pf, st));
  }
  LinearDx x3{};
  x3.T = T; x3.Kc = d; x3.Nout = sh.qd; x3.dy = dyb; x3.lddy = d;
  x3.codes = w.code[QLS_O]; x3.absmax = w.amax[QLS_O]; x3.ldq = sh.qd;
  x3.du = du; x3.lddu = r; x3.Acat = lw + S->wa[QLS_O]; x3.rc = r;
  x3.out = S->at<uint16_t>(S->p.dattn); x3.ldo = sh.qd; x3.epi = EPI_BF16; x3.ws = part;
  QLS_RC(S->run_dx(x3, st));
  QLS_RC(S->mark(l, PART_O));

  // ---- attention + RoPE
  AttnBwdArgs ab{};
  ab.qkv = S->at<uint16_t>(S->p.qkv); ab.ld = sh.nqkv; ab.q_off = 0; ab.k_off = sh.qd; ab.v_off = sh.qd + sh.kvd;
  ab.S = Sq; ab.H = sh.c.n_heads; ab.KV = sh.c.n_kv_heads; ab.hd = sh.c.head_dim;
  ab.scale = 1.f / std::sqrt((float)sh.c.head_dim);
  ab.dO = S->at<uint16_t>(S->p.dattn); ab.O = attn; ab.lddo = sh.qd;
  ab.lse = S->at<float>(S->p.lse); ab.D = S->at<float>(S->p.Dv);
  ab.dq = S->at<float>(S->p.dqf); ab.lddq = sh.qd;
  ab.dk = S->at<float>(S->p.dkf); ab.dv = S->at<float>(S->p.dvf); ab.lddkv = sh.qd;
  QLS_RC(attn_bwd(ab, B, st));
  uint16_t* dqkv = S->at<uint16_t>(S->p.dqkv);
  QLS_RC(rope_bwd(ab.dq, ab.dk, ab.dv, dqkv, sh.nqkv, T, Sq, sh.c.n_heads, sh.c.n_kv_heads, sh.c.head_dim,
                  S->at<float>(S->p.rope), st));

  // ---- q, k, v: the three du, then the three dB and the dA of all three (they contract n1: one product)
  {
    const int col[3] = {0, sh.qd, sh.qd + sh.kvd};
    const int nout[3] = {sh.qd, sh.kvd, sh.kvd};
    SkinnyProd g1[3], g2[4];
    for (int k = 0; k < 3; ++k) {
      const int m = QLS_Q + k;
      g1[k] = sk_du(dqkv + col[k], sh.nqkv, T, nout[k], lw + S->wb[m], r, s, du + k * r, 3 * r);
      g2[k] = sk_dB(dqkv + col[k], sh.nqkv, T, nout[k], uqkv + k * r, 3 * r, s, dB(m), r);
    }
    float* const dA_qkv[3] = {dA(QLS_Q), dA(QLS_K), dA(QLS_V)};
    g2[3] = sk_dA_multi(du, 3 * r, T, r, 3, n1, d, d, dA_qkv);
    QLS_RC(skinny_group(g1, 3, part, pf, st));
    QLS_RC(skinny_group(g2, 4, part, pf, st));
  }
  LinearDx x4{};
  x4.T = T; x4.Kc = sh.nqkv; x4.Nout = d; x4.dy = dqkv; x4.lddy = sh.nqkv;
  x4.codes = w.code[QLS_Q]; x4.absmax = w.amax[QLS_Q]; x4.ldq = d;
  x4.du = du; x4.lddu = 3 * r; x4.Acat = lw + S->wa[QLS_Q]; x4.rc = 3 * r;
  x4.out = dn; x4.ldo = d; x4.epi = EPI_F32; x4.ws = part;
  QLS_RC(S->run_dx(x4, st));
  QLS_RC(S->mark(l, PART_QKV));
  QLS_RC(rmsnorm_bwd(x, w.na, sh.c.rms_eps, dn, dh, g, dyb, T, d, st));
  return QLS_OK;
}

// ---------------------------------------------------------------- head
// Pass 1 over vocabulary chunks: per-row (max, sum exp) per 128-column tile and
// the target logit, then the log-sum-exp and per-row log-prob.
// LM-head chunks with at least 192 output tiles of 256 x 256 (one wave of
// workgroups over the CUs) run on the large-tile kernels.
bool head_big(int T, int width) { return cdiv(T, 256) * cdiv(width, 256) >= 192; }

int head_fwd(qls_session* S, const uint16_t* xL, int T, float* logp_out) {
  const Shape& sh = S->sh;
  const int d = sh.c.hidden, V = sh.c.vocab;
  hipStream_t st = S->cs;
  uint16_t* hf = S->at<uint16_t>(S->p.hf);
  rmsnorm_fwd(xL, S->res.d_final_norm, sh.c.rms_eps, hf, T, d, st);
  for (int c = 0; c < S->z.nchunks; ++c) {
    const int col0 = c * S->z.Vc, width = std::min(S->z.Vc, V - col0);
    GemmArgs g{};
    g.M = T; g.N = width; g.K = d;
    g.A = hf; g.lda = d;
    g.Bh = S->res.d_lm_head + (int64_t)col0 * d; g.ldb = d;
    g.tgt = S->at<int32_t>(S->p.tgt);
    g.stats = S->at<float>(S->p.stats); g.stats_ld = S->z.ntiles;
    g.tgt_logit = S->at<float>(S->p.tgt_logit); g.col0 = col0;
    if (head_big(T, width) && gemm_big_ok(g, B_BF16_NT, EPI_CE_STATS))
      QLS_RC(gemm_big_launch(g, B_BF16_NT, EPI_CE_STATS, st));
    else
      QLS_RC(gemm_launch(g, A_ROW, B_BF16_NT, EPI_CE_STATS, kTile, st));
  }
  ce_finalize(S->at<float>(S->p.stats), S->z.ntiles, S->at<float>(S->p.tgt_logit),
              S->at<int32_t>(S->p.tgt), T, S->at<float>(S->p.lse_t), logp_out, st);
  return QLS_OK;
}

// Pass 2: dlogits = w (softmax - onehot) chunk by chunk, dhf = sum_c dlogits_c W_c,
// then back through the final RMSNorm into g.
int head_bwd(qls_session* S, const uint16_t* xL, int T) {
  const Shape& sh = S->sh;
  const int d = sh.c.hidden, V = sh.c.vocab;
  hipStream_t st = S->cs;
  float* dhf = S->at<float>(S->p.dhf);
  uint16_t* dlog = S->at<uint16_t>(S->p.dlog);
  for (int c = 0; c < S->z.nchunks; ++c) {
    const int col0 = c * S->z.Vc, width = std::min(S->z.Vc, V - col0);
    GemmArgs g{};
    g.M = T; g.N = width; g.K = d;
    g.A = S->at<uint16_t>(S->p.hf); g.lda = d;
    g.Bh = S->res.d_lm_head + (int64_t)col0 * d; g.ldb = d;
    g.C = dlog; g.ldc = S->z.Vc;
    g.tgt = S->at<int32_t>(S->p.tgt); g.lse = S->at<float>(S->p.lse_t); g.roww = S->at<float>(S->p.roww);
    g.col0 = col0;
    if (head_big(T, width) && gemm_big_ok(g, B_BF16_NT, EPI_CE_GRAD))
      QLS_RC(gemm_big_launch(g, B_BF16_NT, EPI_CE_GRAD, st));
    else
      QLS_RC(gemm_launch(g, A_ROW, B_BF16_NT, EPI_CE_GRAD, kTile, st));
    GemmArgs h{};
    h.M = T; h.N = d; h.K = width;
    h.A = dlog; h.lda = S->z.Vc;
    h.Bh = S->res.d_lm_head + (int64_t)col0 * d; h.ldb = d;
    h.alpha = 1.f; h.C = dhf; h.ldc = d;
    h.partial = S->at<float>(S->p.part);
    const int epi = c == 0 ? EPI_F32 : EPI_F32_ACC;
    // dh on 256 x 256 tiles when the product fills the GPU (with split-K at
    // small T), under the same rule as the dequant-GEMMs.
    const GemmPlan pl = plan_nf4(T, d, width, true);
    h.ksplit = pl.ksplit;
    if (pl.big && gemm_big_ok(h, B_BF16_NN, epi)) {
      QLS_RC(gemm_big_launch(h, B_BF16_NN, epi, st));
    } else {
      h.ksplit = big_split(T, d, width);
      QLS_RC(gemm_launch(h, A_ROW, B_BF16_NN, epi, kTile, st));
    }
  }
  QLS_RC(rmsnorm_bwd(xL, S->res.d_final_norm, sh.c.rms_eps, dhf, nullptr, S->at<float>(S->p.g),
                     S->at<uint16_t>(S->p.dyb), T, d, st));
  return QLS_OK;
}

int check_tokens(qls_session* S, int B, int Sq) {
  if (B <= 0 || Sq < 2) return fail(QLS_EINVAL, "need B >= 1 and S >= 2");
  if (Sq > S->run.max_seq) return fail(QLS_EINVAL, "S exceeds max_seq");
  if ((int64_t)B * Sq > S->run.max_tokens) return fail(QLS_EINVAL, "B*S exceeds max_tokens");
  return QLS_OK;
}

// bf16 working copy of one layer's LoRA matrices, made just before the layer's
// first forward of a step (so all but layer 0's cast overlap the stream).
void cast_lora_layer(qls_session* S, const float* d_lora, int l) {
  const int64_t pl = S->ll.per_layer;
  lora_cast(d_lora + (int64_t)l * pl, pl, S->at<uint16_t>(S->p.lbf) + (int64_t)l * pl, pl, 1, S->seg, S->cs);
}

int begin_step(qls_session* S) {
  if (S->timing) {
    S->step_ev.push_back({S->next_ev(), S->next_ev()});
    QLS_HIP(hipEventRecord(S->step_ev.back().a, S->cs));
  }
  int rc = prefetch(S, 0, 1);
  if (!rc && S->sh.c.n_layers > 1) rc = prefetch(S, 1, 1);
  return rc;
}

// The embedding gather raises a device flag for a token id outside [0, vocab);
// it stays set until a call reports it.  Reads it after the compute stream
// has drained: QLS_EINVAL (and the flag cleared) when it was set.
int report_bad_ids(qls_session* S) {
  int bad = 0;
  QLS_HIP(hipMemcpy(&bad, S->at<int>(S->p.scal), sizeof(int), hipMemcpyDeviceToHost));
  if (!bad) return QLS_OK;
  QLS_HIP(hipMemset(S->at<int>(S->p.scal), 0, sizeof(int)));
  return fail(QLS_EINVAL, "token id outside [0, vocab) in a step since the last check");
}

int end_step(qls_session* S, float* h_loss, const float* d_loss) {
  S->steps += 1;
  if (S->timing) QLS_HIP(hipEventRecord(S->step_ev.back().b, S->cs));
  if (h_loss) {
    QLS_HIP(hipStreamSynchronize(S->cs));
    int rc = report_bad_ids(S);
    if (rc) return rc;
    if (d_loss) QLS_HIP(hipMemcpy(h_loss, d_loss, sizeof(float), hipMemcpyDeviceToHost));
  }
  return QLS_OK;
}

// Per-call bookkeeping before any launch: the workspace high-water mark and
// the capture buffer's size.
int begin_call(qls_session* S, int T, int Sq) {
  qls_run_cfg r = S->run;
  r.max_tokens = T;
  r.max_seq = Sq;
  S->peak_ws = std::max(S->peak_ws, make_plan(S->sh, S->lay, r, S->ll.per_layer * S->sh.c.n_layers).total);
  if (S->cap && S->cap_n < (int64_t)(S->sh.c.n_layers + 1) * T * S->sh.c.hidden)
    return fail(QLS_EINVAL, "gradient capture buffer smaller than (n_layers + 1) * tokens * hidden floats");
  return QLS_OK;
}

// Forward sweep; policy into the checkpoints, and (if ref) the adapters-disabled
// reference stream alongside on each resident layer.  d_lora (with lora):
// the float32 LoRA vector, cast layer by layer as the sweep reaches it.
int forward_sweep(qls_session* S, int T, int B, int Sq, bool lora, bool ref, const float* d_lora) {
  const int L = S->sh.c.n_layers;
  uint16_t* xr[2] = {S->at<uint16_t>(S->p.xref0), S->at<uint16_t>(S->p.xref1)};
  S->acts_layer = -1;
  S->acts0_saved = false;
  S->parts_next = true;
  for (int l = 0; l < L; ++l) {
    const uint8_t* rec;
    TimedEv te{};
    int rc = acquire(S, l, &rec, &te);
    if (rc) return rc;
    if (ref) {
      rc = fwd_layer(S, l, rec, xr[l & 1], xr[(l + 1) & 1], false, T, B, Sq);
      if (rc) return rc;
    }
    if (lora) cast_lora_layer(S, d_lora, l);
    rc = fwd_layer(S, l, rec, S->ck(l), S->ck(l + 1), lora, T, B, Sq);
    if (rc) return rc;
    S->acts_layer = lora ? l : -1;
    rc = release(S, l, &te);
    if (rc) return rc;
    if (l == 0 && lora && L > 1) {
      // Keep layer 0's intermediates for its backward, which closes the step
      // while the copy engine has nothing left to load; ordered after the
      // slot's release so the next copy is not held back.
      QLS_HIP(hipMemcpyAsync(S->at<uint8_t>(S->p.acts0), S->at<uint8_t>(S->p.n1), (size_t)(S->p.g - S->p.n1),
                             hipMemcpyDeviceToDevice, S->cs));
      S->acts0_saved = true;
    }
    if (l + 1 < L && S->slot_layer[(l + 1) & 1] != l + 1 && (rc = prefetch(S, l + 1, 1))) return rc;
  }
  S->parts_next = false;
  return QLS_OK;
}

// Test hook: copy the float32 residual gradient g = dL/dx_l into entry l of
// the capture buffer.
int capture(qls_session* S, int l, int T) {
  if (!S->cap) return QLS_OK;
  const int64_t n = (int64_t)T * S->sh.c.hidden;
  QLS_HIP(hipMemcpyAsync(S->cap + (int64_t)l * n, S->at<float>(S->p.g), (size_t)n * 4, hipMemcpyDeviceToDevice,
                         S->cs));
  return QLS_OK;
}

int backward_sweep(qls_session* S, int T, int B, int Sq, float* grads) {
  const int L = S->sh.c.n_layers;
  const bool shortcuts = !(S->dbg & QLS_DBG_RECOMPUTE_ALL);
  S->parts_next = true;
  for (int l = L - 1; l >= 0; --l) {
    const uint8_t* rec;
    TimedEv te{};
    int rc = acquire(S, l, &rec, &te);
    if (rc) return rc;
    // Recompute the layer's forward from its checkpoint, except at the two
    // ends of the sweep, where the copy engine idles: the last layer's
    // intermediates are still in the workspace at the turn, and layer 0's were
    // saved by the forward sweep (the same kernels would reproduce them bit
    // for bit).
    if (shortcuts && l == 0 && S->acts0_saved && l != S->acts_layer) {
      QLS_HIP(hipMemcpyAsync(S->at<uint8_t>(S->p.n1), S->at<uint8_t>(S->p.acts0), (size_t)(S->p.g - S->p.n1),
                             hipMemcpyDeviceToDevice, S->cs));
    } else if (!shortcuts || l != S->acts_layer) {
      rc = fwd_layer(S, l, rec, S->ck(l), S->at<uint16_t>(S->p.xo), true, T, B, Sq);
      if (rc) return rc;
    }
    S->acts_layer = -1;
    if (l == 0) S->acts0_saved = false;
    if ((rc = capture(S, l + 1, T))) return rc;
    rc = bwd_layer(S, l, rec, S->ck(l), grads, T, B, Sq);
    if (rc) return rc;
    if (l == 0 && (rc = capture(S, 0, T))) return rc;
    if (S->opt.on) {
      // Fused AdamW: layer l's gradients are final, update its slice now.
      const int64_t pl = S->ll.per_layer, o = (int64_t)l * pl;
      const FusedOpt& f = S->opt;
      adamw_update(f.p + o, grads + o, f.m + o, f.v + o, pl, f.t, f.lr, f.b1, f.b2, f.eps, f.wd, S->cs);
    }
    rc = release(S, l, &te);
    if (rc) return rc;
    if (l - 1 >= 0 && S->slot_layer[(l - 1) & 1] != l - 1 && (rc = prefetch(S, l - 1, -1))) return rc;
  }
  S->parts_next = false;
  return QLS_OK;
}

void fill_rope_table(const Shape& sh, int Smax, std::vector<float>* out) {
  const int h2 = sh.c.head_dim / 2;
  out->assign((size_t)Smax * h2 * 2, 0.f);
  for (int j = 0; j < h2; ++j) {
    const float inv = (float)std::pow((double)sh.c.rope_theta, -2.0 * j / sh.c.head_dim);
    for (int p = 0; p < Smax; ++p) {
      const float ang = (float)p * inv;
      (*out)[((size_t)p * h2 + j) * 2] = (float)std::cos((double)ang);
      (*out)[((size_t)p * h2 + j) * 2 + 1] = (float)std::sin((double)ang);
    }
  }
}

}  // namespace

// ================================================================ C ABI
extern "C" {

int qls_workspace_bytes(const qls_store* st, const qls_run_cfg* run, int64_t* out) {
  if (!st || !out) return fail(QLS_EINVAL, "NULL argument");
  const Shape& sh = store_shape(st);
  std::string why;
  if (!check_run(sh, run, &why)) return fail(QLS_EINVAL, why);
  *out = make_plan(sh, store_layout(st), *run, lora_layout(sh).per_layer * sh.c.n_layers).total;
  return QLS_OK;
}

int qls_session_create(const qls_store* st, const qls_run_cfg* run, void* d_ws, int64_t ws_bytes,
                       void* compute_stream, void* copy_stream, const qls_resident* res,
                       qls_session** out) {
  if (!out) return fail(QLS_EINVAL, "out is NULL");
  *out = nullptr;
  if (!st || !run || !d_ws || !res || !res->d_embed || !res->d_lm_head || !res->d_final_norm)
    return fail(QLS_EINVAL, "NULL argument");
  if (((uintptr_t)d_ws | (uintptr_t)res->d_embed | (uintptr_t)res->d_lm_head | (uintptr_t)res->d_final_norm) & 255)
    return fail(QLS_EINVAL, "workspace and resident tensors must be 256-byte aligned");
  const Shape& sh = store_shape(st);
  std::string why;
  if (!check_run(sh, run, &why)) return fail(QLS_EINVAL, why);
  int missing = -1;
  if (!store_complete(st, &missing))
    return fail(QLS_ESTATE, "store layer " + std::to_string(missing) + " was never set");
  auto* S = new (std::nothrow) qls_session;
  if (!S) return fail(QLS_ENOMEM, "host allocation failed");
  S->st = st;
  S->sh = sh;
  S->lay = store_layout(st);
  S->ll = lora_layout(sh);
  S->run = *run;
  S->z = sizes_of(sh, *run);
  const int64_t lora_numel = S->ll.per_layer * sh.c.n_layers;
  S->p = make_plan(sh, S->lay, *run, lora_numel);
  S->part_n = part_floats(sh, S->z.Tm);
  if (ws_bytes < S->p.total) {
    delete S;
    return fail(QLS_ENOMEM, "workspace of " + std::to_string(ws_bytes) + " bytes is smaller than the " +
                                std::to_string(S->p.total) + " this session needs");
  }
  S->ws = reinterpret_cast<uint8_t*>(d_ws);
  S->cs = (hipStream_t)compute_stream;
  S->ps = (hipStream_t)copy_stream;
  S->res = *res;
  S->timing = run->timing != 0;
  // bf16 working copy: A_q A_k A_v A_o A_gate A_up A_down, then the Bs in module order.
  const int r = sh.c.lora_r;
  int64_t off = 0;
  for (int m = 0; m < QLS_NMOD; ++m) { S->wa[m] = off; off += (int64_t)r * sh.mod[m].in; }
  for (int m = 0; m < QLS_NMOD; ++m) { S->wb[m] = off; off += (int64_t)sh.mod[m].out * r; }
  S->seg.nseg = 2 * QLS_NMOD;
  for (int m = 0; m < QLS_NMOD; ++m) {
    S->seg.so[2 * m] = S->ll.a_off[m]; S->seg.dof[2 * m] = S->wa[m]; S->seg.n[2 * m] = (int64_t)r * sh.mod[m].in;
    S->seg.so[2 * m + 1] = S->ll.b_off[m]; S->seg.dof[2 * m + 1] = S->wb[m]; S->seg.n[2 * m + 1] = (int64_t)sh.mod[m].out * r;
  }
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess && khz > 0)
    S->wall_khz = khz;
  auto cleanup = [&](int rc) { qls_session_destroy(S); return rc; };
  for (int i = 0; i < 2; ++i) {
    if (hipEventCreateWithFlags(&S->copied[i], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&S->released[i], hipEventDisableTiming) != hipSuccess)
      return cleanup(fail(QLS_EHIP, "hipEventCreate failed"));
    if (hipEventRecord(S->released[i], S->cs) != hipSuccess)
      return cleanup(fail(QLS_EHIP, "hipEventRecord failed"));
    for (int part = 0; part < PART_REST; ++part)
      if (hipEventCreateWithFlags(&S->part_rel[i][part], hipEventDisableTiming) != hipSuccess ||
          hipEventRecord(S->part_rel[i][part], S->cs) != hipSuccess)
        return cleanup(fail(QLS_EHIP, "hipEventCreate failed"));
  }
  if (hipMemset(S->at<int>(S->p.scal), 0, 64) != hipSuccess) return cleanup(fail(QLS_EHIP, "hipMemset failed"));
  std::vector<float> tab;
  fill_rope_table(sh, run->max_seq, &tab);
  hipError_t e = hipMemcpy(S->at<float>(S->p.rope), tab.data(), tab.size() * 4, hipMemcpyHostToDevice);
  if (e != hipSuccess) return cleanup(hip_fail(e, "rope table upload"));
  S->ram_layers = store_ram_layers(st);
  const DiskFile* df = store_disk(st);
  if (run->mode == QLS_STREAMED && S->ram_layers < sh.c.n_layers) {
    S->disk.reset(new (std::nothrow) DiskReader);
    if (!S->disk || S->disk->init(df, S->ram_layers, sh.c.n_layers, 3, &why))
      return cleanup(fail(QLS_ENOPIN, S->disk ? why : std::string("host allocation failed")));
  }
  if (run->mode == QLS_RESIDENT) {
    uint8_t* stage = nullptr;
    if (S->ram_layers < sh.c.n_layers) {
      e = hipHostMalloc(reinterpret_cast<void**>(&stage), (size_t)df->record_bytes(), hipHostMallocDefault);
      if (e != hipSuccess || !stage) return cleanup(hip_fail(e, "disk staging buffer"));
    }
    for (int l = 0; l < sh.c.n_layers && e == hipSuccess; ++l) {
      const uint8_t* src = store_record(st, l);
      if (!src) {
        const int rd = df->read_any(l - S->ram_layers, stage);
        if (rd) {
          (void)hipHostFree(stage);
          return cleanup(fail(QLS_EIO, std::string("disk tier read failed: ") + std::strerror(-rd)));
        }
        src = stage;
      }
      e = hipMemcpy(S->at<uint8_t>(S->p.slots) + (int64_t)l * S->lay.bytes, src, S->lay.bytes,
                    hipMemcpyHostToDevice);
    }
    if (stage) (void)hipHostFree(stage);
    if (e != hipSuccess) return cleanup(hip_fail(e, "resident store upload"));
  }
  *out = S;
  return QLS_OK;
}

void qls_session_destroy(qls_session* S) {
  if (!S) return;
  if (S->cs) (void)hipStreamSynchronize(S->cs);
  if (S->ps) (void)hipStreamSynchronize(S->ps);
  for (int i = 0; i < 2; ++i) {
    if (S->copied[i]) (void)hipEventDestroy(S->copied[i]);
    if (S->released[i]) (void)hipEventDestroy(S->released[i]);
    for (auto e : S->part_rel[i])
      if (e) (void)hipEventDestroy(e);
  }
  for (auto e : S->ev_pool) (void)hipEventDestroy(e);
  delete S;
}

int qls_sft_step(qls_session* S, const int32_t* d_ids, int B, int Sq, const float* d_lora,
                 float* d_grads, float* d_loss, float* h_loss) {
  if (!S || !d_ids || !d_lora || !d_grads || !d_loss) return fail(QLS_EINVAL, "NULL argument");
  int rc = check_tokens(S, B, Sq);
  if (rc) return rc;
  const int T = B * Sq;
  const Shape& sh = S->sh;
  if ((rc = begin_call(S, T, Sq)) || (rc = begin_step(S))) return rc;
  embed_gather(d_ids, S->res.d_embed, S->ck(0), T, sh.c.hidden, sh.c.vocab, S->at<int>(S->p.scal), S->cs);
  ce_targets(d_ids, B, Sq, S->at<int32_t>(S->p.tgt), S->cs);
  if ((rc = forward_sweep(S, T, B, Sq, true, false, d_lora))) return rc;
  const uint16_t* xL = S->ck(sh.c.n_layers);
  if ((rc = head_fwd(S, xL, T, S->at<float>(S->p.logp)))) return rc;
  sft_weights_loss(S->at<float>(S->p.logp), S->at<int32_t>(S->p.tgt), T, B * (Sq - 1),
                   S->at<float>(S->p.roww), d_loss, S->cs);
  if ((rc = head_bwd(S, xL, T))) return rc;
  if ((rc = backward_sweep(S, T, B, Sq, d_grads))) return rc;
  QLS_HIP(hipGetLastError());
  return end_step(S, h_loss, d_loss);
}

int qls_sft_step_adamw(qls_session* S, const int32_t* d_ids, int B, int Sq, float* d_lora, float* d_grads,
                       float* d_m, float* d_v, int step, double lr, double beta1, double beta2, double eps,
                       double weight_decay, float* d_loss, float* h_loss) {
  if (!S || !d_m || !d_v) return fail(QLS_EINVAL, "NULL argument");
  if (step < 1) return fail(QLS_EINVAL, "step must be >= 1");
  if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0) || !(eps > 0.0))
    return fail(QLS_EINVAL, "betas must be in [0, 1) and eps positive");
  S->opt.on = true;
  S->opt.p = d_lora; S->opt.m = d_m; S->opt.v = d_v; S->opt.t = step;
  S->opt.lr = lr; S->opt.b1 = beta1; S->opt.b2 = beta2; S->opt.eps = eps; S->opt.wd = weight_decay;
  const int rc = qls_sft_step(S, d_ids, B, Sq, d_lora, d_grads, d_loss, h_loss);
  S->opt.on = false;
  return rc;
}

int qls_logprobs(qls_session* S, const int32_t* d_ids, int B, int Sq, int prompt_len, const float* d_lora,
                 float* d_seq_logp, float* d_tok_logp) {
  if (!S || !d_ids || !d_seq_logp) return fail(QLS_EINVAL, "NULL argument");
  int rc = check_tokens(S, B, Sq);
  if (rc) return rc;
  if (prompt_len < 1 || prompt_len >= Sq) return fail(QLS_EINVAL, "prompt_len must be in [1, S)");
  const int T = B * Sq;
  const Shape& sh = S->sh;
  if ((rc = begin_call(S, T, Sq)) || (rc = begin_step(S))) return rc;

  embed_gather(d_ids, S->res.d_embed, S->ck(0), T, sh.c.hidden, sh.c.vocab, S->at<int>(S->p.scal), S->cs);
  ce_targets(d_ids, B, Sq, S->at<int32_t>(S->p.tgt), S->cs);
  if ((rc = forward_sweep(S, T, B, Sq, d_lora != nullptr, false, d_lora))) return rc;
  if ((rc = head_fwd(S, S->ck(sh.c.n_layers), T, S->at<float>(S->p.logp)))) return rc;
  seq_logp(S->at<float>(S->p.logp), B, Sq, prompt_len, d_seq_logp, d_tok_logp, S->cs);
  QLS_HIP(hipGetLastError());
  return end_step(S, nullptr, nullptr);
}

int qls_pref_step(qls_session* S, const qls_pref_cfg* cfg, const int32_t* d_chosen, const int32_t* d_rejected,
                  int Sq, int prompt_len, const float* d_lora, float* d_grads, float* d_loss, float* h_loss,
                  float* d_aux) {
  if (!S || !cfg || !d_chosen || !d_rejected || !d_lora || !d_grads || !d_loss)
    return fail(QLS_EINVAL, "NULL argument");
  if (cfg->kind < QLS_PREF_DPO || cfg->kind > QLS_PREF_KTO) return fail(QLS_EINVAL, "unknown preference kind");
  const float prm[5] = {cfg->beta, cfg->gamma, cfg->lambda, cfg->lambda_d, cfg->lambda_u};
  for (float x : prm)
    if (!std::isfinite(x)) return fail(QLS_EINVAL, "preference parameters must be finite");
  if (cfg->kind != QLS_PREF_ORPO && !(cfg->beta > 0.f)) return fail(QLS_EINVAL, "beta must be > 0");
  if (cfg->lambda < 0.f || cfg->lambda_d < 0.f || cfg->lambda_u < 0.f)
    return fail(QLS_EINVAL, "loss weights must be >= 0");
  int rc = check_tokens(S, 2, Sq);
  if (rc) return rc;
  if (prompt_len < 1 || prompt_len >= Sq) return fail(QLS_EINVAL, "prompt_len must be in [1, S)");
  const bool ref = cfg->kind == QLS_PREF_DPO || cfg->kind == QLS_PREF_KTO;
  const int B = 2, T = 2 * Sq;
  const Shape& sh = S->sh;
  const int d = sh.c.hidden;
  if ((rc = begin_call(S, T, Sq)) || (rc = begin_step(S))) return rc;
  int32_t* ids = S->at<int32_t>(S->p.ids);
  QLS_HIP(hipMemcpyAsync(ids, d_chosen, Sq * 4, hipMemcpyDeviceToDevice, S->cs));
  QLS_HIP(hipMemcpyAsync(ids + Sq, d_rejected, Sq * 4, hipMemcpyDeviceToDevice, S->cs));
  embed_gather(ids, S->res.d_embed, S->ck(0), T, d, sh.c.vocab, S->at<int>(S->p.scal), S->cs);
  if (ref)
    QLS_HIP(hipMemcpyAsync(S->at<uint16_t>(S->p.xref0), S->ck(0), (size_t)T * d * 2, hipMemcpyDeviceToDevice,
                           S->cs));
  ce_targets(ids, B, Sq, S->at<int32_t>(S->p.tgt), S->cs);
  if ((rc = forward_sweep(S, T, B, Sq, true, ref, d_lora))) return rc;
  const int L = sh.c.n_layers;
  if (ref) {
    const uint16_t* xref = S->at<uint16_t>(L & 1 ? S->p.xref1 : S->p.xref0);
    if ((rc = head_fwd(S, xref, T, S->at<float>(S->p.logp_ref)))) return rc;
  }
  const uint16_t* xL = S->ck(L);
  if ((rc = head_fwd(S, xL, T, S->at<float>(S->p.logp)))) return rc;
  PrefArgs a{cfg->kind, cfg->beta, cfg->gamma, cfg->lambda, cfg->lambda_d, cfg->lambda_u};
  pref_loss(a, S->at<float>(S->p.logp), ref ? S->at<float>(S->p.logp_ref) : nullptr, Sq, prompt_len,
            S->at<float>(S->p.roww), d_loss, d_aux, S->cs);
  if ((rc = head_bwd(S, xL, T))) return rc;
  if ((rc = backward_sweep(S, T, B, Sq, d_grads))) return rc;
  QLS_HIP(hipGetLastError());
  return end_step(S, h_loss, d_loss);
}

int qls_dpo_step(qls_session* S, const int32_t* d_chosen, const int32_t* d_rejected, int Sq, int prompt_len,
                 float beta, const float* d_lora, float* d_grads, float* d_loss, float* h_loss, float* d_aux) {
  qls_pref_cfg c{};
  c.kind = QLS_PREF_DPO;
  c.beta = beta;
  return qls_pref_step(S, &c, d_chosen, d_rejected, Sq, prompt_len, d_lora, d_grads, d_loss, h_loss, d_aux);
}

int qls_layer_fwd_bwd(qls_session* S, int layer, const uint16_t* d_x, const uint16_t* d_gout, int B, int Sq,
                      const float* d_lora, uint16_t* d_out, float* d_gin, float* d_grads) {
  if (!S || !d_x || !d_gout || !d_lora || !d_out || !d_gin || !d_grads) return fail(QLS_EINVAL, "NULL argument");
  if (layer < 0 || layer >= S->sh.c.n_layers) return fail(QLS_EINVAL, "layer out of range");
  int rc = check_tokens(S, B, Sq);
  if (rc) return rc;
  const int T = B * Sq, d = S->sh.c.hidden;
  if ((rc = begin_call(S, T, Sq))) return rc;
  if (S->timing) {
    S->step_ev.push_back({S->next_ev(), S->next_ev()});
    QLS_HIP(hipEventRecord(S->step_ev.back().a, S->cs));
  }
  if ((rc = prefetch(S, layer, 1))) return rc;
  cast_lora_layer(S, d_lora, layer);
  const uint8_t* rec;
  TimedEv te{};
  if ((rc = acquire(S, layer, &rec, &te))) return rc;
  if ((rc = fwd_layer(S, layer, rec, d_x, d_out, true, T, B, Sq))) return rc;
  if ((rc = fwd_layer(S, layer, rec, d_x, S->at<uint16_t>(S->p.xo), true, T, B, Sq))) return rc;
  bf16_to_f32(d_gout, S->at<float>(S->p.g), (int64_t)T * d, S->cs);
  QLS_HIP(hipMemcpyAsync(S->at<uint16_t>(S->p.dyb), d_gout, (size_t)T * d * 2, hipMemcpyDeviceToDevice, S->cs));
  if ((rc = bwd_layer(S, layer, rec, d_x, d_grads, T, B, Sq))) return rc;
  QLS_HIP(hipMemcpyAsync(d_gin, S->at<float>(S->p.g), (size_t)T * d * 4, hipMemcpyDeviceToDevice, S->cs));
  if ((rc = release(S, layer, &te))) return rc;
  QLS_HIP(hipGetLastError());
  return end_step(S, nullptr, nullptr);
}

int qls_session_checkpoints(qls_session* S, const uint16_t** d_ptr, int64_t* tokens) {
  if (!S || !d_ptr || !tokens) return fail(QLS_EINVAL, "NULL argument");
  *d_ptr = S->ck(0);
  *tokens = S->z.Tm;
  return QLS_OK;
}

int qls_session_stats(qls_session* S, qls_stats* o) {
  if (!S || !o) return fail(QLS_EINVAL, "NULL argument");
  QLS_HIP(hipStreamSynchronize(S->cs));
  QLS_HIP(hipStreamSynchronize(S->ps));
  std::memset(o, 0, sizeof(*o));
  o->steps = S->steps;
  o->layer_loads = S->loads;
  o->h2d_bytes = S->h2d;
  o->ws_bytes = S->p.total;
  o->peak_ws_bytes = S->peak_ws;
  if (S->disk) {
    const DiskReader::Stats d = S->disk->stats();
    o->disk_reads = d.reads;
    o->disk_bytes = d.bytes;
    o->disk_read_ms = d.read_ms;
    o->disk_wait_ms = d.wait_ms;
  }
  if (S->timing && !S->step_ev.empty()) {
    hipEvent_t t0 = S->step_ev.front().a;
    auto rel = [&](hipEvent_t e) { float ms = 0; (void)hipEventElapsedTime(&ms, t0, e); return (double)ms; };
    auto span = [&](hipEvent_t a, hipEvent_t b) { float ms = 0; (void)hipEventElapsedTime(&ms, a, b); return (double)ms; };
    std::vector<std::pair<double, double>> comp;
    for (auto& c : S->comp_ev) {
      comp.push_back({rel(c.a), rel(c.b)});
      o->compute_ms += comp.back().second - comp.back().first;
    }
    for (auto& c : S->copy_ev) {
      const double a = rel(c.a), b = rel(c.b);
      o->copy_ms += b - a;
      for (auto& k : comp) o->overlap_ms += std::max(0.0, std::min(b, k.second) - std::max(a, k.first));
    }
    for (auto& e : S->step_ev) o->step_ms += span(e.a, e.b);
    o->step_ms /= (double)S->step_ev.size();
    for (auto& k : S->kf_ev) {
      const double ms = span(k.a, k.b);
      o->dq_fwd_ms += ms; o->dq_fwd_gflop += k.gflop;
      const double red = k.c ? span(k.b, k.c) : 0.0;
      o->dq_fwd_reduce_ms += red;
      if (k.big) {
        o->dq_fwd_big_ms += ms; o->dq_fwd_big_gflop += k.gflop; ++o->dq_fwd_big_launches;
        o->dq_fwd_big_reduce_ms += red;
      }
    }
    for (auto& k : S->kd_ev) {
      const double ms = span(k.a, k.b);
      o->dq_dx_ms += ms; o->dq_dx_gflop += k.gflop;
      const double red = k.c ? span(k.b, k.c) : 0.0;
      o->dq_dx_reduce_ms += red;
      if (k.big) {
        o->dq_dx_big_ms += ms; o->dq_dx_big_gflop += k.gflop; ++o->dq_dx_big_launches;
        o->dq_dx_big_reduce_ms += red;
      }
    }
    o->dq_fwd_launches = (int64_t)S->kf_ev.size();
    o->dq_dx_launches = (int64_t)S->kd_ev.size();
    o->exposed_copy_ms = std::max(0.0, o->copy_ms - o->overlap_ms);
  }
  return report_bad_ids(S);
}

int qls_session_reset_stats(qls_session* S) {
  if (!S) return fail(QLS_EINVAL, "NULL argument");
  QLS_HIP(hipStreamSynchronize(S->cs));
  QLS_HIP(hipStreamSynchronize(S->ps));
  S->steps = S->loads = S->h2d = 0;
  S->peak_ws = 0;
  S->clear_timing();
  if (S->disk) S->disk->reset_stats();
  return QLS_OK;
}

int qls_debug_capture_grads(qls_session* S, float* d_buf, int64_t n_floats) {
  if (!S) return fail(QLS_EINVAL, "NULL argument");
  if (d_buf && n_floats <= 0) return fail(QLS_EINVAL, "n_floats must be positive");
  S->cap = d_buf;
  S->cap_n = d_buf ? n_floats : 0;
  return QLS_OK;
}

int qls_debug_set(qls_session* S, uint32_t flags, int delay_us) {
  if (!S) return fail(QLS_EINVAL, "NULL argument");
  if (delay_us < 0 || delay_us > 1000000) return fail(QLS_EINVAL, "delay_us must be in [0, 1e6]");
  S->dbg = flags;
  S->delay_us = delay_us;
  if (flags & (QLS_DBG_POISON_ON_RELEASE | QLS_DBG_NO_REUSE)) S->slot_layer[0] = S->slot_layer[1] = -1;
  return QLS_OK;
}

}  // extern "C"
