// Attention backward that allocates nothing, for callers that cannot call
// hipMalloc (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation).  It runs the kernels of qls_attention_bwd; their
// scratch (the D vector and the per-query-head dK / dV partials) lives in the
// fixed file-scope device array below instead of a caller workspace.  Each
// GPU the library runs on holds its own copy of the array, at its own
// address, until the process ends.  Every call on a GPU shares that GPU's
// copy: calls that overlap on one GPU race.  Every kernel writes the whole
// part of the scratch it reads, so nothing needs clearing between calls.
#include <mutex>
#include <string>
#include <vector>

#include "attn.h"
#include "internal.h"

static __device__ __align__(256) unsigned char scratch[QLS_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_mu;
std::vector<void*> g_scratch;   // device address of `scratch` per device (nullptr: not looked up yet)

// The device address of the current device's copy of `scratch`, looked up
// once per device with that device current.  The array's name in host code is
// only a host-side stand-in and is never passed to a kernel or a copy.
int scratch_address(void** out) {
  int dev = 0, n = 0;
  QLS_HIP(hipGetDevice(&dev));
  QLS_HIP(hipGetDeviceCount(&n));
  if (dev < 0 || dev >= n) return fail(QLS_EHIP, "current device out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  if ((int)g_scratch.size() < n) g_scratch.resize(n, nullptr);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    QLS_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(QLS_EHIP, "hipGetSymbolAddress returned a null scratch address");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return QLS_OK;
}

}  // namespace

extern "C" int qls_attention_bwd_noalloc(const uint16_t* d_qkv, const uint16_t* d_out, const uint16_t* d_dout,
                                         const float* d_lse, int B, int S, int H, int KV, int hd, float* d_dq,
                                         float* d_dk, float* d_dv, void* stream) {
  if (B <= 0 || S <= 0 || H <= 0 || hd <= 0) return fail(QLS_EINVAL, "sizes must be positive");
  const int64_t need = qls_attention_ws_bytes(B, S, H, hd);
  if (need > QLS_NOALLOC_SCRATCH_BYTES)
    return fail(QLS_EINVAL, "attention scratch of " + std::to_string(need) + " bytes exceeds the " +
                                std::to_string((int64_t)QLS_NOALLOC_SCRATCH_BYTES) +
                                "-byte fixed scratch of the allocation-free entry point");
  void* ws = nullptr;
  int rc = scratch_address(&ws);
  if (rc) return rc;
  return attention_bwd_run(d_qkv, d_out, d_dout, d_lse, B, S, H, KV, hd, d_dq, d_dk, d_dv, ws,
                           QLS_NOALLOC_SCRATCH_BYTES, (hipStream_t)stream);
}
