// NF4 codebook (host) and the device dequantiser.
//
// The frozen store is NF4 (page "Can You Fine-Tune Llama 3.1 8B on a 4GB GPU?
// ...", section "Why NF4 matters so much").  The 16 levels follow QLoRA's
// NormalFloat construction: with delta = (1/30 + 1/32) / 2 and p_hi = 1 - delta,
// 8 positive levels Phi^-1(p) for p equally spaced from p_hi down to 1/2 (9
// points, the last dropped), 7 negative levels -Phi^-1(p) for 8 points from
// p_hi to 1/2 (last dropped), and 0; all divided by Phi^-1(p_hi).  Phi^-1 is
// evaluated here by bisection + Newton on the double-precision erfc.
#include <cmath>
#include <mutex>

#include "common.h"
#include "internal.h"

namespace {

double norm_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

double norm_ppf(double p) {
  double lo = -12.0, hi = 12.0;
  for (int i = 0; i < 200; ++i) {
    const double mid = 0.5 * (lo + hi);
    if (norm_cdf(mid) < p) lo = mid;
    else hi = mid;
  }
  double x = 0.5 * (lo + hi);
  const double inv_sqrt_2pi = 0.39894228040143267794;
  for (int i = 0; i < 2; ++i) {
    const double d = inv_sqrt_2pi * std::exp(-0.5 * x * x);
    if (d <= 0) break;
    x -= (norm_cdf(x) - p) / d;
  }
  return x;
}

__global__ void __launch_bounds__(256) nf4_dequant_kernel(const uint32_t* __restrict__ codes,
                                                          const float* __restrict__ absmax,
                                                          int64_t n8, u32x4* __restrict__ out,
                                                          const float* __restrict__ cb) {
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = cb[threadIdx.x];
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const uint32_t c = codes[i];
  const float a = absmax[i >> 3];
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = lut[(c >> (8 * (e >> 1) + 4 * (1 - (e & 1)))) & 15u] * a;
  out[i] = u32x4{pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]), pack2_bf16(v[4], v[5]),
                 pack2_bf16(v[6], v[7])};
}

// Double-quantised absmax decode: out[i] = float32(q8[i] * s[group]), one
// IEEE float32 multiply.  The layer form walks the seven modules of a record:
// the 8-bit codes and the expanded floats are back to back over the layer, the
// group scales restart their 256-block grouping at each module.
struct ExpandArgs {
  const uint8_t* q8;             // the layer's 8-bit codes (module order, back to back)
  const float* scales;           // the layer's group scales (module order, back to back)
  int64_t block_start[QLS_NMOD + 1];
  int64_t scale_start[QLS_NMOD];
  float* out;
};

__global__ void __launch_bounds__(256) absmax_expand_kernel(ExpandArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.block_start[QLS_NMOD]) return;
  int m = 0;
#pragma unroll
  for (int j = 1; j < QLS_NMOD; ++j) m += i >= a.block_start[j];
  const int64_t local = i - a.block_start[m];
  a.out[i] = (float)a.q8[i] * a.scales[a.scale_start[m] + local / 256];
}

std::once_flag g_cb_once;
float* g_cb_dev = nullptr;
int g_cb_err = 0;

}  // namespace

void nf4_codebook_host(float out[16]) {
  const double delta = 0.5 * (1.0 / 30.0 + 1.0 / 32.0);
  const double p_hi = 1.0 - delta;
  const double top = norm_ppf(p_hi);
  double v[16];
  int n = 0;
  for (int j = 0; j < 7; ++j) v[n++] = -norm_ppf(p_hi - j * (p_hi - 0.5) / 7.0) / top;
  v[n++] = 0.0;
  for (int i = 7; i >= 0; --i) v[n++] = norm_ppf(p_hi - i * (p_hi - 0.5) / 8.0) / top;
  // ascending by construction: -1 ... 0 ... +1
  for (int i = 0; i < 16; ++i) out[i] = (float)v[i];
}

// Device copy of the codebook, created once per process on the current device.
const float* nf4_codebook_dev() {
  std::call_once(g_cb_once, [] {
    float h[16];
    nf4_codebook_host(h);
    if (hipMalloc(&g_cb_dev, 16 * sizeof(float)) != hipSuccess) {
      g_cb_err = 1;
      g_cb_dev = nullptr;
      return;
    }
    if (hipMemcpy(g_cb_dev, h, sizeof(h), hipMemcpyHostToDevice) != hipSuccess) g_cb_err = 1;
  });
  return g_cb_err ? nullptr : g_cb_dev;
}

int nf4_dequant_launch(const uint8_t* codes, const float* absmax, int64_t n, uint16_t* out,
                       hipStream_t st) {
  const float* cb = nf4_codebook_dev();
  if (!cb) return -1;
  const int64_t n8 = n / 8;
  if (n8 == 0) return 0;
  hipLaunchKernelGGL(nf4_dequant_kernel, dim3((unsigned)ceil_div64(n8, 256)), dim3(256), 0, st,
                     reinterpret_cast<const uint32_t*>(codes), absmax, n8,
                     reinterpret_cast<u32x4*>(out), cb);
  return 0;
}

int absmax_expand_launch(const uint8_t* rec, const RecordLayout& lay, float* out, hipStream_t st) {
  ExpandArgs a{};
  a.q8 = rec + lay.q8_off[0];
  a.scales = reinterpret_cast<const float*>(rec + lay.scale_off[0]);
  for (int m = 0; m <= QLS_NMOD; ++m) a.block_start[m] = lay.block_start[m];
  for (int m = 0; m < QLS_NMOD; ++m) a.scale_start[m] = lay.scale_start[m];
  a.out = out;
  if (lay.nblocks == 0) return 0;
  hipLaunchKernelGGL(absmax_expand_kernel, dim3((unsigned)ceil_div64(lay.nblocks, 256)), dim3(256), 0, st, a);
  return 0;
}

int absmax_expand_flat_launch(const uint8_t* q8, const float* scales, int64_t nb, float* out,
                              hipStream_t st) {
  ExpandArgs a{};
  a.q8 = q8;
  a.scales = scales;
  for (int m = 1; m <= QLS_NMOD; ++m) a.block_start[m] = nb;   // one module holds everything
  a.out = out;
  if (nb == 0) return 0;
  hipLaunchKernelGGL(absmax_expand_kernel, dim3((unsigned)ceil_div64(nb, 256)), dim3(256), 0, st, a);
  return 0;
}
