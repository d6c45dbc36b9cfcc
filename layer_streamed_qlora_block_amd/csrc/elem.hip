// Memory-bound layer kernels: RMSNorm, RoPE, SwiGLU, embedding gather, casts,
// cross-entropy reductions and the DPO head.  All are row- or element-parallel
// with 16-byte accesses where the layout allows; reductions use a fixed order
// so repeated runs give identical bits.
#include <cmath>

#include "common.h"
#include "ops.h"

namespace {

constexpr int TB = 256;

QLS_DEV float block_sum(float v, float* red) {
  v = warp_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i];
  return s;
}

// y = bf16(x * rho * w), rho = (mean(x^2) + eps)^-1/2, one block per row.
__global__ void __launch_bounds__(TB) rmsnorm_fwd_k(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ w, float eps,
                                                    uint16_t* __restrict__ y, int d) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + row * d);
  const int nc = d / 8;
  // The first kKeep chunks of each thread stay in registers for the second pass.
  constexpr int kKeep = 4;
  u32x4 keep[kKeep];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kKeep; ++i) {
    const int c = threadIdx.x + i * TB;
    keep[i] = c < nc ? xr[c] : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a = bflo(keep[i][q]), b = bfhi(keep[i][q]);
      ss += a * a + b * b;
    }
  }
  for (int c = threadIdx.x + kKeep * TB; c < nc; c += TB) {
    const u32x4 v = xr[c];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a = bflo(v[q]), b = bfhi(v[q]);
      ss += a * a + b * b;
    }
  }
  const float tot = block_sum(ss, red);
  const float rho = 1.f / sqrtf(tot / (float)d + eps);
  const u32x4* wr = reinterpret_cast<const u32x4*>(w);
  u32x4* yr = reinterpret_cast<u32x4*>(y + row * d);
  const auto put = [&](int c, const u32x4& v) {
    const u32x4 ww = wr[c];
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = pack2_bf16(bflo(v[q]) * rho * bflo(ww[q]), bfhi(v[q]) * rho * bfhi(ww[q]));
    yr[c] = o;
  };
#pragma unroll
  for (int i = 0; i < kKeep; ++i)
    if (threadIdx.x + i * TB < nc) put(threadIdx.x + i * TB, keep[i]);
  for (int c = threadIdx.x + kKeep * TB; c < nc; c += TB) put(c, xr[c]);
}

// out = gres + rho (dy*w - xhat * mean(dy*w*xhat)), xhat = rho x, one row per
// workgroup, for d <= 8 * TB * NC (d % 8 == 0): the thread's (up to NC)
// 8-wide chunks of x, dy, w (and gres) stay in registers across the three
// passes.
template <int NC>
__global__ void __launch_bounds__(TB) rmsnorm_bwd_vec_k(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ w, float eps,
                                                        const float* __restrict__ dy,
                                                        const float* gres, float* out,
                                                        uint16_t* __restrict__ out_bf16, int d) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int nc = d / 8;
  float xv[NC][8], dv[NC][8];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int c = threadIdx.x + k * TB;
#pragma unroll
    for (int e = 0; e < 8; ++e) { xv[k][e] = 0.f; dv[k][e] = 0.f; }
    if (c < nc) {
      const u32x4 xx = reinterpret_cast<const u32x4*>(x + row * d)[c];
      const u32x4 ww = reinterpret_cast<const u32x4*>(w)[c];
      const f32x4 d0 = reinterpret_cast<const f32x4*>(dy + row * d)[2 * c];
      const f32x4 d1 = reinterpret_cast<const f32x4*>(dy + row * d)[2 * c + 1];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xv[k][2 * q] = bflo(xx[q]);
        xv[k][2 * q + 1] = bfhi(xx[q]);
      }
      const float dd[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        dv[k][2 * q] = dd[2 * q] * bflo(ww[q]);          // dy * w
        dv[k][2 * q + 1] = dd[2 * q + 1] * bfhi(ww[q]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += xv[k][e] * xv[k][e];
    }
  }
  const float rho = 1.f / sqrtf(block_sum(ss, red) / (float)d + eps);
  float dot = 0.f;
#pragma unroll
  for (int k = 0; k < NC; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) dot += dv[k][e] * (xv[k][e] * rho);
  const float mean = block_sum(dot, red) / (float)d;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int c = threadIdx.x + k * TB;
    if (c >= nc) continue;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = rho * (dv[k][e] - xv[k][e] * rho * mean);
    if (gres) {
      const f32x4 g0 = reinterpret_cast<const f32x4*>(gres + row * d)[2 * c];
      const f32x4 g1 = reinterpret_cast<const f32x4*>(gres + row * d)[2 * c + 1];
      o[0] += g0.x; o[1] += g0.y; o[2] += g0.z; o[3] += g0.w;
      o[4] += g1.x; o[5] += g1.y; o[6] += g1.z; o[7] += g1.w;
    }
    reinterpret_cast<f32x4*>(out + row * d)[2 * c] = f32x4{o[0], o[1], o[2], o[3]};
    reinterpret_cast<f32x4*>(out + row * d)[2 * c + 1] = f32x4{o[4], o[5], o[6], o[7]};
    if (out_bf16)
      reinterpret_cast<u32x4*>(out_bf16 + row * d)[c] =
          u32x4{pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3]), pack2_bf16(o[4], o[5]), pack2_bf16(o[6], o[7])};
  }
}

// In-place rotate-half RoPE of the q and k heads of qkv; cs: [S][hd/2][2]
// (cos, sin).  Four consecutive pairs per thread (h2 % 4 == 0): 8-byte loads
// and stores of the bf16 halves and 16-byte loads of (cos, sin).
__global__ void rope_fwd4_k(uint16_t* __restrict__ qkv, int64_t ld, int T, int S, int nh_q, int nh_k, int hd,
                            const float* __restrict__ cs) {
  const int h2 = hd / 2, h8 = h2 / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_t = (int64_t)(nh_q + nh_k) * h8;
  if (idx >= (int64_t)T * per_t) return;
  const int t = (int)(idx / per_t);
  const int rem = (int)(idx % per_t);
  const int head = rem / h8, j = 4 * (rem % h8);
  const int pos = t % S;
  const f32x4 c01 = *reinterpret_cast<const f32x4*>(cs + ((int64_t)pos * h2 + j) * 2);
  const f32x4 c23 = *reinterpret_cast<const f32x4*>(cs + ((int64_t)pos * h2 + j + 2) * 2);
  const float c[4] = {c01.x, c01.z, c23.x, c23.z}, sn[4] = {c01.y, c01.w, c23.y, c23.w};
  uint16_t* p = qkv + (int64_t)t * ld + (int64_t)head * hd;
  const u32x2 a = *reinterpret_cast<const u32x2*>(p + j), b = *reinterpret_cast<const u32x2*>(p + j + h2);
  const float x1[4] = {bflo(a.x), bfhi(a.x), bflo(a.y), bfhi(a.y)};
  const float x2[4] = {bflo(b.x), bfhi(b.x), bflo(b.y), bfhi(b.y)};
  float y1[4], y2[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    y1[e] = x1[e] * c[e] - x2[e] * sn[e];
    y2[e] = x2[e] * c[e] + x1[e] * sn[e];
  }
  *reinterpret_cast<u32x2*>(p + j) = u32x2{pack2_bf16(y1[0], y1[1]), pack2_bf16(y1[2], y1[3])};
  *reinterpret_cast<u32x2*>(p + j + h2) = u32x2{pack2_bf16(y2[0], y2[1]), pack2_bf16(y2[2], y2[3])};
}

// RoPE backward into the bf16 dq | dk | dv rows of out (ld): dq = R^-1 dq',
// dk = R^-1 (sum of the kv head's query-head partials), dv = that sum for v,
// four consecutive pairs (or v elements) per thread.
__global__ void rope_bwd4_k(const float* __restrict__ dq, const float* __restrict__ dk,
                            const float* __restrict__ dv, uint16_t* __restrict__ out, int64_t ld,
                            int T, int S, int nh_q, int nh_k, int hd, const float* __restrict__ cs) {
  const int h2 = hd / 2, h8 = h2 / 4;
  const int qd = nh_q * hd, kvd = nh_k * hd;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_t = (int64_t)(nh_q + nh_k) * h8 + kvd / 4;
  if (idx >= (int64_t)T * per_t) return;
  const int t = (int)(idx / per_t);
  const int rem = (int)(idx % per_t);
  uint16_t* o = out + (int64_t)t * ld;
  const int grp = nh_q / nh_k;
  if (rem < (nh_q + nh_k) * h8) {
    const int head = rem / h8, j = 4 * (rem % h8);
    const int pos = t % S;
    const f32x4 c01 = *reinterpret_cast<const f32x4*>(cs + ((int64_t)pos * h2 + j) * 2);
    const f32x4 c23 = *reinterpret_cast<const f32x4*>(cs + ((int64_t)pos * h2 + j + 2) * 2);
    const float c[4] = {c01.x, c01.z, c23.x, c23.z}, sn[4] = {c01.y, c01.w, c23.y, c23.w};
    f32x4 x1, x2;
    if (head < nh_q) {
      const float* src = dq + (int64_t)t * qd + (int64_t)head * hd;
      x1 = *reinterpret_cast<const f32x4*>(src + j);
      x2 = *reinterpret_cast<const f32x4*>(src + j + h2);
    } else {                      // kv head: sum the query-head partials in order
      const float* src = dk + (int64_t)t * qd + (int64_t)(head - nh_q) * grp * hd;
      x1 = f32x4{0.f, 0.f, 0.f, 0.f};
      x2 = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int i = 0; i < grp; ++i) {
        x1 += *reinterpret_cast<const f32x4*>(src + i * hd + j);
        x2 += *reinterpret_cast<const f32x4*>(src + i * hd + j + h2);
      }
    }
    float y1[4], y2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y1[e] = x1[e] * c[e] + x2[e] * sn[e];
      y2[e] = x2[e] * c[e] - x1[e] * sn[e];
    }
    *reinterpret_cast<u32x2*>(o + (int64_t)head * hd + j) = u32x2{pack2_bf16(y1[0], y1[1]), pack2_bf16(y1[2], y1[3])};
    *reinterpret_cast<u32x2*>(o + (int64_t)head * hd + j + h2) =
        u32x2{pack2_bf16(y2[0], y2[1]), pack2_bf16(y2[2], y2[3])};
  } else {
    const int e = 4 * (rem - (nh_q + nh_k) * h8);      // element of the kv-width v row
    const int g = e / hd, j = e % hd;
    const float* src = dv + (int64_t)t * qd + (int64_t)g * grp * hd + j;
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < grp; ++i) v += *reinterpret_cast<const f32x4*>(src + i * hd);
    *reinterpret_cast<u32x2*>(o + qd + kvd + e) = u32x2{pack2_bf16(v.x, v.y), pack2_bf16(v.z, v.w)};
  }
}

// a = bf16(g sigmoid(g) u); gu rows hold g in [0, I) and u in [I, 2I).
__global__ void swiglu_fwd_k(const uint16_t* __restrict__ gu, uint16_t* __restrict__ a, int T, int I) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int i8 = I / 8;
  if (idx >= (int64_t)T * i8) return;
  const int t = (int)(idx / i8), c = (int)(idx % i8);
  const u32x4 g = reinterpret_cast<const u32x4*>(gu + (int64_t)t * 2 * I)[c];
  const u32x4 u = reinterpret_cast<const u32x4*>(gu + (int64_t)t * 2 * I + I)[c];
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float g0 = bflo(g[q]), g1 = bfhi(g[q]);
    const float s0 = 1.f / (1.f + __expf(-g0)), s1 = 1.f / (1.f + __expf(-g1));
    o[q] = pack2_bf16(g0 * s0 * bflo(u[q]), g1 * s1 * bfhi(u[q]));
  }
  reinterpret_cast<u32x4*>(a + (int64_t)t * I)[c] = o;
}

// x[t] = E[ids[t]]; an out-of-range id yields a zero row and sets *bad.
__global__ void embed_k(const int32_t* __restrict__ ids, const uint16_t* __restrict__ E,
                        uint16_t* __restrict__ x, int d, int V, int* bad) {
  const int t = blockIdx.x;
  const int id = ids[t];
  u32x4* dst = reinterpret_cast<u32x4*>(x + (int64_t)t * d);
  if (id < 0 || id >= V) {
    for (int c = threadIdx.x; c < d / 8; c += blockDim.x) dst[c] = u32x4{0, 0, 0, 0};
    if (threadIdx.x == 0 && bad) atomicOr(bad, 1);
    return;
  }
  const u32x4* src = reinterpret_cast<const u32x4*>(E + (int64_t)id * d);
  for (int c = threadIdx.x; c < d / 8; c += blockDim.x) dst[c] = src[c];
}

__global__ void f32_to_bf16_k(const float* __restrict__ x, uint16_t* __restrict__ y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = f2bf(x[i]);
}

__global__ void bf16_to_f32_k(const uint16_t* __restrict__ x, float* __restrict__ y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = bf2f(x[i]);
}

__global__ void lora_cast_k(const float* __restrict__ src, int64_t ss, uint16_t* __restrict__ dst,
                            int64_t ds, CastSeg seg) {
  const int j = blockIdx.y, l = blockIdx.z;
  const int64_t n = seg.n[j];
  const float* s = src + (int64_t)l * ss + seg.so[j];
  uint16_t* d = dst + (int64_t)l * ds + seg.dof[j];
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    d[i] = f2bf(s[i]);
}

__global__ void ce_targets_k(const int32_t* __restrict__ ids, int B, int S, int32_t* __restrict__ tgt) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * S) return;
  const int s = i % S;
  tgt[i] = s < S - 1 ? ids[i + 1] : -1;
}

// Per row: lse = log sum over the vocabulary tiles of sum_i exp(m_i) s_i; logp = tgt_logit - lse.
__global__ void ce_finalize_k(const float* __restrict__ stats, int ntiles,
                              const float* __restrict__ tgt_logit, const int32_t* __restrict__ tgt,
                              int T, float* __restrict__ lse, float* __restrict__ logp) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (row >= T) return;
  const float* st = stats + (int64_t)row * ntiles * 2;
  float m = -INFINITY;
  for (int i = l; i < ntiles; i += 64) m = fmaxf(m, st[2 * i]);
  m = warp_max(m);
  float s = 0.f;
  for (int i = l; i < ntiles; i += 64) s += st[2 * i + 1] * __expf(st[2 * i] - m);
  s = warp_sum(s);
  if (l == 0) {
    const float v = m + logf(s);
    lse[row] = v;
    logp[row] = tgt[row] >= 0 ? tgt_logit[row] - v : 0.f;
  }
}

// w_t = 1/N on rows with a target; loss = sum_t w_t (lse_t - tgt_logit_t), fixed-order sum.
__global__ void __launch_bounds__(TB) sft_loss_k(const float* __restrict__ logp,
                                                 const int32_t* __restrict__ tgt, int T, int N,
                                                 float* __restrict__ w, float* __restrict__ loss) {
  __shared__ float red[4];
  const float inv = 1.f / (float)N;
  float acc = 0.f;
  for (int t = threadIdx.x; t < T; t += TB) {
    const bool ok = tgt[t] >= 0;
    w[t] = ok ? inv : 0.f;
    acc += ok ? -logp[t] : 0.f;
  }
  const float s = block_sum(acc, red);
  if (threadIdx.x == 0) *loss = s * inv;
}

__global__ void __launch_bounds__(TB) seq_logp_k(const float* __restrict__ logp, int S, int P,
                                                 float* __restrict__ seq, float* __restrict__ tok) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  float acc = 0.f;
  for (int t = threadIdx.x; t < S; t += TB) {
    const float v = logp[(int64_t)b * S + t];
    if (tok) tok[(int64_t)b * S + t] = v;
    if (t >= P - 1 && t < S - 1) acc += v;
  }
  const float s = block_sum(acc, red);
  if (threadIdx.x == 0) seq[b] = s;
}

QLS_DEV double sigmoid_d(double a) {
  if (a >= 0) return 1.0 / (1.0 + exp(-a));
  const double e = exp(a);
  return e / (1.0 + e);
}
QLS_DEV double softplus_d(double a) { return fmax(a, 0.0) + log1p(exp(-fabs(a))); }

// Preference head on one pair (rows [0, S) chosen, [S, 2S) rejected), one
// block: sums the response log-likelihoods pi_x (and the reference rho_x when
// lr is set), evaluates the head in double precision and writes the row
// weights w_t = -dL/dpi_x on the response rows of sequence x (0 elsewhere).
//   DPO    z = beta((pi_c - rho_c) - (pi_r - rho_r)),      L = softplus(-z)
//   SimPO  z = beta pi_c / n - beta pi_r / n - gamma,       L = softplus(-z)
//   ORPO   l_x = pi_x / n, lo_x = l_x - log(1 - e^l_x),    L = -l_c + lam softplus(lo_r - lo_c)
//   KTO    r_x = pi_x - rho_x, z0 = max(0, (r_c + r_r)/2) held constant,
//          L = (lam_d (1 - sig(beta(r_c - z0))) + lam_u (1 - sig(beta(z0 - r_r)))) / 2
// with n = S - P response tokens per sequence.
__global__ void __launch_bounds__(TB) pref_k(const float* __restrict__ lp, const float* __restrict__ lr,
                                             int S, int P, PrefArgs a, float* __restrict__ w,
                                             float* __restrict__ loss, float* aux) {
  __shared__ float red[4];
  __shared__ float wsh[2];
  float v[4];
  for (int q = 0; q < 4; ++q) {
    const float* src = (q & 2) ? lr : lp;
    const int b = q & 1;
    float acc = 0.f;
    if (src)
      for (int t = threadIdx.x; t < S; t += TB)
        if (t >= P - 1 && t < S - 1) acc += src[(int64_t)b * S + t];
    v[q] = block_sum(acc, red);
  }
  // v = pi_c, pi_r, rho_c, rho_r
  if (threadIdx.x == 0) {
    const double pc = v[0], pr = v[1], rc = v[2], rr = v[3], n = (double)(S - P), beta = a.beta;
    double L = 0, gc = 0, gr = 0;
    if (a.kind == PREF_DPO || a.kind == PREF_SIMPO) {
      const double z = a.kind == PREF_DPO ? beta * ((pc - rc) - (pr - rr)) : beta * pc / n - beta * pr / n - a.gamma;
      const double sg = sigmoid_d(-z);
      L = softplus_d(-z);
      gc = -beta * sg;
      gr = beta * sg;
      if (a.kind == PREF_SIMPO) { gc /= n; gr /= n; }
    } else if (a.kind == PREF_ORPO) {
      const double lc = pc / n, lrn = pr / n;
      const double qc = -expm1(lc), qr = -expm1(lrn);       // 1 - p_x
      const double ratio = (lc - log(qc)) - (lrn - log(qr));
      const double sg = sigmoid_d(-ratio);
      L = -lc + a.lam * softplus_d(-ratio);
      gc = (-1.0 - a.lam * sg / qc) / n;
      gr = (a.lam * sg / qr) / n;
    } else {
      const double xc = pc - rc, xr = pr - rr;
      const double z0 = fmax(0.0, 0.5 * (xc + xr));
      const double su = sigmoid_d(beta * (xc - z0)), sv = sigmoid_d(beta * (z0 - xr));
      L = 0.5 * (a.lam_d * (1.0 - su) + a.lam_u * (1.0 - sv));
      gc = -0.5 * a.lam_d * beta * su * (1.0 - su);
      gr = 0.5 * a.lam_u * beta * sv * (1.0 - sv);
    }
    *loss = (float)L;
    wsh[0] = (float)(-gc);
    wsh[1] = (float)(-gr);
    if (aux) { aux[0] = v[0]; aux[1] = v[1]; aux[2] = v[2]; aux[3] = v[3]; }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < 2 * S; t += TB) {
    const int s = t % S;
    const bool resp = s >= P - 1 && s < S - 1;
    w[t] = resp ? wsh[t < S ? 0 : 1] : 0.f;
  }
}

// Bounded spin of `ticks` wall-clock ticks (at most 2^24 polls).
__global__ void spin_k(int64_t ticks) {
  const int64_t t0 = wall_clock64();
  for (int i = 0; i < (1 << 24); ++i) {
    if (wall_clock64() - t0 >= ticks) break;
    __builtin_amdgcn_s_sleep(2);
  }
}

}  // namespace

void rmsnorm_fwd(const uint16_t* x, const uint16_t* w, float eps, uint16_t* y, int T, int d,
                 hipStream_t st) {
  if (T <= 0) return;
  hipLaunchKernelGGL(rmsnorm_fwd_k, dim3(T), dim3(TB), 0, st, x, w, eps, y, d);
}
int rmsnorm_bwd(const uint16_t* x, const uint16_t* w, float eps, const float* dy, const float* gres,
                float* out, uint16_t* out_bf16, int T, int d, hipStream_t st) {
  if (T <= 0) return 0;
  const auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool vec = d % 8 == 0 && a16(x) && a16(w) && a16(dy) && a16(out) && (!gres || a16(gres)) &&
                   (!out_bf16 || a16(out_bf16));
  if (!vec || d > 8 * TB * 4) return -1;
  if (d <= 8 * TB * 2)
    hipLaunchKernelGGL(rmsnorm_bwd_vec_k<2>, dim3(T), dim3(TB), 0, st, x, w, eps, dy, gres, out, out_bf16, d);
  else
    hipLaunchKernelGGL(rmsnorm_bwd_vec_k<4>, dim3(T), dim3(TB), 0, st, x, w, eps, dy, gres, out, out_bf16, d);
  return 0;
}
int rope_fwd(uint16_t* qkv, int64_t ld, int T, int S, int H, int KV, int hd, const float* cs, hipStream_t st) {
  const int64_t n = (int64_t)T * (H + KV) * (hd / 2);
  if (n <= 0) return 0;
  if (hd % 8 || ld % 4 || (reinterpret_cast<uintptr_t>(qkv) & 7) || (reinterpret_cast<uintptr_t>(cs) & 15))
    return -1;
  hipLaunchKernelGGL(rope_fwd4_k, dim3((unsigned)ceil_div64(n / 4, 256)), dim3(256), 0, st, qkv, ld, T, S, H, KV,
                     hd, cs);
  return 0;
}
int rope_bwd(const float* dq, const float* dk, const float* dv, uint16_t* dqkv, int64_t ld, int T, int S, int H,
             int KV, int hd, const float* cs, hipStream_t st) {
  const int64_t n4 = (int64_t)T * ((H + KV) * (hd / 8) + KV * hd / 4);   // threads: 4 pairs or 4 v elements each
  if (n4 <= 0) return 0;
  if (hd % 8 || ld % 4 || (reinterpret_cast<uintptr_t>(dqkv) & 7) || (reinterpret_cast<uintptr_t>(cs) & 15) ||
      ((reinterpret_cast<uintptr_t>(dq) | reinterpret_cast<uintptr_t>(dk) | reinterpret_cast<uintptr_t>(dv)) & 15))
    return -1;
  hipLaunchKernelGGL(rope_bwd4_k, dim3((unsigned)ceil_div64(n4, 256)), dim3(256), 0, st, dq, dk, dv, dqkv, ld, T,
                     S, H, KV, hd, cs);
  return 0;
}
void swiglu_fwd(const uint16_t* gu, uint16_t* a, int T, int I, hipStream_t st) {
  const int64_t n = (int64_t)T * (I / 8);
  if (n <= 0) return;
  hipLaunchKernelGGL(swiglu_fwd_k, dim3((unsigned)ceil_div64(n, 256)), dim3(256), 0, st, gu, a, T, I);
}
void embed_gather(const int32_t* ids, const uint16_t* E, uint16_t* x, int T, int d, int V, int* bad,
                  hipStream_t st) {
  if (T <= 0) return;
  hipLaunchKernelGGL(embed_k, dim3(T), dim3(256), 0, st, ids, E, x, d, V, bad);
}
void f32_to_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t st) {
  if (n <= 0) return;
  hipLaunchKernelGGL(f32_to_bf16_k, dim3((unsigned)ceil_div64(n, 256)), dim3(256), 0, st, x, y, n);
}
void bf16_to_f32(const uint16_t* x, float* y, int64_t n, hipStream_t st) {
  if (n <= 0) return;
  hipLaunchKernelGGL(bf16_to_f32_k, dim3((unsigned)ceil_div64(n, 256)), dim3(256), 0, st, x, y, n);
}
void lora_cast(const float* src, int64_t ss, uint16_t* dst, int64_t ds, int L, const CastSeg& seg,
               hipStream_t st) {
  int64_t mx = 0;
  for (int j = 0; j < seg.nseg; ++j) mx = seg.n[j] > mx ? seg.n[j] : mx;
  const unsigned gx = (unsigned)(ceil_div64(mx, 256) < 1024 ? ceil_div64(mx, 256) : 1024);
  hipLaunchKernelGGL(lora_cast_k, dim3(gx, seg.nseg, L), dim3(256), 0, st, src, ss, dst, ds, seg);
}
void ce_targets(const int32_t* ids, int B, int S, int32_t* tgt, hipStream_t st) {
  hipLaunchKernelGGL(ce_targets_k, dim3(ceil_div(B * S, 256)), dim3(256), 0, st, ids, B, S, tgt);
}
void ce_finalize(const float* stats, int ntiles, const float* tgt_logit, const int32_t* tgt, int T,
                 float* lse, float* logp, hipStream_t st) {
  hipLaunchKernelGGL(ce_finalize_k, dim3(ceil_div(T, 4)), dim3(256), 0, st, stats, ntiles, tgt_logit,
                     tgt, T, lse, logp);
}
void sft_weights_loss(const float* logp, const int32_t* tgt, int T, int N, float* w, float* loss,
                      hipStream_t st) {
  hipLaunchKernelGGL(sft_loss_k, dim3(1), dim3(TB), 0, st, logp, tgt, T, N, w, loss);
}
void seq_logp(const float* logp, int B, int S, int prompt_len, float* seq, float* tok, hipStream_t st) {
  hipLaunchKernelGGL(seq_logp_k, dim3(B), dim3(TB), 0, st, logp, S, prompt_len, seq, tok);
}
void pref_loss(const PrefArgs& a, const float* logp_pol, const float* logp_ref, int S, int prompt_len,
               float* w, float* loss, float* aux, hipStream_t st) {
  hipLaunchKernelGGL(pref_k, dim3(1), dim3(TB), 0, st, logp_pol, logp_ref, S, prompt_len, a, w, loss, aux);
}
void spin_delay(int64_t ticks, hipStream_t st) {
  if (ticks <= 0) return;
  hipLaunchKernelGGL(spin_k, dim3(1), dim3(64), 0, st, ticks);
}
