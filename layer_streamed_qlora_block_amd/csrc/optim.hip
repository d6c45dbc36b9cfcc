// AdamW on the packed float32 LoRA vector: the training loop around the
// streamed step (the pages train at lr 2e-5 and compare 20 streamed with 20
// resident steps; page "Fine-Tune an 8B Model on a 4GB Laptop GPU: Hands-On
// Guide", section "The gotchas nobody's mentioning yet").
//
// Built with floating-point contraction off, so each multiply and add rounds
// on its own in the order stated in the header, and the result equals the
// oracle's float32 update bit for bit.
#include <cmath>

#include "common.h"
#include "ops.h"

namespace {

// Correctly rounded float32 square root: the hardware estimate is within one
// ulp, so the neighbour whose square brackets x is chosen with exact fused
// residuals x - s' * s (the refinement LLVM uses for IEEE sqrt on AMDGPU).
// Inputs below 2^-96 are scaled by 2^32 first (exact) so the residuals stay
// normal numbers.
__device__ __forceinline__ float sqrt_rn(float x) {
  if (!(x > 0.f) || __builtin_isinf(x)) return __builtin_amdgcn_sqrtf(x);   // 0, < 0, inf, NaN
  const bool small = x < 0x1p-96f;
  const float xs = small ? x * 0x1p32f : x;
  const float s = __builtin_amdgcn_sqrtf(xs);
  const float dn = __uint_as_float(__float_as_uint(s) - 1u);
  const float up = __uint_as_float(__float_as_uint(s) + 1u);
  const float rd = __builtin_fmaf(-dn, s, xs);
  const float ru = __builtin_fmaf(-up, s, xs);
  float r = s;
  if (rd <= 0.f) r = dn;
  if (ru > 0.f) r = up;
  return small ? r * 0x1p-16f : r;
}

// AdamW on the float32 LoRA vector, one element per thread, every operation
// rounded on its own (no contraction) in the order the oracle states.
struct AdamWArgs {
  float* p; const float* g; float* m; float* v; int64_t n;
  float decay, b1, omb1, b2, omb2, step_size, inv_sqrt_bc2, eps;
};
__global__ void __launch_bounds__(256) adamw_k(AdamWArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.n) return;
  const float g = a.g[i];
  const float p1 = __fmul_rn(a.p[i], a.decay);
  const float m1 = __fadd_rn(__fmul_rn(a.b1, a.m[i]), __fmul_rn(a.omb1, g));
  const float v1 = __fadd_rn(__fmul_rn(a.b2, a.v[i]), __fmul_rn(a.omb2, __fmul_rn(g, g)));
  const float denom = __fadd_rn(__fmul_rn(sqrt_rn(v1), a.inv_sqrt_bc2), a.eps);
  a.p[i] = __fsub_rn(p1, __fmul_rn(a.step_size, __fdiv_rn(m1, denom)));
  a.m[i] = m1;
  a.v[i] = v1;
}

}  // namespace

void adamw_update(float* p, const float* g, float* m, float* v, int64_t n, int t, double lr, double b1,
                  double b2, double eps, double wd, hipStream_t st) {
  if (n <= 0) return;
  // Every constant is formed in double from the double hyper-parameters and
  // rounded once to float32.
  AdamWArgs a{p, g, m, v, n};
  a.decay = (float)(1.0 - lr * wd);
  a.b1 = (float)b1;
  a.omb1 = (float)(1.0 - b1);
  a.b2 = (float)b2;
  a.omb2 = (float)(1.0 - b2);
  a.step_size = (float)(lr / (1.0 - std::pow(b1, t)));
  a.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(1.0 - std::pow(b2, t)));
  a.eps = (float)eps;
  hipLaunchKernelGGL(adamw_k, dim3((unsigned)ceil_div64(n, 256)), dim3(256), 0, st, a);
}
