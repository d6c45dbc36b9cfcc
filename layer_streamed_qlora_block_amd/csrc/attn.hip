// Causal grouped-query attention for gfx950 with v_mfma_f32_16x16x32_bf16.
//
// Forward: one workgroup per (64 query rows, query head, sequence); each of
// the 4 waves owns 16 query rows and walks the key blocks up to the diagonal
// with an online softmax (running max / sum in fp32).  Scores are formed
// transposed, S^T = K Q^T, so a lane's accumulator column is its query row:
// the softmax statistics stay per lane and the probabilities feed the P V
// product directly as the B operand (the contraction slots of a lane are the
// keys it already holds).  P is rounded to bf16 for the product; the final
// division by the fp32 row sum follows it.  The log-sum-exp per row is saved.
//
// Backward (no atomics, fixed summation order):
//   dq kernel  -- per (64 query rows, head): recompute P from the saved LSE,
//                 dP^T = V dO^T, dS = P (dP - D), dQ = dS K / sqrt(hd).
//   dkv kernel -- per (64 keys, query head): loops over the query blocks on
//                 or below the diagonal, dV_h += P^T dO, dK_h += dS^T Q /
//                 sqrt(hd), one float partial per query head; the sum over the
//                 heads that share a kv head is taken in head order by the
//                 RoPE-backward kernel that consumes dK and dV.
//   D = rowsum(dO o) comes from a small preprocessing kernel.
#include "common.h"
#include "attn.h"

namespace {

constexpr int NT = 256;
constexpr int BQ = 64;                 // query rows / keys per block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// rows [r0, r0+64) x HD from base[row * ld + j] into s[64][HD + 8]; rows >= S read 0.
template <int HD>
QLS_DEV void stage_rows(uint16_t* s, const uint16_t* base, int64_t ld, int r0, int S) {
  constexpr int CH = HD / 8;
  for (int c = threadIdx.x; c < BQ * CH; c += NT) {
    const int row = c / CH, c8 = c % CH;
    u32x4 v = {0, 0, 0, 0};
    if (r0 + row < S) v = *reinterpret_cast<const u32x4*>(base + (int64_t)(r0 + row) * ld + 8 * c8);
    *reinterpret_cast<u32x4*>(s + row * (HD + 8) + 8 * c8) = v;
  }
}

// transposed: s[j][row] (pitch 72) = element (row, j); each thread moves
// 8 rows x R columns and transposes them in registers.  Column group jg and
// row group kg are interleaved so that each 8 / 16 consecutive lanes write 16
// distinct bank quads (a plain jg = t % 32 mapping puts four of them on one).
template <int HD>
QLS_DEV void stage_cols(uint16_t* s, const uint16_t* base, int64_t ld, int r0, int S) {
  constexpr int R = HD / 32;
  static_assert(HD / R == 32, "32 column groups");
  const int t = threadIdx.x;
  const int jg = ((t >> 2) & 3) | (((t >> 4) & 7) << 2);   // 0..31
  const int kg = (t & 3) | ((t >> 7) << 2);                // 0..7
  uint32_t w[8][R / 2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = r0 + 8 * kg + i;
    if (row < S) {
      const uint16_t* src = base + (int64_t)row * ld + R * jg;
      if constexpr (R == 4) {
        const u32x2 x = *reinterpret_cast<const u32x2*>(src);
        w[i][0] = x.x;
        w[i][1] = x.y;
      } else {
        w[i][0] = *reinterpret_cast<const uint32_t*>(src);
      }
    } else {
#pragma unroll
      for (int c = 0; c < R / 2; ++c) w[i][c] = 0;
    }
  }
#pragma unroll
  for (int c = 0; c < R; ++c) {
    const int sh = 16 * (c & 1);
    u32x4 d;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      d[q] = ((w[2 * q][c >> 1] >> sh) & 0xFFFFu) | (((w[2 * q + 1][c >> 1] >> sh) & 0xFFFFu) << 16);
    *reinterpret_cast<u32x4*>(s + (R * jg + c) * (BQ + 8) + 8 * kg) = d;
  }
}

// 8 bf16 contraction slots {base+4g..+3, base+16+4g..+3} of row `row` of a
// transposed tile (pitch 72): matches the key/query order of a 16x16 C block pair.
QLS_DEV u32x4 read_pair(const uint16_t* s, int row, int base, int g4) {
  const u32x2 a = *reinterpret_cast<const u32x2*>(s + row * (BQ + 8) + base + 4 * g4);
  const u32x2 b = *reinterpret_cast<const u32x2*>(s + row * (BQ + 8) + base + 16 + 4 * g4);
  return u32x4{a.x, a.y, b.x, b.y};
}

QLS_DEV u32x4 pack8(const f32x4& a, const f32x4& b) {
  return u32x4{pack2_bf16(a[0], a[1]), pack2_bf16(a[2], a[3]), pack2_bf16(b[0], b[1]),
               pack2_bf16(b[2], b[3])};
}

template <int HD>
__global__ void __launch_bounds__(NT) attn_fwd_k(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[BQ * (HD + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[HD * (BQ + 8)];
  const int nqb = (a.S + BQ - 1) / BQ;
  const int qb = nqb - 1 - (int)blockIdx.x;       // long rows first
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = h / (a.H / a.KV);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, g4 = lane >> 4, c16 = lane & 15;
  const int q0 = qb * BQ;
  const int myq = q0 + 16 * w + c16;
  const int64_t tb = (int64_t)b * a.S;
  const uint16_t* Q = a.qkv + tb * a.ld + a.q_off + (int64_t)h * HD;
  const uint16_t* K = a.qkv + tb * a.ld + a.k_off + (int64_t)g * HD;
  const uint16_t* V = a.qkv + tb * a.ld + a.v_off + (int64_t)g * HD;

  u32x4 qf[HD / 32];
#pragma unroll
  for (int s = 0; s < HD / 32; ++s)
    qf[s] = myq < a.S ? *reinterpret_cast<const u32x4*>(Q + (int64_t)myq * a.ld + 32 * s + 8 * g4)
                      : u32x4{0, 0, 0, 0};
  f32x4 o[HD / 16];
#pragma unroll
  for (int i = 0; i < HD / 16; ++i) o[i] = f32x4{0, 0, 0, 0};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.scale * kLog2e;

  for (int kb = 0; kb <= qb; ++kb) {
    const int k0 = kb * BQ;
    stage_rows<HD>(sK, K, a.ld, k0, a.S);
    stage_cols<HD>(sVt, V, a.ld, k0, a.S);
    __syncthreads();
    f32x4 sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[j] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < HD / 32; ++s) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(sK + (16 * j + c16) * (HD + 8) + 32 * s + 8 * g4);
        sc[j] = mfma16(ka, qf[s], sc[j]);
      }
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + 16 * j + 4 * g4 + i;
        const float x = (key <= myq && key < a.S) ? sc[j][i] * c : -INFINITY;
        sc[j][i] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(sc[j][i] - m_use);
        sc[j][i] = p;
        ls += p;
      }
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < HD / 16; ++i) o[i] *= alpha;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const u32x4 pf = pack8(sc[2 * tt], sc[2 * tt + 1]);
#pragma unroll
      for (int hb = 0; hb < HD / 16; ++hb) {
        const u32x4 va = read_pair(sVt, 16 * hb + c16, 32 * tt, g4);
        o[hb] = mfma16(va, pf, o[hb]);
      }
    }
    __syncthreads();
  }
  float lt = l_run + __shfl_xor(l_run, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  if (myq < a.S) {
    const float inv = 1.f / lt;
    uint16_t* O = a.out + (tb + myq) * a.ldo + (int64_t)h * HD;
#pragma unroll
    for (int hb = 0; hb < HD / 16; ++hb) {
      const u32x2 v = {pack2_bf16(o[hb][0] * inv, o[hb][1] * inv), pack2_bf16(o[hb][2] * inv, o[hb][3] * inv)};
      *reinterpret_cast<u32x2*>(O + 16 * hb + 4 * g4) = v;
    }
    if (g4 == 0) a.lse[((int64_t)b * a.H + h) * a.S + myq] = m_run * kLn2 + logf(lt);
  }
}

// D[b,h,q] = sum_j dO[q, h, j] * O[q, h, j]; one wave per (row, head).
template <int HD>
__global__ void attn_pre_k(const uint16_t* __restrict__ dO, const uint16_t* __restrict__ O,
                           int64_t ld, int S, int H, int T, float* __restrict__ D) {
  const int64_t wid = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (wid >= (int64_t)T * H) return;
  const int tok = (int)(wid / H), h = (int)(wid % H);
  float acc = 0.f;
  for (int j = lane; j < HD; j += 64)
    acc += bf2f(dO[(int64_t)tok * ld + h * HD + j]) * bf2f(O[(int64_t)tok * ld + h * HD + j]);
  acc = warp_sum(acc);
  if (lane == 0) {
    const int b = tok / S, s = tok % S;
    D[((int64_t)b * H + h) * S + s] = acc;
  }
}

template <int HD>
__global__ void __launch_bounds__(NT) attn_dq_k(AttnBwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[BQ * (HD + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t sV[BQ * (HD + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t sKt[HD * (BQ + 8)];
  const int nqb = (a.S + BQ - 1) / BQ;
  const int qb = nqb - 1 - (int)blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = h / (a.H / a.KV);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, g4 = lane >> 4, c16 = lane & 15;
  const int q0 = qb * BQ;
  const int myq = q0 + 16 * w + c16;
  const int64_t tb = (int64_t)b * a.S;
  const uint16_t* Q = a.qkv + tb * a.ld + a.q_off + (int64_t)h * HD;
  const uint16_t* K = a.qkv + tb * a.ld + a.k_off + (int64_t)g * HD;
  const uint16_t* V = a.qkv + tb * a.ld + a.v_off + (int64_t)g * HD;
  const uint16_t* dO = a.dO + tb * a.lddo + (int64_t)h * HD;

  u32x4 qf[HD / 32], df[HD / 32];
#pragma unroll
  for (int s = 0; s < HD / 32; ++s) {
    const bool ok = myq < a.S;
    qf[s] = ok ? *reinterpret_cast<const u32x4*>(Q + (int64_t)myq * a.ld + 32 * s + 8 * g4) : u32x4{0, 0, 0, 0};
    df[s] = ok ? *reinterpret_cast<const u32x4*>(dO + (int64_t)myq * a.lddo + 32 * s + 8 * g4) : u32x4{0, 0, 0, 0};
  }
  const int64_t row_id = ((int64_t)b * a.H + h) * a.S + myq;
  const float lse2 = myq < a.S ? a.lse[row_id] * kLog2e : 0.f;
  const float Dq = myq < a.S ? a.D[row_id] : 0.f;
  const float c = a.scale * kLog2e;
  f32x4 dq[HD / 16];
#pragma unroll
  for (int i = 0; i < HD / 16; ++i) dq[i] = f32x4{0, 0, 0, 0};

  for (int kb = 0; kb <= qb; ++kb) {
    const int k0 = kb * BQ;
    stage_rows<HD>(sK, K, a.ld, k0, a.S);
    stage_rows<HD>(sV, V, a.ld, k0, a.S);
    stage_cols<HD>(sKt, K, a.ld, k0, a.S);
    __syncthreads();
    f32x4 sc[4], dp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[j] = f32x4{0, 0, 0, 0};
      dp[j] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < HD / 32; ++s) {
        const int off = (16 * j + c16) * (HD + 8) + 32 * s + 8 * g4;
        sc[j] = mfma16(*reinterpret_cast<const u32x4*>(sK + off), qf[s], sc[j]);
        dp[j] = mfma16(*reinterpret_cast<const u32x4*>(sV + off), df[s], dp[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + 16 * j + 4 * g4 + i;
        const float p = (key <= myq && key < a.S && myq < a.S) ? exp2f(sc[j][i] * c - lse2) : 0.f;
        sc[j][i] = p * (dp[j][i] - Dq);     // dS (rounded to bf16 below)
      }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const u32x4 dsf = pack8(sc[2 * tt], sc[2 * tt + 1]);
#pragma unroll
      for (int hb = 0; hb < HD / 16; ++hb)
        dq[hb] = mfma16(dsf, read_pair(sKt, 16 * hb + c16, 32 * tt, g4), dq[hb]);
    }
    __syncthreads();
  }
  // dq[hb][i] = dQ[q0 + 16w + 4 g4 + i][16 hb + c16]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = q0 + 16 * w + 4 * g4 + i;
    if (q >= a.S) continue;
    float* dst = a.dq + (tb + q) * a.lddq + (int64_t)h * HD;
#pragma unroll
    for (int hb = 0; hb < HD / 16; ++hb) dst[16 * hb + c16] = dq[hb][i] * a.scale;
  }
}

template <int HD>
__global__ void __launch_bounds__(NT) attn_dkv_k(AttnBwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sQ[BQ * (HD + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[BQ * (HD + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t sQt[HD * (BQ + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t sdOt[HD * (BQ + 8)];
  __shared__ float sL[BQ], sD[BQ];
  const int nqb = (a.S + BQ - 1) / BQ;
  const int kb = (int)blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = h / (a.H / a.KV);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, g4 = lane >> 4, c16 = lane & 15;
  const int k0 = kb * BQ;
  const int myk = k0 + 16 * w + c16;
  const int64_t tb = (int64_t)b * a.S;
  const uint16_t* K = a.qkv + tb * a.ld + a.k_off + (int64_t)g * HD;
  const uint16_t* V = a.qkv + tb * a.ld + a.v_off + (int64_t)g * HD;
  u32x4 kf[HD / 32], vf[HD / 32];
#pragma unroll
  for (int s = 0; s < HD / 32; ++s) {
    const bool ok = myk < a.S;
    kf[s] = ok ? *reinterpret_cast<const u32x4*>(K + (int64_t)myk * a.ld + 32 * s + 8 * g4) : u32x4{0, 0, 0, 0};
    vf[s] = ok ? *reinterpret_cast<const u32x4*>(V + (int64_t)myk * a.ld + 32 * s + 8 * g4) : u32x4{0, 0, 0, 0};
  }
  const float c = a.scale * kLog2e;
  f32x4 dk[HD / 16], dv[HD / 16];
#pragma unroll
  for (int i = 0; i < HD / 16; ++i) { dk[i] = f32x4{0, 0, 0, 0}; dv[i] = f32x4{0, 0, 0, 0}; }

  {
    const uint16_t* Q = a.qkv + tb * a.ld + a.q_off + (int64_t)h * HD;
    const uint16_t* dO = a.dO + tb * a.lddo + (int64_t)h * HD;
    for (int qb = kb; qb < nqb; ++qb) {
      const int q0 = qb * BQ;
      stage_rows<HD>(sQ, Q, a.ld, q0, a.S);
      stage_rows<HD>(sdO, dO, a.lddo, q0, a.S);
      stage_cols<HD>(sQt, Q, a.ld, q0, a.S);
      stage_cols<HD>(sdOt, dO, a.lddo, q0, a.S);
      if (t < BQ) {
        const int q = q0 + t;
        const int64_t rid = ((int64_t)b * a.H + h) * a.S + q;
        sL[t] = q < a.S ? a.lse[rid] * kLog2e : 0.f;
        sD[t] = q < a.S ? a.D[rid] : 0.f;
      }
      __syncthreads();
      f32x4 sc[4], dp[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sc[j] = f32x4{0, 0, 0, 0};
        dp[j] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < HD / 32; ++s) {
          const int off = (16 * j + c16) * (HD + 8) + 32 * s + 8 * g4;
          sc[j] = mfma16(*reinterpret_cast<const u32x4*>(sQ + off), kf[s], sc[j]);
          dp[j] = mfma16(*reinterpret_cast<const u32x4*>(sdO + off), vf[s], dp[j]);
        }
      }
      // sc[j][i] = S[q = q0 + 16j + 4g4 + i][key = myk]
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ql = 16 * j + 4 * g4 + i;
          const int q = q0 + ql;
          const float p = (myk <= q && q < a.S && myk < a.S) ? exp2f(sc[j][i] * c - sL[ql]) : 0.f;
          sc[j][i] = p;
          dp[j][i] = p * (dp[j][i] - sD[ql]);
        }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const u32x4 pf = pack8(sc[2 * tt], sc[2 * tt + 1]);
        const u32x4 dsf = pack8(dp[2 * tt], dp[2 * tt + 1]);
#pragma unroll
        for (int hb = 0; hb < HD / 16; ++hb) {
          dv[hb] = mfma16(pf, read_pair(sdOt, 16 * hb + c16, 32 * tt, g4), dv[hb]);
          dk[hb] = mfma16(dsf, read_pair(sQt, 16 * hb + c16, 32 * tt, g4), dk[hb]);
        }
      }
      __syncthreads();
    }
  }
  // dk[hb][i] = this query head's share of dK[key = k0 + 16w + 4g4 + i][16hb + c16]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = k0 + 16 * w + 4 * g4 + i;
    if (key >= a.S) continue;
    float* dkr = a.dk + (tb + key) * a.lddkv + (int64_t)h * HD;
    float* dvr = a.dv + (tb + key) * a.lddkv + (int64_t)h * HD;
#pragma unroll
    for (int hb = 0; hb < HD / 16; ++hb) {
      dkr[16 * hb + c16] = dk[hb][i] * a.scale;
      dvr[16 * hb + c16] = dv[hb][i];
    }
  }
}

}  // namespace

int attn_fwd(const AttnArgs& a, int B, hipStream_t st) {
  const dim3 grid((a.S + BQ - 1) / BQ, a.H, B);
  if (a.hd == 128) hipLaunchKernelGGL(attn_fwd_k<128>, grid, dim3(NT), 0, st, a);
  else if (a.hd == 64) hipLaunchKernelGGL(attn_fwd_k<64>, grid, dim3(NT), 0, st, a);
  else return -1;
  return 0;
}

int attn_bwd(const AttnBwdArgs& a, int B, hipStream_t st) {
  const int T = B * a.S;
  const int64_t waves = (int64_t)T * a.H;
  const dim3 gq((a.S + BQ - 1) / BQ, a.H, B), gk((a.S + BQ - 1) / BQ, a.H, B);
  if (a.hd == 128) {
    hipLaunchKernelGGL(attn_pre_k<128>, dim3((unsigned)ceil_div64(waves * 64, 256)), dim3(256), 0, st,
                       a.dO, a.O, a.lddo, a.S, a.H, T, a.D);
    hipLaunchKernelGGL(attn_dq_k<128>, gq, dim3(NT), 0, st, a);
    hipLaunchKernelGGL(attn_dkv_k<128>, gk, dim3(NT), 0, st, a);
  } else if (a.hd == 64) {
    hipLaunchKernelGGL(attn_pre_k<64>, dim3((unsigned)ceil_div64(waves * 64, 256)), dim3(256), 0, st,
                       a.dO, a.O, a.lddo, a.S, a.H, T, a.D);
    hipLaunchKernelGGL(attn_dq_k<64>, gq, dim3(NT), 0, st, a);
    hipLaunchKernelGGL(attn_dkv_k<64>, gk, dim3(NT), 0, st, a);
  } else {
    return -1;
  }
  return 0;
}
