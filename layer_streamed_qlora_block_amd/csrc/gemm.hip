// bf16 / NF4 GEMM family for gfx950: v_mfma_f32_32x32x16_bf16, fp32 accumulation.
//
// One kernel template covers every contraction on the step:
//   * the dequant-GEMM  Y = X W^T (+ s U B^T) (+ residual) with W NF4 [N, K]
//     dequantised tile by tile into LDS (bf16 = RNE(float32(cb[c] * absmax)));
//   * the transposed variant dX = dY W (+ du A) for the backward, where the
//     contraction runs over W's rows and the dequantised tile is transposed in
//     registers before it lands in LDS;
//   * the vocabulary-chunked LM-head products of the cross-entropy;
//   * the skinny LoRA products (U, du, dA, dB) with deterministic split-K.
//
// Tile: BM x BN output per 256-thread workgroup, 4 waves in a 2 x 2 grid, each
// wave (BM/2) x (BN/2) built from 32 x 32 MFMA blocks; BK = 64 (one NF4 block
// along a row when K % 64 == 0).  Global loads for tile k+1 are issued into
// registers before the MFMAs of tile k; LDS is double-buffered so one barrier
// per k-step suffices.  Rows of LDS are padded to 72 bf16 (144 B) so the
// 16-byte fragment reads of 16 consecutive rows hit distinct banks.
#include "common.h"
#include "gemm.h"

namespace {

constexpr int NT = 256;
constexpr int BK = 64;
constexpr int PITCH = BK + 8;

// ---------------------------------------------------------------- loaders
// Each loader moves one ROWS x BK operand tile: load() issues the global reads
// into registers, store() writes bf16 [ROWS][PITCH] into LDS (contraction
// contiguous, the layout the MFMA fragments read).

// bf16, contraction contiguous: element (row, k) at p[row * ld + k].  Rows
// outside [rlo, rows) and k >= K read as zero.  Needs K % 8 == 0, ld % 8 == 0.
template <int ROWS>
struct LdBf16Row {
  static constexpr int E = ROWS * BK / NT;
  static constexpr int TPR = BK / E;
  static constexpr int NV = E / 8;
  u32x4 v[NV];
  QLS_DEV void load(const uint16_t* p, int64_t ld, int rlo, int rows, int r0, int k0, int K) {
    const int t = threadIdx.x;
    const int gr = r0 + t / TPR;
    const int kk = k0 + (t % TPR) * E;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int kg = kk + 8 * j;
      if (gr >= rlo && gr < rows && kg < K)
        v[j] = *reinterpret_cast<const u32x4*>(p + (int64_t)gr * ld + kg);
      else
        v[j] = u32x4{0, 0, 0, 0};
    }
  }
  QLS_DEV void store(uint16_t* s) const {
    const int t = threadIdx.x;
    uint16_t* d = s + (t / TPR) * PITCH + (t % TPR) * E;
#pragma unroll
    for (int j = 0; j < NV; ++j) *reinterpret_cast<u32x4*>(d + 8 * j) = v[j];
  }
};

// bf16, tile rows contiguous: element (row, k) at p[k * ld + row].  Each thread
// reads 8 k-rows x R tile rows and transposes them in registers.  Needs the
// row count and ld to be multiples of 8.
template <int ROWS>
struct LdBf16Col {
  static constexpr int R = ROWS / 32;          // tile rows per thread (4 or 2)
  uint32_t w[8][R / 2];
  QLS_DEV void load(const uint16_t* p, int64_t ld, int rows, int r0, int k0, int K) {
    const int t = threadIdx.x;
    const int row = r0 + R * (t % 32);
    const int kb = k0 + 8 * (t / 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = kb + i;
      if (k < K && row < rows) {
        const uint16_t* src = p + (int64_t)k * ld + row;
        if constexpr (R == 4) {
          u32x2 x = *reinterpret_cast<const u32x2*>(src);
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
  }
  QLS_DEV void store(uint16_t* s) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int c = 0; c < R; ++c) {
      const int sh = 16 * (c & 1);
      u32x4 d;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = (w[2 * q][c >> 1] >> sh) & 0xFFFFu;
        const uint32_t hi = (w[2 * q + 1][c >> 1] >> sh) & 0xFFFFu;
        d[q] = lo | (hi << 16);
      }
      *reinterpret_cast<u32x4*>(s + (R * (t % 32) + c) * PITCH + 8 * (t / 32)) = d;
    }
  }
};

// NF4 nibble e (0..7) of a little-endian code word: element 2k sits in the
// high nibble of byte k.
QLS_DEV uint32_t nib(uint32_t w, int e) { return (w >> (8 * (e >> 1) + 4 * (1 - (e & 1)))) & 15u; }

// NF4, contraction contiguous: W flat element (row, k) = row * ldq + k.
// Needs ldq % 8 == 0 and K % 8 == 0 (8 codes per 32-bit word, one absmax).
template <int ROWS>
struct LdNf4Nt {
  static constexpr int E = ROWS * BK / NT;
  static constexpr int TPR = BK / E;
  static constexpr int NV = E / 8;
  uint32_t c[NV];
  float a[NV];
  QLS_DEV void load(const uint8_t* q, const float* sc, int64_t ldq, int rows, int r0, int k0, int K) {
    const int t = threadIdx.x;
    const int gr = r0 + t / TPR;
    const int kk = k0 + (t % TPR) * E;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int kg = kk + 8 * j;
      if (gr < rows && kg < K) {
        const int64_t f = (int64_t)gr * ldq + kg;
        c[j] = *reinterpret_cast<const uint32_t*>(q + (f >> 1));
        a[j] = sc[f >> 6];
      } else {
        c[j] = 0x77777777u;   // code 7 is the exact 0.0 level
        a[j] = 0.f;
      }
    }
  }
  QLS_DEV void store(uint16_t* s, const float* lut) const {
    const int t = threadIdx.x;
    uint16_t* d = s + (t / TPR) * PITCH + (t % TPR) * E;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = lut[nib(c[j], e)] * a[j];
      u32x4 o = {pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]), pack2_bf16(v[4], v[5]),
                 pack2_bf16(v[6], v[7])};
      *reinterpret_cast<u32x4*>(d + 8 * j) = o;
    }
  }
};

// NF4, tile rows contiguous: W flat element (k, row) = k * ldq + row (the
// contraction runs over W's rows).  Each thread dequantises KPT W-rows x 8
// W-columns and transposes them in registers.  Needs ldq % 8 == 0 and the
// row count % 8 == 0.
template <int ROWS>
struct LdNf4Nn {
  static constexpr int KPT = ROWS / 32;        // contraction rows per thread (4 or 2)
  static constexpr int RG = ROWS / 8;          // 8-column groups
  uint32_t c[KPT];
  float a[KPT];
  QLS_DEV void load(const uint8_t* q, const float* sc, int64_t ldq, int rows, int r0, int k0, int K) {
    const int t = threadIdx.x;
    const int col = r0 + 8 * (t % RG);
    const int kb = k0 + KPT * (t / RG);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int k = kb + i;
      if (k < K && col < rows) {
        const int64_t f = (int64_t)k * ldq + col;
        c[i] = *reinterpret_cast<const uint32_t*>(q + (f >> 1));
        a[i] = sc[f >> 6];
      } else {
        c[i] = 0x77777777u;
        a[i] = 0.f;
      }
    }
  }
  QLS_DEV void store(uint16_t* s, const float* lut) const {
    const int t = threadIdx.x;
    float v[KPT][8];
#pragma unroll
    for (int i = 0; i < KPT; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] = lut[nib(c[i], e)] * a[i];
    uint16_t* base = s + (8 * (t % RG)) * PITCH + KPT * (t / RG);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (KPT == 4) {
        u32x2 o = {pack2_bf16(v[0][e], v[1][e]), pack2_bf16(v[2][e], v[3][e])};
        *reinterpret_cast<u32x2*>(base + e * PITCH) = o;
      } else {
        *reinterpret_cast<uint32_t*>(base + e * PITCH) = pack2_bf16(v[0][e], v[1][e]);
      }
    }
  }
};

// ---------------------------------------------------------------- MFMA core
template <int BM, int BN>
QLS_DEV void mma_tile(const uint16_t* sA, const uint16_t* sB, f32x16 (&acc)[BM / 64][BN / 64],
                      int wm, int wn, int lane) {
  constexpr int MI = BM / 64, NI = BN / 64;
#pragma unroll
  for (int s = 0; s < BK / 16; ++s) {
    const int kofs = 16 * s + 8 * (lane >> 5);
    u32x4 a[MI], b[NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
      a[i] = *reinterpret_cast<const u32x4*>(sA + (wm * (BM / 2) + 32 * i + (lane & 31)) * PITCH + kofs);
#pragma unroll
    for (int j = 0; j < NI; ++j)
      b[j] = *reinterpret_cast<const u32x4*>(sB + (wn * (BN / 2) + 32 * j + (lane & 31)) * PITCH + kofs);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
  }
}

template <int ROWS, int BL>
struct BLoaderOf;
template <int ROWS> struct BLoaderOf<ROWS, B_BF16_NT> { using T = LdBf16Row<ROWS>; };
template <int ROWS> struct BLoaderOf<ROWS, B_BF16_NN> { using T = LdBf16Col<ROWS>; };
template <int ROWS> struct BLoaderOf<ROWS, B_NF4_NT> { using T = LdNf4Nt<ROWS>; };
template <int ROWS> struct BLoaderOf<ROWS, B_NF4_NN> { using T = LdNf4Nn<ROWS>; };

template <int ROWS, int AL>
struct ALoaderOf;
template <int ROWS> struct ALoaderOf<ROWS, A_ROW> { using T = LdBf16Row<ROWS>; };
template <int ROWS> struct ALoaderOf<ROWS, A_COL> { using T = LdBf16Col<ROWS>; };

template <int BM, int AL>
QLS_DEV void a_load(typename ALoaderOf<BM, AL>::T& la, const GemmArgs& g, int m0, int k0) {
  if constexpr (AL == A_ROW) la.load(g.A, g.lda, 0, g.M, m0, k0, g.K);
  else la.load(g.A, g.lda, g.M, m0, k0, g.K);
}
template <int BN, int BL>
QLS_DEV void b_load(typename BLoaderOf<BN, BL>::T& lb, const GemmArgs& g, int n0, int k0) {
  if constexpr (BL == B_BF16_NT) lb.load(g.Bh, g.ldb, 0, g.N, n0, k0, g.K);
  else if constexpr (BL == B_BF16_NN) lb.load(g.Bh, g.ldb, g.N, n0, k0, g.K);
  else lb.load(g.Bq, g.Bs, g.ldq, g.N, n0, k0, g.K);
}
template <int BN, int BL>
QLS_DEV void b_store(const typename BLoaderOf<BN, BL>::T& lb, uint16_t* s, const float* lut) {
  if constexpr (BL == B_NF4_NT || BL == B_NF4_NN) lb.store(s, lut);
  else lb.store(s);
}

QLS_DEV float sigmoidf_(float x) { return 1.f / (1.f + __expf(-x)); }

template <int BM, int BN, int AL, int BL, int EPI>
__global__ void __launch_bounds__(NT) gemm_kernel(GemmArgs g, const float* __restrict__ cb) {
  constexpr int MI = BM / 64, NI = BN / 64;
  constexpr int STAGE = (BM + BN) * PITCH;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];
  __shared__ float lut[16];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = (g.N + BN - 1) / BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  if constexpr (BL == B_NF4_NT || BL == B_NF4_NN) {
    if (t < 16) lut[t] = cb[t];
  }

  const int nk = (g.K + BK - 1) / BK;
  const int ks = g.ksplit > 0 ? g.ksplit : 1;
  const int kb = (int)((int64_t)nk * blockIdx.z / ks);
  const int ke = (int)((int64_t)nk * (blockIdx.z + 1) / ks);

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = f32x16{};

  typename ALoaderOf<BM, AL>::T la;
  typename BLoaderOf<BN, BL>::T lb;
  __syncthreads();
  if (kb < ke) {
    a_load<BM, AL>(la, g, m0, kb * BK);
    b_load<BN, BL>(lb, g, n0, kb * BK);
    la.store(smem);
    b_store<BN, BL>(lb, smem + BM * PITCH, lut);
    __syncthreads();
    for (int kt = kb; kt < ke; ++kt) {
      uint16_t* cur = smem + ((kt - kb) & 1) * STAGE;
      uint16_t* nxt = smem + (((kt - kb) & 1) ^ 1) * STAGE;
      const bool more = kt + 1 < ke;
      if (more) {
        a_load<BM, AL>(la, g, m0, (kt + 1) * BK);
        b_load<BN, BL>(lb, g, n0, (kt + 1) * BK);
      }
      mma_tile<BM, BN>(cur, cur + BM * PITCH, acc, wm, wn, lane);
      if (more) {
        la.store(nxt);
        b_store<BN, BL>(lb, nxt + BM * PITCH, lut);
      }
      __syncthreads();
    }
  }

  // ---- LoRA second contraction
  f32x16 acc2[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc2[i][j] = f32x16{};
  if constexpr (BL == B_NF4_NT && EPI == EPI_BF16) {
    if (g.lora == LORA_FWD) {
      // acc2 = U_g B_g^T over the modules g whose column range meets this tile;
      // columns of other modules read B as zero.
      int start = 0;
      for (int gi = 0; gi < g.nmod; ++gi) {
        const int end = g.mod_end[gi];
        if (end > n0 && start < n0 + BN) {
          const uint16_t* bp = g.modB[gi] - (int64_t)start * g.K2;
          for (int k0 = 0; k0 < g.K2; k0 += BK) {
            LdBf16Row<BM> ua;
            LdBf16Row<BN> ub;
            ua.load(g.A2 + gi * g.K2, g.lda2, 0, g.M, m0, k0, g.K2);
            ub.load(bp, g.K2, start, end, n0, k0, g.K2);
            ua.store(smem);
            ub.store(smem + BM * PITCH);
            __syncthreads();
            mma_tile<BM, BN>(smem, smem + BM * PITCH, acc2, wm, wn, lane);
            __syncthreads();
          }
        }
        start = end;
      }
    }
  }
  if constexpr (BL == B_NF4_NN) {
    if (g.lora == LORA_DX) {
      // acc += du_cat A_cat over the concatenated rank dimension.
      for (int k0 = 0; k0 < g.K2; k0 += BK) {
        LdBf16Row<BM> ua;
        LdBf16Col<BN> ub;
        ua.load(g.A2, g.lda2, 0, g.M, m0, k0, g.K2);
        ub.load(g.B2, g.ldb2, g.N, n0, k0, g.K2);
        ua.store(smem);
        ub.store(smem + BM * PITCH);
        __syncthreads();
        mma_tile<BM, BN>(smem, smem + BM * PITCH, acc, wm, wn, lane);
        __syncthreads();
      }
    }
  }

  // ---- epilogues
  if constexpr (EPI == EPI_CE_STATS) {
    // Stage the fp32 tile in LDS, then two threads per row reduce 64 columns each.
    constexpr int TP = BN + 4;
    float* sT = reinterpret_cast<float*>(smem);
    static_assert(BM * TP * 4 <= 2 * STAGE * 2, "tile does not fit");
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int mm = wm * (BM / 2) + 32 * i + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
          const int nn = wn * (BN / 2) + 32 * j + (lane & 31);
          sT[mm * TP + nn] = acc[i][j][q];
        }
    __syncthreads();
    const int row = t >> 1, half = t & 1;
    const int m = m0 + row;
    const int nvalid = min(BN, g.N - n0);
    const float* rp = sT + row * TP;
    float mx = -INFINITY;
    for (int c = half * (BN / 2); c < (half + 1) * (BN / 2); ++c)
      if (c < nvalid) mx = fmaxf(mx, rp[c]);
    mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
    float sm = 0.f;
    for (int c = half * (BN / 2); c < (half + 1) * (BN / 2); ++c)
      if (c < nvalid) sm += __expf(rp[c] - mx);
    sm += __shfl_xor(sm, 1, 64);
    if (half == 0 && m < g.M) {
      const int gt = (g.col0 + n0) / BN;
      g.stats[((int64_t)m * g.stats_ld + gt) * 2 + 0] = mx;
      g.stats[((int64_t)m * g.stats_ld + gt) * 2 + 1] = sm;
      const int tg = g.tgt[m] - g.col0 - n0;
      if (tg >= 0 && tg < nvalid) g.tgt_logit[m] = rp[tg];
    }
    return;
  } else {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int m = m0 + wm * (BM / 2) + 32 * i + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
          const int n = n0 + wn * (BN / 2) + 32 * j + (lane & 31);
          if (m >= g.M || n >= g.N) continue;
          const float v = acc[i][j][q];
          if constexpr (EPI == EPI_BF16) {
            float y = g.alpha * v;
            if constexpr (BL == B_NF4_NT) {
              if (g.lora == LORA_FWD) y += g.s2 * acc2[i][j][q];
            }
            if (g.R) y += bf2f(g.R[(int64_t)m * g.ldr + n]);
            reinterpret_cast<uint16_t*>(g.C)[(int64_t)m * g.ldc + n] = f2bf(y);
          } else if constexpr (EPI == EPI_F32) {
            reinterpret_cast<float*>(g.C)[(int64_t)m * g.ldc + n] = g.alpha * v;
          } else if constexpr (EPI == EPI_F32_ACC) {
            reinterpret_cast<float*>(g.C)[(int64_t)m * g.ldc + n] += g.alpha * v;
          } else if constexpr (EPI == EPI_PARTIAL) {
            g.partial[((int64_t)blockIdx.z * g.M + m) * g.N + n] = v;
          } else if constexpr (EPI == EPI_SWIGLU_BWD) {
            const float gg = bf2f(g.gu[(int64_t)m * g.ldgu + n]);
            const float uu = bf2f(g.gu[(int64_t)m * g.ldgu + g.I + n]);
            const float sg = sigmoidf_(gg);
            const float dg = v * uu * sg * (1.f + gg * (1.f - sg));
            const float du = v * (gg * sg);
            uint16_t* out = reinterpret_cast<uint16_t*>(g.C) + (int64_t)m * g.ldc;
            out[n] = f2bf(dg);
            out[g.I + n] = f2bf(du);
          } else if constexpr (EPI == EPI_CE_GRAD) {
            const float w = g.roww[m];
            float d = 0.f;
            if (w != 0.f) {
              d = __expf(v - g.lse[m]);
              if (g.tgt[m] == g.col0 + n) d -= 1.f;
              d *= w;
            }
            reinterpret_cast<uint16_t*>(g.C)[(int64_t)m * g.ldc + n] = f2bf(d);
          }
        }
  }
}

__global__ void reduce_kernel(const float* __restrict__ P, int ks, int M, int N, float alpha,
                              int mode, void* C, int64_t ldc) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t MN = (int64_t)M * N;
  if (idx >= MN) return;
  const int m = (int)(idx / N), n = (int)(idx % N);
  float s = 0.f;
  for (int z = 0; z < ks; ++z) s += P[z * MN + idx];
  if (mode == 0) reinterpret_cast<uint16_t*>(C)[(int64_t)m * ldc + n] = f2bf(alpha * s);
  else reinterpret_cast<float*>(C)[(int64_t)m * ldc + n] = alpha * s;
}

template <int BM, int BN, int AL, int BL, int EPI>
void launch_t(const GemmArgs& g, const float* cb, hipStream_t st) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  const int ks = g.ksplit > 0 ? g.ksplit : 1;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, AL, BL, EPI>), dim3(tiles, 1, ks), dim3(NT), 0, st, g, cb);
}

}  // namespace

const float* nf4_codebook_dev();  // defined in nf4.hip

int gemm_launch(const GemmArgs& g, int aload, int bload, int epi, int tile, hipStream_t st) {
  const float* cb = (bload == B_NF4_NT || bload == B_NF4_NN) ? nf4_codebook_dev() : nullptr;
#define QLS_CASE(BMV, AL, BL, EP)                                           \
  if (tile == BMV && aload == AL && bload == BL && epi == EP) {             \
    launch_t<BMV, BMV, AL, BL, EP>(g, cb, st);                              \
    return 0;                                                               \
  }
  QLS_CASE(128, A_ROW, B_NF4_NT, EPI_BF16)
  QLS_CASE(128, A_ROW, B_NF4_NN, EPI_F32)
  QLS_CASE(128, A_ROW, B_NF4_NN, EPI_BF16)
  QLS_CASE(128, A_ROW, B_NF4_NN, EPI_SWIGLU_BWD)
  QLS_CASE(128, A_ROW, B_BF16_NT, EPI_CE_STATS)
  QLS_CASE(128, A_ROW, B_BF16_NT, EPI_CE_GRAD)
  QLS_CASE(128, A_ROW, B_BF16_NN, EPI_F32)
  QLS_CASE(128, A_ROW, B_BF16_NN, EPI_F32_ACC)
  QLS_CASE(64, A_ROW, B_BF16_NT, EPI_PARTIAL)
  QLS_CASE(64, A_ROW, B_BF16_NN, EPI_PARTIAL)
  QLS_CASE(64, A_COL, B_BF16_NN, EPI_PARTIAL)
#undef QLS_CASE
  return -1;  // combination not instantiated
}

void gemm_reduce(const float* partial, int ksplit, int M, int N, float alpha, int mode, void* C,
                 int64_t ldc, hipStream_t st) {
  const int64_t MN = (int64_t)M * N;
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)ceil_div64(MN, 256)), dim3(256), 0, st, partial,
                     ksplit, M, N, alpha, mode, C, ldc);
}

int64_t gemm_partial_elems(int M, int N, int ksplit) { return (int64_t)M * N * ksplit; }
