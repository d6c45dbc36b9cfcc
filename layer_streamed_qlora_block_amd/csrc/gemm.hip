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
// along a row when K % 64 == 0).  Global loads run two k-tiles ahead through
// two register stages; LDS is double-buffered so one barrier per k-step
// suffices.  Rows of LDS are padded to 72 bf16 (144 B) so the 16-byte fragment
// reads of 16 consecutive rows hit distinct banks.  The LoRA term is
// contracted first into the same accumulator (scaled by s), then the base
// product accumulates on top, so one accumulator set serves both and the
// kernel keeps two waves per SIMD.  Large-M dequant-GEMMs use the 256 x 256
// kernels of gemm_big.hip instead.
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
  QLS_DEV void store(uint16_t* s, const float* lut) const;
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
  QLS_DEV void store(uint16_t* s, const float* lut) const;
};

// ---------------------------------------------------------------- fast loaders
// Used when the shape is aligned (see fast_ok): raw buffer loads through a
// resource whose size ends at the last valid element, so the hardware range
// check returns zero past the edge without per-element masking; each thread's
// offset inside the tile is computed once and the k-step advance goes through
// the scalar offset operand.
QLS_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}
QLS_DEV u32x4 bld128(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, v, s, 0));
}
QLS_DEV u32x2 bld64(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, v, s, 0));
}
QLS_DEV uint32_t bld32(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, v, s, 0);
}

// Eight NF4 codes of a word -> eight float32 cb[c] * a.  The LUT byte offsets
// 4*nibble are cut out of the word with two shifts and masks for all eight.
QLS_DEV void deq8(uint32_t c, float a, const float* lut, float v[8]) {
  const uint32_t hi4 = (c >> 2) & 0x3C3C3C3Cu;   // elements 0, 2, 4, 6 (high nibbles)
  const uint32_t lo4 = (c << 2) & 0x3C3C3C3Cu;   // elements 1, 3, 5, 7 (low nibbles)
  const char* lb = reinterpret_cast<const char*>(lut);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    v[2 * b] = *reinterpret_cast<const float*>(lb + ((hi4 >> (8 * b)) & 0xFFu)) * a;
    v[2 * b + 1] = *reinterpret_cast<const float*>(lb + ((lo4 >> (8 * b)) & 0xFFu)) * a;
  }
}

// bf16, contraction contiguous (K % 64 == 0); rows >= `rows` read zero.
template <int ROWS>
struct FBf16Row {
  static constexpr int E = ROWS * BK / NT;
  static constexpr int TPR = BK / E;
  static constexpr int NV = E / 8;
  __amdgpu_buffer_rsrc_t r;
  uint32_t voff;
  u32x4 v[NV];
  QLS_DEV void init(const uint16_t* p, int64_t ld, int rows, int r0) {
    r = make_rsrc(p + (int64_t)r0 * ld, (int64_t)(rows - r0) * ld * 2);
    const int t = threadIdx.x;
    voff = (uint32_t)(((t / TPR) * ld + (t % TPR) * E) * 2);
  }
  QLS_DEV void load(int k0) {
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] = bld128(r, voff + 16 * j, (uint32_t)k0 * 2);
  }
  QLS_DEV void store(uint16_t* s) const {
    const int t = threadIdx.x;
    uint16_t* d = s + (t / TPR) * PITCH + (t % TPR) * E;
#pragma unroll
    for (int j = 0; j < NV; ++j) *reinterpret_cast<u32x4*>(d + 8 * j) = v[j];
  }
};

// bf16, tile rows contiguous (element (row, k) at p[k * ld + row]); every
// tile row valid; k >= K reads zero.
template <int ROWS>
struct FBf16Col {
  static constexpr int R = ROWS / 32;
  __amdgpu_buffer_rsrc_t r;
  uint32_t voff;
  int ld;
  uint32_t w[8][R / 2];
  QLS_DEV void init(const uint16_t* p, int64_t ld_, int K, int r0) {
    r = make_rsrc(p + r0, ((int64_t)K * ld_ - r0) * 2);
    ld = (int)ld_;
    const int t = threadIdx.x;
    voff = (uint32_t)((8 * (t / 32) * ld_ + R * (t % 32)) * 2);
  }
  QLS_DEV void load(int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t so = (uint32_t)(k0 + i) * (uint32_t)ld * 2;
      if constexpr (R == 4) {
        const u32x2 x = bld64(r, voff, so);
        w[i][0] = x.x;
        w[i][1] = x.y;
      } else {
        w[i][0] = bld32(r, voff, so);
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
      for (int q = 0; q < 4; ++q)
        d[q] = ((w[2 * q][c >> 1] >> sh) & 0xFFFFu) | (((w[2 * q + 1][c >> 1] >> sh) & 0xFFFFu) << 16);
      *reinterpret_cast<u32x4*>(s + (R * (t % 32) + c) * PITCH + 8 * (t / 32)) = d;
    }
  }
};

// NF4, contraction contiguous (K % 64 == 0, ldq % 64 == 0): a thread's E
// codes are consecutive in one row and share one absmax.
template <int ROWS>
struct FNf4Nt {
  static constexpr int E = ROWS * BK / NT;
  static constexpr int TPR = BK / E;
  static constexpr int NV = E / 8;
  __amdgpu_buffer_rsrc_t rq, rs;
  uint32_t vq, vs;
  uint32_t c[NV];
  float a;
  QLS_DEV void init(const uint8_t* q, const float* sc, int64_t ldq, int rows, int r0) {
    rq = make_rsrc(q + (int64_t)r0 * ldq / 2, (int64_t)(rows - r0) * ldq / 2);
    rs = make_rsrc(sc + (int64_t)r0 * (ldq / 64), (int64_t)(rows - r0) * (ldq / 64) * 4);
    const int t = threadIdx.x;
    vq = (uint32_t)(((t / TPR) * ldq + (t % TPR) * E) / 2);
    vs = (uint32_t)((t / TPR) * (ldq / 64) * 4);
  }
  QLS_DEV void load(int k0) {
    if constexpr (NV == 4) {
      const u32x4 x = bld128(rq, vq, (uint32_t)k0 / 2);
      c[0] = x.x; c[1] = x.y; c[2] = x.z; c[3] = x.w;
    } else {
      const u32x2 x = bld64(rq, vq, (uint32_t)k0 / 2);
      c[0] = x.x; c[1] = x.y;
    }
    a = __uint_as_float(bld32(rs, vs, (uint32_t)k0 / 16));
  }
  QLS_DEV void store(uint16_t* s, const float* lut) const {
    const int t = threadIdx.x;
    uint16_t* d = s + (t / TPR) * PITCH + (t % TPR) * E;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      float v[8];
      deq8(c[j], a, lut, v);
      *reinterpret_cast<u32x4*>(d + 8 * j) = u32x4{pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]),
                                                   pack2_bf16(v[4], v[5]), pack2_bf16(v[6], v[7])};
    }
  }
};

// NF4, tile rows contiguous (W flat (k, col) = k * ldq + col, ldq % 64 == 0,
// every tile column valid); k >= K reads zero.
template <int ROWS>
struct FNf4Nn {
  static constexpr int KPT = ROWS / 32;
  static constexpr int RG = ROWS / 8;
  __amdgpu_buffer_rsrc_t rq, rs;
  uint32_t vq, vs;
  int ldq;
  uint32_t c[KPT];
  float a[KPT];
  QLS_DEV void init(const uint8_t* q, const float* sc, int64_t ldq_, int K, int r0) {
    rq = make_rsrc(q + r0 / 2, ((int64_t)K * ldq_ - r0) / 2);
    rs = make_rsrc(sc + r0 / 64, ((int64_t)K * ldq_ - r0) / 64 * 4);
    ldq = (int)ldq_;
    const int t = threadIdx.x;
    const int col = 8 * (t % RG), kb = KPT * (t / RG);
    vq = (uint32_t)((kb * ldq_ + col) / 2);
    vs = (uint32_t)((kb * (ldq_ / 64) + col / 64) * 4);
  }
  QLS_DEV void load(int k0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      c[i] = bld32(rq, vq, (uint32_t)(k0 + i) * (uint32_t)ldq / 2);
      a[i] = __uint_as_float(bld32(rs, vs, (uint32_t)(k0 + i) * (uint32_t)(ldq / 64) * 4));
    }
  }
  QLS_DEV void store(uint16_t* s, const float* lut) const {
    const int t = threadIdx.x;
    float v[KPT][8];
#pragma unroll
    for (int i = 0; i < KPT; ++i) deq8(c[i], a[i], lut, v[i]);
    uint16_t* base = s + (8 * (t % RG)) * PITCH + KPT * (t / RG);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (KPT == 4) {
        *reinterpret_cast<u32x2*>(base + e * PITCH) =
            u32x2{pack2_bf16(v[0][e], v[1][e]), pack2_bf16(v[2][e], v[3][e])};
      } else {
        *reinterpret_cast<uint32_t*>(base + e * PITCH) = pack2_bf16(v[0][e], v[1][e]);
      }
    }
  }
};

template <int ROWS>
QLS_DEV void LdNf4Nt<ROWS>::store(uint16_t* s, const float* lut) const {
  const int t = threadIdx.x;
  uint16_t* d = s + (t / TPR) * PITCH + (t % TPR) * E;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    float v[8];
    deq8(c[j], a[j], lut, v);
    *reinterpret_cast<u32x4*>(d + 8 * j) = u32x4{pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]),
                                                 pack2_bf16(v[4], v[5]), pack2_bf16(v[6], v[7])};
  }
}

template <int ROWS>
QLS_DEV void LdNf4Nn<ROWS>::store(uint16_t* s, const float* lut) const {
  const int t = threadIdx.x;
  float v[KPT][8];
#pragma unroll
  for (int i = 0; i < KPT; ++i) deq8(c[i], a[i], lut, v[i]);
  uint16_t* base = s + (8 * (t % RG)) * PITCH + KPT * (t / RG);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if constexpr (KPT == 4) {
      *reinterpret_cast<u32x2*>(base + e * PITCH) =
          u32x2{pack2_bf16(v[0][e], v[1][e]), pack2_bf16(v[2][e], v[3][e])};
    } else {
      *reinterpret_cast<uint32_t*>(base + e * PITCH) = pack2_bf16(v[0][e], v[1][e]);
    }
  }
}

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

template <int ROWS, int BL, bool F>
struct BLoaderOf;
template <int ROWS> struct BLoaderOf<ROWS, B_BF16_NT, false> { using T = LdBf16Row<ROWS>; };
template <int ROWS> struct BLoaderOf<ROWS, B_BF16_NN, false> { using T = LdBf16Col<ROWS>; };
template <int ROWS> struct BLoaderOf<ROWS, B_NF4_NT, false> { using T = LdNf4Nt<ROWS>; };
template <int ROWS> struct BLoaderOf<ROWS, B_NF4_NN, false> { using T = LdNf4Nn<ROWS>; };
template <int ROWS> struct BLoaderOf<ROWS, B_BF16_NT, true> { using T = FBf16Row<ROWS>; };
template <int ROWS> struct BLoaderOf<ROWS, B_BF16_NN, true> { using T = FBf16Col<ROWS>; };
template <int ROWS> struct BLoaderOf<ROWS, B_NF4_NT, true> { using T = FNf4Nt<ROWS>; };
template <int ROWS> struct BLoaderOf<ROWS, B_NF4_NN, true> { using T = FNf4Nn<ROWS>; };

template <int ROWS, int AL, bool F>
struct ALoaderOf;
template <int ROWS> struct ALoaderOf<ROWS, A_ROW, false> { using T = LdBf16Row<ROWS>; };
template <int ROWS> struct ALoaderOf<ROWS, A_COL, false> { using T = LdBf16Col<ROWS>; };
template <int ROWS> struct ALoaderOf<ROWS, A_ROW, true> { using T = FBf16Row<ROWS>; };
template <int ROWS> struct ALoaderOf<ROWS, A_COL, true> { using T = FBf16Col<ROWS>; };

template <int BM, int AL, bool F>
QLS_DEV void a_init(typename ALoaderOf<BM, AL, F>::T& la, const GemmArgs& g, int m0) {
  if constexpr (F) {
    if constexpr (AL == A_ROW) la.init(g.A, g.lda, g.M, m0);
    else la.init(g.A, g.lda, g.K, m0);
  }
}
template <int BN, int BL, bool F>
QLS_DEV void b_init(typename BLoaderOf<BN, BL, F>::T& lb, const GemmArgs& g, int n0) {
  if constexpr (F) {
    if constexpr (BL == B_BF16_NT) lb.init(g.Bh, g.ldb, g.N, n0);
    else if constexpr (BL == B_BF16_NN) lb.init(g.Bh, g.ldb, g.K, n0);
    else if constexpr (BL == B_NF4_NT) lb.init(g.Bq, g.Bs, g.ldq, g.N, n0);
    else lb.init(g.Bq, g.Bs, g.ldq, g.K, n0);
  }
}
template <int BM, int AL, bool F>
QLS_DEV void a_load(typename ALoaderOf<BM, AL, F>::T& la, const GemmArgs& g, int m0, int k0) {
  if constexpr (F) la.load(k0);
  else if constexpr (AL == A_ROW) la.load(g.A, g.lda, 0, g.M, m0, k0, g.K);
  else la.load(g.A, g.lda, g.M, m0, k0, g.K);
}
template <int BN, int BL, bool F>
QLS_DEV void b_load(typename BLoaderOf<BN, BL, F>::T& lb, const GemmArgs& g, int n0, int k0) {
  if constexpr (F) lb.load(k0);
  else if constexpr (BL == B_BF16_NT) lb.load(g.Bh, g.ldb, 0, g.N, n0, k0, g.K);
  else if constexpr (BL == B_BF16_NN) lb.load(g.Bh, g.ldb, g.N, n0, k0, g.K);
  else lb.load(g.Bq, g.Bs, g.ldq, g.N, n0, k0, g.K);
}
template <int BN, int BL, bool F>
QLS_DEV void b_store(const typename BLoaderOf<BN, BL, F>::T& lb, uint16_t* s, const float* lut) {
  if constexpr (BL == B_NF4_NT || BL == B_NF4_NN) lb.store(s, lut);
  else lb.store(s);
}

QLS_DEV float sigmoidf_(float x) { return 1.f / (1.f + __expf(-x)); }

// One output tile (tile = tm * tiles_n + tn) of contraction slice z of the
// product g; smem holds two LDS stages of (BM + BN) x PITCH bf16, lut 16 floats.
template <int BM, int BN, int AL, int BL, int EPI, bool F>
QLS_DEV void gemm_body(const GemmArgs& g, int tile, int z, const float* __restrict__ cb, uint16_t* smem,
                       float* lut) {
  constexpr int MI = BM / 64, NI = BN / 64;
  constexpr int STAGE = (BM + BN) * PITCH;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = (g.N + BN - 1) / BN;
  const int tm = tile / tiles_n, tn = tile % tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  if constexpr (BL == B_NF4_NT || BL == B_NF4_NN) {
    if (t < 16) lut[t] = cb[t];
  }

  const int nk = (g.K + BK - 1) / BK;
  const int ks = g.ksplit > 0 ? g.ksplit : 1;
  const int kb = (int)((int64_t)nk * z / ks);
  const int ke = (int)((int64_t)nk * (z + 1) / ks);

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = f32x16{};

  // ---- LoRA contraction first (split 0 only), so no second accumulator is
  // needed: FWD starts the accumulator at (s2/alpha) U_g B_g^T, DX at du_cat A_cat;
  // the base product then accumulates on top in fp32.
  const bool first = z == 0;
  if constexpr (BL == B_NF4_NT && EPI == EPI_BF16) {
    if (g.lora == LORA_FWD && first) {
      // columns of modules other than g read B as zero
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
            mma_tile<BM, BN>(smem, smem + BM * PITCH, acc, wm, wn, lane);
            __syncthreads();
          }
        }
        start = end;
      }
      const float sc = g.s2 / g.alpha;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] *= sc;
    }
  }
  if constexpr (BL == B_NF4_NN) {
    if (g.lora == LORA_DX && first) {
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

  // Two register stages and two LDS stages: while tile k is multiplied out of
  // LDS, tile k+1 waits in registers to be written to the other LDS stage and
  // the global loads of tile k+2 are in flight, so each load has two MFMA
  // phases to arrive.
  typename ALoaderOf<BM, AL, F>::T la0, la1;
  typename BLoaderOf<BN, BL, F>::T lb0, lb1;
  a_init<BM, AL, F>(la0, g, m0);
  a_init<BM, AL, F>(la1, g, m0);
  b_init<BN, BL, F>(lb0, g, n0);
  b_init<BN, BL, F>(lb1, g, n0);
  uint16_t* const s0 = smem;
  uint16_t* const s1 = smem + STAGE;
  __syncthreads();
  if (kb < ke) {
    a_load<BM, AL, F>(la0, g, m0, kb * BK);
    b_load<BN, BL, F>(lb0, g, n0, kb * BK);
    if (kb + 1 < ke) {
      a_load<BM, AL, F>(la1, g, m0, (kb + 1) * BK);
      b_load<BN, BL, F>(lb1, g, n0, (kb + 1) * BK);
    }
    la0.store(s0);
    b_store<BN, BL, F>(lb0, s0 + BM * PITCH, lut);
    __syncthreads();
    for (int kt = kb; kt < ke; kt += 2) {
      // tile kt in s0, tile kt+1 in registers 1
      if (kt + 2 < ke) {
        a_load<BM, AL, F>(la0, g, m0, (kt + 2) * BK);
        b_load<BN, BL, F>(lb0, g, n0, (kt + 2) * BK);
      }
      mma_tile<BM, BN>(s0, s0 + BM * PITCH, acc, wm, wn, lane);
      if (kt + 1 < ke) {
        la1.store(s1);
        b_store<BN, BL, F>(lb1, s1 + BM * PITCH, lut);
      }
      __syncthreads();
      if (kt + 1 >= ke) break;
      // tile kt+1 in s1, tile kt+2 in registers 0
      if (kt + 3 < ke) {
        a_load<BM, AL, F>(la1, g, m0, (kt + 3) * BK);
        b_load<BN, BL, F>(lb1, g, n0, (kt + 3) * BK);
      }
      mma_tile<BM, BN>(s1, s1 + BM * PITCH, acc, wm, wn, lane);
      if (kt + 2 < ke) {
        la0.store(s0);
        b_store<BN, BL, F>(lb0, s0 + BM * PITCH, lut);
      }
      __syncthreads();
    }
  }

  // ---- split-K: store alpha*acc as a float partial;
  // gemm_reduce_epi sums the splits in index order and applies the epilogue.
  if constexpr (EPI != EPI_PARTIAL && EPI != EPI_CE_STATS && EPI != EPI_CE_GRAD) {
    if (ks > 1) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int m = m0 + wm * (BM / 2) + 32 * i + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
            const int n = n0 + wn * (BN / 2) + 32 * j + (lane & 31);
            if (m >= g.M || n >= g.N) continue;
            const float v = g.alpha * acc[i][j][q];
            g.partial[((int64_t)z * g.M + m) * g.N + n] = v;
          }
      return;
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
            if (g.R) y += bf2f(g.R[(int64_t)m * g.ldr + n]);
            reinterpret_cast<uint16_t*>(g.C)[(int64_t)m * g.ldc + n] = f2bf(y);
          } else if constexpr (EPI == EPI_F32) {
            reinterpret_cast<float*>(g.C)[(int64_t)m * g.ldc + n] = g.alpha * v;
          } else if constexpr (EPI == EPI_F32_ACC) {
            reinterpret_cast<float*>(g.C)[(int64_t)m * g.ldc + n] += g.alpha * v;
          } else if constexpr (EPI == EPI_PARTIAL) {
            g.partial[((int64_t)z * g.M + m) * g.N + n] = v;
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

template <int BM, int BN, int AL, int BL, int EPI, bool F>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2)))
gemm_kernel(GemmArgs g, const float* __restrict__ cb) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * PITCH];
  __shared__ float lut[16];
  gemm_body<BM, BN, AL, BL, EPI, F>(g, blockIdx.x, blockIdx.z, cb, smem, lut);
}

// Several products of one loader combination in one launch (split-K float
// partials, summed by reduce_group_kernel): workgroups [end[p-1], end[p])
// take the tiles and slices of product p, slice-major.
template <int BM, int BN, int AL, int BL, bool F>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2)))
gemm_group_kernel(GemmGroup gg) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * PITCH];
  __shared__ float lut[16];
  int p = 0;
  while (p + 1 < gg.n && (int)blockIdx.x >= gg.end[p]) ++p;
  const int local = (int)blockIdx.x - (p ? gg.end[p - 1] : 0);
  const GemmArgs& g = gg.g[p];
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  gemm_body<BM, BN, AL, BL, EPI_PARTIAL, F>(g, local % tiles, local / tiles, nullptr, smem, lut);
}

// Split-order sums of the partials of several products, each with its own
// output: bf16 (mode 0) or float (mode 1) alpha * sum at C (ldc), or, with
// rows > 0, row block m / rows of the sum to Cr[m / rows] (float).
__global__ void reduce_group_kernel(ReduceGroup rg) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int p = 0;
  while (p + 1 < rg.n && idx >= rg.end[p]) ++p;
  if (idx >= rg.end[p]) return;
  const ReduceJob& j = rg.j[p];
  const int64_t local = idx - (p ? rg.end[p - 1] : 0);
  const int64_t MN = (int64_t)j.M * j.N;
  const int m = (int)(local / j.N), n = (int)(local % j.N);
  float s = 0.f;
  for (int z = 0; z < j.ks; ++z) s += j.P[z * MN + local];
  if (j.rows > 0)
    j.Cr[m / j.rows][(int64_t)(m % j.rows) * j.ldc + n] = j.alpha * s;
  else if (j.mode == 0)
    reinterpret_cast<uint16_t*>(j.C)[(int64_t)m * j.ldc + n] = f2bf(j.alpha * s);
  else
    reinterpret_cast<float*>(j.C)[(int64_t)m * j.ldc + n] = j.alpha * s;
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

// reduce_kernel's sum (fp32 output), with row block m / rows of the product
// going to its own matrix: C[m / rows], row m % rows.
struct RowBlocks { float* c[4]; int rows; };
__global__ void reduce_rows_kernel(const float* __restrict__ P, int ks, int M, int N, float alpha,
                                   RowBlocks o, int64_t ldc) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t MN = (int64_t)M * N;
  if (idx >= MN) return;
  const int m = (int)(idx / N), n = (int)(idx % N);
  float s = 0.f;
  for (int z = 0; z < ks; ++z) s += P[z * MN + idx];
  o.c[m / o.rows][(int64_t)(m % o.rows) * ldc + n] = alpha * s;
}

// Sum of the split-K partials in split order, then the GEMM's own epilogue;
// four consecutive columns per thread (N % 4 == 0).
__global__ void reduce_epi_kernel(GemmArgs g, int epi) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int n4 = g.N / 4;
  if (q >= (int64_t)g.M * n4) return;
  const int m = (int)(q / n4), n = 4 * (int)(q % n4);
  const int64_t MN = (int64_t)g.M * g.N;
  const float* p = g.partial + (int64_t)m * g.N + n;
  f32x4 s = *reinterpret_cast<const f32x4*>(p);
  for (int z = 1; z < g.ksplit; ++z) s += *reinterpret_cast<const f32x4*>(p + z * MN);
  if (epi == EPI_BF16) {
    if (g.R) {
      const uint16_t* r = g.R + (int64_t)m * g.ldr + n;
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] += bf2f(r[i]);
    }
    uint16_t* c = reinterpret_cast<uint16_t*>(g.C) + (int64_t)m * g.ldc + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = f2bf(s[i]);
  } else if (epi == EPI_F32) {
    float* c = reinterpret_cast<float*>(g.C) + (int64_t)m * g.ldc + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = s[i];
  } else if (epi == EPI_F32_ACC) {
    float* c = reinterpret_cast<float*>(g.C) + (int64_t)m * g.ldc + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] += s[i];
  } else if (epi == EPI_SWIGLU_BWD) {
    uint16_t* out = reinterpret_cast<uint16_t*>(g.C) + (int64_t)m * g.ldc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float gg = bf2f(g.gu[(int64_t)m * g.ldgu + n + i]);
      const float uu = bf2f(g.gu[(int64_t)m * g.ldgu + g.I + n + i]);
      const float sg = sigmoidf_(gg);
      out[n + i] = f2bf(s[i] * uu * sg * (1.f + gg * (1.f - sg)));
      out[g.I + n + i] = f2bf(s[i] * (gg * sg));
    }
  }
}

template <int BM, int BN, int AL, int BL, int EPI, bool F>
void launch_t(const GemmArgs& g, const float* cb, hipStream_t st) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  const int ks = g.ksplit > 0 ? g.ksplit : 1;
  if (g.ev0) (void)hipEventRecord(g.ev0, st);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, AL, BL, EPI, F>), dim3(tiles, 1, ks), dim3(NT), 0, st, g, cb);
  if (g.ev1) (void)hipEventRecord(g.ev1, st);
  if (ks > 1 && EPI != EPI_PARTIAL && EPI != EPI_CE_STATS && EPI != EPI_CE_GRAD) {
    const int64_t n = (int64_t)g.M * (g.N / 4);
    hipLaunchKernelGGL(reduce_epi_kernel, dim3((unsigned)ceil_div64(n, 256)), dim3(256), 0, st, g, EPI);
  }
}

// Shapes the fast (buffer-load) loaders accept: contraction-contiguous
// operands need K % 64 == 0; row-contiguous ones need every tile row valid;
// NF4 needs 64-aligned rows; every resource stays below 2 GiB.
bool fast_ok(const GemmArgs& g, int aload, int bload, int tile) {
  const int64_t lim = 0x7fffffffLL;
  if (aload == A_ROW && (g.K % 64 || g.lda % 8 || (int64_t)g.M * g.lda * 2 > lim)) return false;
  if (aload == A_COL && (g.M % tile || g.lda % 8 || (int64_t)g.K * g.lda * 2 > lim)) return false;
  if (bload == B_BF16_NT && (g.K % 64 || g.ldb % 8 || (int64_t)g.N * g.ldb * 2 > lim)) return false;
  if (bload == B_BF16_NN && (g.N % tile || g.ldb % 8 || (int64_t)g.K * g.ldb * 2 > lim)) return false;
  if (bload == B_NF4_NT && (g.K % 64 || g.ldq % 64 || (int64_t)g.N * g.ldq / 2 > lim)) return false;
  if (bload == B_NF4_NN && (g.N % tile || g.ldq % 64 || (int64_t)g.K * g.ldq / 2 > lim)) return false;
  return true;
}

}  // namespace

const float* nf4_codebook_dev();  // defined in nf4.hip

int gemm_launch(const GemmArgs& g, int aload, int bload, int epi, int tile, hipStream_t st) {
  if (g.ksplit > 1 && !g.partial) return -1;   // split-K partials need a buffer
  const float* cb = (bload == B_NF4_NT || bload == B_NF4_NN) ? nf4_codebook_dev() : nullptr;
  const bool fast = fast_ok(g, aload, bload, tile);
#define QLS_CASE(BMV, AL, BL, EP)                                           \
  if (tile == BMV && aload == AL && bload == BL && epi == EP) {             \
    if (fast) launch_t<BMV, BMV, AL, BL, EP, true>(g, cb, st);              \
    else launch_t<BMV, BMV, AL, BL, EP, false>(g, cb, st);                  \
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
  QLS_CASE(64, A_ROW, B_BF16_NT, EPI_BF16)
  QLS_CASE(64, A_ROW, B_BF16_NN, EPI_BF16)
  QLS_CASE(64, A_COL, B_BF16_NN, EPI_F32)
#undef QLS_CASE
  return -1;  // combination not instantiated
}

void gemm_reduce(const float* partial, int ksplit, int M, int N, float alpha, int mode, void* C,
                 int64_t ldc, hipStream_t st) {
  const int64_t MN = (int64_t)M * N;
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)ceil_div64(MN, 256)), dim3(256), 0, st, partial,
                     ksplit, M, N, alpha, mode, C, ldc);
}

int gemm_reduce_rows(const float* partial, int ksplit, int M, int N, float alpha, float* const* C, int rows,
                     int64_t ldc, hipStream_t st) {
  RowBlocks o{};
  if (rows <= 0 || M % rows || M / rows > 4) return -1;
  for (int i = 0; i < M / rows; ++i) o.c[i] = C[i];
  o.rows = rows;
  const int64_t MN = (int64_t)M * N;
  hipLaunchKernelGGL(reduce_rows_kernel, dim3((unsigned)ceil_div64(MN, 256)), dim3(256), 0, st, partial,
                     ksplit, M, N, alpha, o, ldc);
  return 0;
}

int64_t gemm_partial_elems(int M, int N, int ksplit) { return (int64_t)M * N * ksplit; }

static_assert(sizeof(GemmGroup) <= 4096, "grouped GEMM arguments must fit the kernel argument segment");
static_assert(sizeof(ReduceGroup) <= 4096, "grouped reduce arguments must fit the kernel argument segment");

int gemm_group_launch(const GemmGroup& gg, int aload, int bload, hipStream_t st) {
  if (gg.n < 1 || gg.n > kMaxGroup) return -1;
  bool fast = true;
  for (int i = 0; i < gg.n; ++i) {
    if (!gg.g[i].partial || gg.g[i].ksplit < 1) return -1;
    fast = fast && fast_ok(gg.g[i], aload, bload, 64);
  }
  const dim3 grid((unsigned)gg.end[gg.n - 1]);
#define QLS_GCASE(AL, BL)                                                                         \
  if (aload == AL && bload == BL) {                                                               \
    if (fast) hipLaunchKernelGGL((gemm_group_kernel<64, 64, AL, BL, true>), grid, dim3(NT), 0, st, gg);  \
    else hipLaunchKernelGGL((gemm_group_kernel<64, 64, AL, BL, false>), grid, dim3(NT), 0, st, gg);      \
    return 0;                                                                                     \
  }
  QLS_GCASE(A_ROW, B_BF16_NN)
  QLS_GCASE(A_COL, B_BF16_NN)
  QLS_GCASE(A_ROW, B_BF16_NT)
#undef QLS_GCASE
  return -1;
}

int reduce_group_launch(const ReduceGroup& rg, hipStream_t st) {
  if (rg.n < 1 || rg.n > kMaxGroup) return -1;
  const int64_t n = rg.end[rg.n - 1];
  if (n <= 0) return 0;
  hipLaunchKernelGGL(reduce_group_kernel, dim3((unsigned)ceil_div64(n, 256)), dim3(256), 0, st, rg);
  return 0;
}

void gemm_reduce_epi(const GemmArgs& g, int epi, hipStream_t st) {
  const int64_t n = (int64_t)g.M * (g.N / 4);
  hipLaunchKernelGGL(reduce_epi_kernel, dim3((unsigned)ceil_div64(n, 256)), dim3(256), 0, st, g, epi);
}
