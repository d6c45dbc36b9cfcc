// Large-M dequant-GEMMs for gfx950: 256 x 256 output tile per 512-thread
// workgroup, v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//
//   * NT:  Y = X W^T (+ s U_g B_g^T) (+ residual), W NF4 [N, K] (the forward);
//   * NN:  dX = dY W (+ du_cat A_cat), contraction over W's rows (the backward);
//   * bf16 W: the LM head, [N, K] for the logits (cross-entropy epilogues) and
//     [K, N] for dh = dlogits W (float output, plain or accumulated).
//
// Eight waves, two per SIMD, in a 2 x 4 grid; each wave owns 128 x 64 of the
// tile (4 x 2 MFMA blocks, 128 accumulators per lane), so the other wave on
// the SIMD can issue while one waits on LDS or a barrier.  The k-loop runs in
// steps of 64 (one NF4 block along K for NT): global loads run two steps
// ahead: the activation tile goes straight from global memory into LDS
// (buffer_load ... lds, 16 bytes per lane), the NF4 codes through two register
// stages.  Each step dequantises the NF4 tile of the next step (bf16 =
// RNE(float32(cb[c] * absmax)), one 2 KB LDS table that maps a code byte to its
// two codebook values) into the other of two LDS stages while the MFMAs
// consume the current one.  Activation tiles are unpadded 128-byte rows whose
// 16-byte chunks are XOR-swizzled by row; weight tiles are padded to 72 bf16
// per row (NT) or chunk-swizzled (NN), so fragment reads are free of bank
// conflicts.  The epilogue goes through LDS, 32 rows at a time, so residual
// loads and output stores are 16 bytes per lane and row-contiguous.
#include "common.h"
#include "gemm.h"

namespace {

constexpr int NT = 512;
constexpr int BM = 256, BN = 256, BK = 64, PITCH = BK + 8;
constexpr int ATILE = BM * BK;      // bf16 elements of an activation tile (unpadded rows)
constexpr int TILE = BN * PITCH;     // bf16 elements of a weight tile
constexpr int TP = BN + 4;           // fp32 pitch of the staged epilogue rows
constexpr int EROWS = 32;            // epilogue rows staged at a time (through weight stage 0)
#ifndef QLS_LORA_STEPS
#define QLS_LORA_STEPS 2
#endif
constexpr int kLoraSteps = QLS_LORA_STEPS;   // split-K weight of one 64-deep LoRA step
static_assert(EROWS * TP * 4 <= TILE * 2, "epilogue rows must fit a weight stage");

QLS_DEV __amdgpu_buffer_rsrc_t rsrc(const void* p, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}
QLS_DEV u32x4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, v, s, 0));
}
QLS_DEV uint32_t ld32(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, v, s, 0);
}
QLS_DEV float sigm(float x) { return 1.f / (1.f + __expf(-x)); }

// Activation tile: 16-byte chunk c of row r sits at chunk c ^ a_swz(r).  Eight
// consecutive rows (the 128-byte bank span) and sixteen consecutive rows with
// the same parity both map one chunk index to distinct chunks.
QLS_DEV int a_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
QLS_DEV int a_pos(int r, int k) { return r * BK + 8 * ((k >> 3) ^ a_swz(r)) + (k & 7); }

// NN B tile: each thread dequantises 4 contraction rows x 8 columns.  Column
// group cg (8 columns) and row quad kq of thread t are interleaved so that a
// half-wave covers 8 column groups x 4 row quads (so a wave's code loads are
// 4 rows x 64 bytes), and the 16-byte chunks of each LDS row are XOR-swizzled
// by (row / 16), which spreads the transposing 8-byte writes.  Measured on
// gfx950 the writes run at about 3/4 of the conflict-free rate and the 16-byte
// fragment reads at half rate (lanes l and l + 16 of a read take the two
// halves of the same four banks, and here they fall on different granules);
// layouts that fix both need a thread mapping whose code loads cost more.
QLS_DEV int nn_cg(int t) { return (t & 7) | (((t >> 5) & 3) << 3); }
QLS_DEV int nn_kq(int t) { return ((t >> 3) & 3) | ((t >> 7) << 2); }
QLS_DEV int nn_swz(int n) { return 2 * ((n >> 4) & 3); }
// Element offset of contraction index k (multiple of 4) in LDS row n of an NN B tile.
QLS_DEV int nn_pos(int n, int k) { return n * PITCH + 8 * ((k >> 3) ^ nn_swz(n)) + (k & 7); }

// One register stage of NF4 data: NT: 32 codes of one W row + absmax; NN:
// 4 W rows x 8 columns + 4 absmax.  kLoads: the VMEM instructions of a stage.
template <int BL> struct Stage;
template <> struct Stage<B_NF4_NT> { u32x4 q; float s; static constexpr int kLoads = 2; };
template <> struct Stage<B_NF4_NN> { uint32_t q[4]; float s[4]; static constexpr int kLoads = 8; };
// bf16 W[n, k] (the LM head): the weight tile goes to LDS by DMA like the
// activation tile, in the same swizzled layout; nothing passes through registers.
template <> struct Stage<B_BF16_NT> { static constexpr int kLoads = 0; };
// bf16 W[k, n] (dh = dlogits W): the weight tile goes to LDS by DMA as 64
// row-major rows of 256 columns, and the MFMA reads it column-wise with the
// transposing ds_read_b64_tr_b16.
template <> struct Stage<B_BF16_NN> { static constexpr int kLoads = 0; };

// Row-major bf16 weight tile [64 k][256 n]: 16-byte chunk c of row r sits at
// chunk c ^ 4 (r mod 4), so the four rows a 32-lane transposing read covers
// (four adjacent chunks each) land in sixteen distinct 16-byte granules, all
// 64 banks of gfx950's LDS.
QLS_DEV int t_swz(int r) { return 4 * (r & 3); }
QLS_DEV int t_pos(int r, int n) { return r * BN + 8 * ((n >> 3) ^ t_swz(r)) + (n & 7); }

// NT weight tile: the thread that loads and decodes 32 codes (half `half` of
// the k-step) of tile row `row`.  Sixteen consecutive lanes take sixteen
// consecutive rows, so each 16-byte LDS write of the decode covers 16
// distinct granules of the 144-byte-pitch rows (9 r mod 16 is a bijection).
QLS_DEV int nt_row(int t) { return (t & 15) | ((t >> 5) << 4); }
QLS_DEV int nt_half(int t) { return (t >> 4) & 1; }

// Wait until at most n vector-memory operations are outstanding and every LDS
// operation is done (gfx9 s_waitcnt encoding: vmcnt bits 3:0 and 15:14,
// expcnt 6:4 left at its maximum, lgkmcnt 11:8 = 0).
template <int N>
QLS_DEV void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

template <int BL>
struct Big {
  const GemmArgs& g;
  uint16_t* sA[2];
  uint16_t* sB[2];
  const float2* lut2;
  int t, lane, wm, wn, m0, n0;
  __amdgpu_buffer_rsrc_t ra, rq, rs;
  uint32_t vdma[4], vdmb[4], vq, vs;
  __amdgpu_buffer_rsrc_t rb;
  f32x16 acc[4][2];

  QLS_DEV Big(const GemmArgs& g_, uint16_t* a0, uint16_t* a1, uint16_t* b0, uint16_t* b1,
              const float2* lut2_, int m0_, int n0_)
      : g(g_), lut2(lut2_), m0(m0_), n0(n0_) {
    sA[0] = a0; sA[1] = a1; sB[0] = b0; sB[1] = b1;
    t = threadIdx.x;
    lane = t & 63;
    const int wave = t >> 6;
    wm = wave >> 2;
    wn = wave & 3;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    // A rows m0.. through a resource that ends at row M (rows past it read 0).
    // DMA: wave w, instruction j fills LDS rows 8(4w+j) .. +7 (1 KB); lane l
    // lands in row +l/8, chunk slot l%8, which holds chunk (l%8) ^ a_swz(row).
    ra = rsrc(g.A + (int64_t)m0 * g.lda, (int64_t)(g.M - m0) * g.lda * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 8 * (4 * (t >> 6) + j) + (lane >> 3);
      vdma[j] = (uint32_t)((r * g.lda + 8 * ((lane & 7) ^ a_swz(r))) * 2);
    }
    if constexpr (BL == B_BF16_NT) {
      // W rows n0.. (ldb elements apart), rows past N read 0.
      rb = rsrc(g.Bh + (int64_t)n0 * g.ldb, (int64_t)(g.N - n0) * g.ldb * 2);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 8 * (4 * (t >> 6) + j) + (lane >> 3);
        vdmb[j] = (uint32_t)((r * g.ldb + 8 * ((lane & 7) ^ a_swz(r))) * 2);
      }
    } else if constexpr (BL == B_BF16_NN) {
      // W rows k (ldb elements apart), columns n0 .. n0 + 255 (N % 256 == 0).
      // DMA: wave w, instruction j fills tile rows 2 (4w + j) and +1 (1 KB);
      // lane l lands in row +l/32, chunk slot l%32, which holds chunk
      // (l%32) ^ t_swz(row).
      rb = rsrc(g.Bh + n0, ((int64_t)g.K * g.ldb - n0) * 2);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 2 * (4 * (t >> 6) + j) + (lane >> 5);
        vdmb[j] = (uint32_t)((r * g.ldb + 8 * ((lane & 31) ^ t_swz(r))) * 2);
      }
    } else if constexpr (BL == B_NF4_NT) {
      // W rows n0..: codes row n at n * ldq / 2, absmax at n * ldq / 64.
      rq = rsrc(g.Bq + (int64_t)n0 * g.ldq / 2, (int64_t)(g.N - n0) * g.ldq / 2);
      rs = rsrc(g.Bs + (int64_t)n0 * (g.ldq / 64), (int64_t)(g.N - n0) * (g.ldq / 64) * 4);
      vq = (uint32_t)(nt_row(t) * (g.ldq / 2) + 16 * nt_half(t));
      vs = (uint32_t)(nt_row(t) * (g.ldq / 64) * 4);
    } else {
      // W columns n0..: element (k, n) at k * ldq + n; 32 groups of 8 columns,
      // 16 groups of 4 contraction rows.
      const int cg = nn_cg(t), kq = nn_kq(t);
      rq = rsrc(g.Bq + n0 / 2, ((int64_t)g.K * g.ldq - n0) / 2);
      rs = rsrc(g.Bs + n0 / 64, ((int64_t)g.K * g.ldq - n0) / 64 * 4);
      vq = (uint32_t)(((int64_t)4 * kq * g.ldq + 8 * cg) / 2);
      vs = (uint32_t)(((int64_t)4 * kq * (g.ldq / 64) + cg / 8) * 4);
    }
  }

  // Activation tile k0 .. k0+64 straight into LDS (and the bf16 weight tile).
  QLS_DEV void dma(uint16_t* s, int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(s + (4 * (t >> 6) + j) * 512), 16, vdma[j],
          (uint32_t)k0 * 2, 0, 0);
  }
  QLS_DEV void dma_b(uint16_t* s, int k0) {
    // NT: k0 columns along each W row; NN: k0 rows down.
    const uint32_t soff = BL == B_BF16_NN ? (uint32_t)k0 * (uint32_t)g.ldb * 2u : (uint32_t)k0 * 2u;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (__attribute__((address_space(3))) void*)(s + (4 * (t >> 6) + j) * 512), 16, vdmb[j], soff, 0, 0);
  }

  QLS_DEV void load(Stage<BL>& r, int k0) {
    if constexpr (BL == B_BF16_NT || BL == B_BF16_NN) {
      (void)r;
      (void)k0;
    } else if constexpr (BL == B_NF4_NT) {
      r.q = ld128(rq, vq, (uint32_t)k0 / 2);
      r.s = __uint_as_float(ld32(rs, vs, (uint32_t)k0 / 16));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        r.q[i] = ld32(rq, vq, (uint32_t)(k0 + i) * (uint32_t)g.ldq / 2);
        r.s[i] = __uint_as_float(ld32(rs, vs, (uint32_t)(k0 + i) * (uint32_t)(g.ldq / 64) * 4));
      }
    }
  }

  // Dequantise one register stage into weight stage sB.
  QLS_DEV void store(const Stage<BL>& r, uint16_t* sB) const {
    const int row = nt_row(t), half = nt_half(t);
    if constexpr (BL == B_BF16_NT || BL == B_BF16_NN) {
      (void)r;
      (void)sB;
      (void)row;
      (void)half;
    } else if constexpr (BL == B_NF4_NT) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t c = r.q[w];
        u32x4 o;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float2 v = lut2[(c >> (8 * b)) & 0xFFu];
          o[b] = pack2_bf16(v.x * r.s, v.y * r.s);
        }
        *reinterpret_cast<u32x4*>(sB + row * PITCH + 32 * half + 8 * w) = o;
      }
    } else {
      // Byte b of each of the 4 code words holds columns 2b, 2b+1 of one
      // contraction row; each column's 4 rows land as one 8-byte LDS write.
      const int cg = nn_cg(t), kq = nn_kq(t);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        float2 e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = lut2[(r.q[i] >> (8 * b)) & 0xFFu];
        *reinterpret_cast<u32x2*>(sB + nn_pos(8 * cg + 2 * b, 4 * kq)) =
            u32x2{pack2_bf16(e[0].x * r.s[0], e[1].x * r.s[1]), pack2_bf16(e[2].x * r.s[2], e[3].x * r.s[3])};
        *reinterpret_cast<u32x2*>(sB + nn_pos(8 * cg + 2 * b + 1, 4 * kq)) =
            u32x2{pack2_bf16(e[0].y * r.s[0], e[1].y * r.s[1]), pack2_bf16(e[2].y * r.s[2], e[3].y * r.s[3])};
      }
    }
  }

  QLS_DEV void mma(const uint16_t* sA, const uint16_t* sB) {
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int kofs = 16 * s + 8 * (lane >> 5);
      u32x4 a[4], b[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const u32x4*>(sA + a_pos(wm * 128 + 32 * i + (lane & 31), kofs));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = wn * 64 + 32 * j + (lane & 31);
        if constexpr (BL == B_BF16_NN) {
          // 8 contraction rows kofs .. kofs + 7 of column n: a 16-lane group
          // reads rows +0..3 and +4..7, columns nb .. nb + 15 (lane i of the
          // group supplies row i / 4, columns 4 (i % 4) .. + 3).
          typedef short v4s __attribute__((ext_vector_type(4)));
          const int nb = wn * 64 + 32 * j + 16 * ((lane >> 4) & 1);
          const int r = kofs + ((lane & 15) >> 2), c = nb + 4 * (lane & 3);
          const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4s*)(sB + t_pos(r, c)));
          const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4s*)(sB + t_pos(r + 4, c)));
          const u32x2 x = __builtin_bit_cast(u32x2, lo), y = __builtin_bit_cast(u32x2, hi);
          b[j] = u32x4{x.x, x.y, y.x, y.y};
        } else if constexpr (BL == B_NF4_NN)
          b[j] = *reinterpret_cast<const u32x4*>(sB + nn_pos(n, kofs));
        else if constexpr (BL == B_BF16_NT)
          b[j] = *reinterpret_cast<const u32x4*>(sB + a_pos(n, kofs));
        else
          b[j] = *reinterpret_cast<const u32x4*>(sB + n * PITCH + kofs);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
    }
  }

  // ---- LoRA contraction into the accumulator (before the base product).
  // Plain guarded loads: it runs once per tile.
  // Rows r0.. of P (row-major, ld), contraction columns [k0, k0+64) of [0, K),
  // rows outside [rlo, rhi) as zero; `swz`: activation layout, else padded.
  QLS_DEV void stage_rows(uint16_t* s, bool swz, const uint16_t* p, int64_t ld, int rlo, int rhi, int r0,
                          int k0, int K) const {
    const int row = t >> 1, half = t & 1;
    const int gr = r0 + row;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = 32 * half + 8 * j;
      const int k = k0 + kk;
      u32x4 v = u32x4{0, 0, 0, 0};
      if (gr >= rlo && gr < rhi && k < K) v = *reinterpret_cast<const u32x4*>(p + (int64_t)gr * ld + k);
      *reinterpret_cast<u32x4*>(s + (swz ? a_pos(row, kk) : row * PITCH + kk)) = v;
    }
  }
  // Columns n0.. of P stored k-major (element (k, n) at p[k * ld + n]),
  // transposed into the swizzled NN layout:
  QLS_DEV void stage_cols(uint16_t* s, const uint16_t* p, int64_t ld, int ncols, int k0, int K) const {
    const int cg = nn_cg(t), kq = nn_kq(t);   // 8 columns x 4 contraction rows
    uint32_t w[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = k0 + 4 * kq + i;
      const int n = n0 + 8 * cg;
      u32x4 x = u32x4{0, 0, 0, 0};
      if (k < K && n < ncols) x = *reinterpret_cast<const u32x4*>(p + (int64_t)k * ld + n);
      w[i][0] = x.x; w[i][1] = x.y; w[i][2] = x.z; w[i][3] = x.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = 16 * (e & 1);
      const uint32_t x0 = (w[0][e >> 1] >> sh) & 0xFFFFu, x1 = (w[1][e >> 1] >> sh) & 0xFFFFu;
      const uint32_t x2 = (w[2][e >> 1] >> sh) & 0xFFFFu, x3 = (w[3][e >> 1] >> sh) & 0xFFFFu;
      *reinterpret_cast<u32x2*>(s + nn_pos(8 * cg + e, 4 * kq)) = u32x2{x0 | (x1 << 16), x2 | (x3 << 16)};
    }
  }

  QLS_DEV void lora() {
    uint16_t* sa = sA[0];
    uint16_t* sb = sB[0];
    if constexpr (BL == B_NF4_NT) {
      // acc = (s2 / alpha) sum_g U_g B_g^T; B_g is zero outside module g's columns.
      int start = 0;
      for (int gi = 0; gi < g.nmod; ++gi) {
        const int end = g.mod_end[gi];
        if (end > n0 && start < n0 + BN) {
          const uint16_t* bp = g.modB[gi] - (int64_t)start * g.K2;
          for (int k0 = 0; k0 < g.K2; k0 += BK) {
            stage_rows(sa, true, g.A2 + gi * g.K2, g.lda2, 0, g.M, m0, k0, g.K2);
            stage_rows(sb, false, bp, g.K2, start, end, n0, k0, g.K2);
            __syncthreads();
            mma(sa, sb);
            __syncthreads();
          }
        }
        start = end;
      }
      const float sc = g.s2 / g.alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] *= sc;
    } else {
      // acc = du_cat A_cat, A_cat [K2, N] row-major.
      for (int k0 = 0; k0 < g.K2; k0 += BK) {
        stage_rows(sa, true, g.A2, g.lda2, 0, g.M, m0, k0, g.K2);
        stage_cols(sb, g.B2, g.ldb2, g.N, k0, g.K2);
        __syncthreads();
        mma(sa, sb);
        __syncthreads();
      }
    }
  }

  // ---- base product: one barrier per step.  Step kt: the MFMAs read stage
  // kt&1 while the DMA fills the activation tile of kt+1 into the other stage,
  // the NF4 codes of kt+1 (loaded a step earlier) are dequantised into the
  // other weight stage and the codes of kt+2 are loaded.  The DMA is issued
  // before the code loads (a compiler fence keeps the order), so waiting for
  // all but the newest kLoads vector operations before the barrier covers it.
  QLS_DEV void half_step(int kt, int kb, int nk, int cur, Stage<BL>& rld, const Stage<BL>& rst) {
    dma(sA[cur ^ 1], (kb + min(kt + 1, nk - 1)) * BK);
    if constexpr (BL == B_BF16_NT || BL == B_BF16_NN) dma_b(sB[cur ^ 1], (kb + min(kt + 1, nk - 1)) * BK);
    asm volatile("" ::: "memory");
    load(rld, (kb + min(kt + 2, nk - 1)) * BK);
    mma(sA[cur], sB[cur]);
    store(rst, sB[cur ^ 1]);
    wait_vm_lds<Stage<BL>::kLoads>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  // Contraction steps [kb, ke) of 64 (a split-K slice, or all of K).
  QLS_DEV void mainloop(int kb, int ke) {
    const int nk = ke - kb;
    Stage<BL> r0, r1;
    dma(sA[0], kb * BK);
    if constexpr (BL == B_BF16_NT || BL == B_BF16_NN) dma_b(sB[0], kb * BK);
    asm volatile("" ::: "memory");
    load(r0, kb * BK);
    load(r1, (kb + min(1, nk - 1)) * BK);
    store(r0, sB[0]);
    wait_vm_lds<Stage<BL>::kLoads>();     // the first tiles' DMA (issued before r0, r1) is done
    __syncthreads();
    // Loads past the last step re-read step ke-1 (in bounds, never consumed).
    for (int kt = 0;; kt += 2) {
      half_step(kt, kb, nk, 0, r0, r1);
      if (kt + 1 >= nk) break;
      half_step(kt + 1, kb, nk, 1, r1, r0);
      if (kt + 2 >= nk) break;
    }
    __syncthreads();
  }

  // ---- epilogue through LDS (weight stage 0), 32 rows at a time; 8 columns
  // per thread.  Rows 32h .. 32h+31 are block i = h%4 of the waves with wm = h/4.
  // C / ldc: the output (EPI_F32 also serves the split-K partials).
  template <int EPI>
  QLS_DEV void epilogue(void* C, int64_t ldc) {
    float* sT = reinterpret_cast<float*>(sB[0]);
#pragma unroll
    for (int h = 0; h < BM / EROWS; ++h) {
      if (wm == (h >> 2)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i != (h & 3)) continue;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
              const int mm = 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
              const int nn = wn * 64 + 32 * j + (lane & 31);
              sT[mm * TP + nn] = acc[i][j][q];
            }
        }
      }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < EROWS * BN / 8 / NT; ++it) {
        const int rr = (t >> 5) + 16 * it, c8 = 8 * (t & 31);
        const int m = m0 + EROWS * h + rr, n = n0 + c8;
        if constexpr (EPI == EPI_CE_STATS) {
          // Per row and 128-column half of the tile (16 threads): max and
          // sum of exp over the valid columns, and the target's logit.
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(sT + rr * TP + c8);
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(sT + rr * TP + c8 + 4);
          const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          float mx = -INFINITY;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (n + e < g.N) mx = fmaxf(mx, v[e]);
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
          float sm = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (n + e < g.N) sm += __expf(v[e] - mx);
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) sm += __shfl_xor(sm, o, 64);
          const int nh = n0 + 128 * ((t & 31) >> 4);
          if (m < g.M) {
            if ((t & 15) == 0 && nh < g.N) {
              const int gt = (g.col0 + nh) / 128;
              g.stats[((int64_t)m * g.stats_ld + gt) * 2 + 0] = mx;
              g.stats[((int64_t)m * g.stats_ld + gt) * 2 + 1] = sm;
            }
            const int tg = g.tgt[m] - g.col0 - n;
            if (tg >= 0 && tg < 8 && n + tg < g.N) g.tgt_logit[m] = v[tg];
          }
          continue;
        }
        if constexpr (EPI == EPI_CE_GRAD) {
          // dlogits = w_m (softmax - onehot(target)), bf16.
          if (m < g.M && n < g.N) {
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(sT + rr * TP + c8);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(sT + rr * TP + c8 + 4);
            const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            const float w = g.roww[m], ls = g.lse[m];
            const int tg = g.tgt[m] - g.col0 - n;
            float d[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              d[e] = 0.f;
              if (w != 0.f) {
                d[e] = __expf(v[e] - ls);
                if (tg == e) d[e] -= 1.f;
                d[e] *= w;
              }
            }
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = pack2_bf16(d[2 * e], d[2 * e + 1]);
            *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(C) + (int64_t)m * ldc + n) = o;
          }
          continue;
        }
        if (m < g.M && n < g.N) {
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(sT + rr * TP + c8);
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(sT + rr * TP + c8 + 4);
          float y[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] *= g.alpha;
          if constexpr (EPI == EPI_BF16) {
            if (g.R) {
              const u32x4 rv = *reinterpret_cast<const u32x4*>(g.R + (int64_t)m * g.ldr + n);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                y[2 * e] += bflo(rv[e]);
                y[2 * e + 1] += bfhi(rv[e]);
              }
            }
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = pack2_bf16(y[2 * e], y[2 * e + 1]);
            *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(C) + (int64_t)m * ldc + n) = o;
          } else if constexpr (EPI == EPI_F32) {
            float* c = reinterpret_cast<float*>(C) + (int64_t)m * ldc + n;
            *reinterpret_cast<f32x4*>(c) = f32x4{y[0], y[1], y[2], y[3]};
            *reinterpret_cast<f32x4*>(c + 4) = f32x4{y[4], y[5], y[6], y[7]};
          } else if constexpr (EPI == EPI_F32_ACC) {
            float* c = reinterpret_cast<float*>(C) + (int64_t)m * ldc + n;
            const f32x4 c0 = *reinterpret_cast<const f32x4*>(c), c1 = *reinterpret_cast<const f32x4*>(c + 4);
            *reinterpret_cast<f32x4*>(c) = f32x4{c0.x + y[0], c0.y + y[1], c0.z + y[2], c0.w + y[3]};
            *reinterpret_cast<f32x4*>(c + 4) = f32x4{c1.x + y[4], c1.y + y[5], c1.z + y[6], c1.w + y[7]};
          } else if constexpr (EPI == EPI_SWIGLU_BWD) {
            // y = dL/da for a = silu(g) * u: dg = y u silu'(g), du = y silu(g).
            const u32x4 gv = *reinterpret_cast<const u32x4*>(g.gu + (int64_t)m * g.ldgu + n);
            const u32x4 uv = *reinterpret_cast<const u32x4*>(g.gu + (int64_t)m * g.ldgu + g.I + n);
            u32x4 og, ou;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float dg[2], du[2];
#pragma unroll
              for (int p = 0; p < 2; ++p) {
                const float gg = p ? bfhi(gv[e]) : bflo(gv[e]);
                const float uu = p ? bfhi(uv[e]) : bflo(uv[e]);
                const float sg = sigm(gg);
                dg[p] = y[2 * e + p] * uu * sg * (1.f + gg * (1.f - sg));
                du[p] = y[2 * e + p] * (gg * sg);
              }
              og[e] = pack2_bf16(dg[0], dg[1]);
              ou[e] = pack2_bf16(du[0], du[1]);
            }
            uint16_t* out = reinterpret_cast<uint16_t*>(C) + (int64_t)m * ldc;
            *reinterpret_cast<u32x4*>(out + n) = og;
            *reinterpret_cast<u32x4*>(out + g.I + n) = ou;
          }
        }
      }
      __syncthreads();
    }
  }
};

template <int BL, int EPI>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
big_kernel(GemmArgs g, const float* __restrict__ cb) {
  // Separate arrays per stage, so the compiler can tell the DMA's target from
  // the stage the MFMAs read.
  __shared__ __attribute__((aligned(16))) uint16_t sA0[ATILE];
  __shared__ __attribute__((aligned(16))) uint16_t sA1[ATILE];
  __shared__ __attribute__((aligned(16))) uint16_t sB0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sB1[TILE];
  __shared__ __attribute__((aligned(16))) float2 lut2[256];
  const int t = threadIdx.x;
  if (t < 256) lut2[t] = make_float2(cb[t >> 4], cb[t & 15]);   // byte -> (high, low) nibble levels
  const int tiles_n = (g.N + BN - 1) / BN;
  const int m0 = (blockIdx.x / tiles_n) * BM, n0 = (blockIdx.x % tiles_n) * BN;
  Big<BL> k(g, sA0, sA1, sB0, sB1, lut2, m0, n0);
  __syncthreads();
  // Split-K: slice z takes contraction steps [nk z / ks, nk (z+1) / ks), the
  // LoRA term goes into slice 0 only, and each slice writes alpha * acc as a
  // float partial that gemm_reduce_epi sums in slice order.
  const int nk = g.K / BK, ks = g.ksplit > 1 ? g.ksplit : 1, z = blockIdx.z;
  bool lora = false;
  if constexpr (BL == B_NF4_NT || BL == B_NF4_NN)
    lora = (BL == B_NF4_NT && g.lora == LORA_FWD) || (BL == B_NF4_NN && g.lora == LORA_DX);
  if (z == 0 && lora) k.lora();
  if constexpr (EPI == EPI_CE_STATS || EPI == EPI_CE_GRAD) {
    k.mainloop(0, nk);
    k.template epilogue<EPI>(g.C, g.ldc);
    return;
  }
  // Slice 0 also runs the LoRA contraction (staged without prefetch; one
  // 64-deep step of it takes about kLoraSteps base steps), so slice 0 gets
  // kLoraSteps fewer base steps and the slices end closer together (when
  // every slice keeps at least 4 steps).  The boundaries depend on the shape
  // and split only, not on whether the LoRA term runs: with the adapters
  // disabled the base product is summed in the same order as with B = 0, and
  // the two outputs are identical.
  const int lu = ks > 1 && nk >= 4 * ks ? kLoraSteps : 0;
  const int U = nk + lu;
  k.mainloop(z == 0 ? 0 : U * z / ks - lu, U * (z + 1) / ks - lu);
  if (ks > 1)
    k.template epilogue<EPI_F32>(g.partial + (int64_t)z * g.M * g.N, g.N);
  else
    k.template epilogue<EPI>(g.C, g.ldc);
}

}  // namespace

const float* nf4_codebook_dev();  // defined in nf4.hip

namespace {
bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool fits31(int64_t bytes) { return bytes < 0x7fffffffLL; }
}  // namespace

bool gemm_big_ok(const GemmArgs& g, int bload, int epi) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0 || g.K % BK) return false;
  if (bload == B_BF16_NT) {
    if (epi != EPI_CE_STATS && epi != EPI_CE_GRAD) return false;
    if (g.ksplit > 1 || g.lora != LORA_NONE || g.lda % 8 || !a16(g.A) || !fits31((int64_t)g.M * g.lda * 2)) return false;
    if (!g.Bh || !a16(g.Bh) || g.ldb % 8 || g.ldb < g.K || g.N % 8 || !fits31((int64_t)g.N * g.ldb * 2)) return false;
    if (!g.tgt) return false;
    if (epi == EPI_CE_STATS) return g.stats && g.tgt_logit;
    return g.C && a16(g.C) && g.ldc % 8 == 0 && g.lse && g.roww;
  }
  if (g.ksplit > 1 && (!g.partial || !a16(g.partial) || g.N % 8 || g.ksplit > g.K / BK)) return false;
  if (g.lda % 8 || !a16(g.A) || !fits31((int64_t)g.M * g.lda * 2)) return false;
  if (bload == B_BF16_NN) {
    if (epi != EPI_F32 && epi != EPI_F32_ACC) return false;
    if (g.lora != LORA_NONE || !g.Bh || !a16(g.Bh) || g.ldb % 8 || g.ldb < g.N || g.N % BN) return false;
    if (!fits31((int64_t)g.K * g.ldb * 2)) return false;
    return g.C && a16(g.C) && g.ldc % 4 == 0;
  }
  if (g.ldq % 64 || !g.Bq || !g.Bs || !a16(g.C)) return false;
  if (bload == B_NF4_NT) {
    if (epi != EPI_BF16 || g.N % 8 || g.ldc % 8 || g.ldq < g.K) return false;
    if (!fits31((int64_t)g.N * g.ldq / 2)) return false;
    if (g.R && (g.ldr % 8 || !a16(g.R))) return false;
    if (g.lora == LORA_FWD) {
      if (g.K2 % 8 || g.lda2 % 8 || !a16(g.A2) || g.nmod < 1 || g.nmod > 4) return false;
      for (int i = 0; i < g.nmod; ++i)
        if (!a16(g.modB[i])) return false;
    }
    return true;
  }
  if (bload == B_NF4_NN) {
    if (g.N % BN || g.ldq < g.N || !fits31((int64_t)g.K * g.ldq / 2)) return false;
    if (epi == EPI_F32) {
      if (g.ldc % 4) return false;
    } else if (epi == EPI_BF16) {
      if (g.ldc % 8 || g.R) return false;
    } else if (epi == EPI_SWIGLU_BWD) {
      if (g.ldc % 8 || g.ldgu % 8 || g.I % 8 || !a16(g.gu)) return false;
    } else {
      return false;
    }
    if (g.lora == LORA_DX && (g.K2 % 8 || g.lda2 % 8 || g.ldb2 % 8 || !a16(g.A2) || !a16(g.B2)))
      return false;
    return true;
  }
  return false;
}

int gemm_big_launch(const GemmArgs& g, int bload, int epi, hipStream_t st) {
  if (!gemm_big_ok(g, bload, epi)) return -1;
  const float* cb = nf4_codebook_dev();
  const unsigned tiles = (unsigned)(((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN));
  const unsigned ks = g.ksplit > 1 ? (unsigned)g.ksplit : 1u;
  const dim3 grid(tiles, 1, ks);
  if (g.ev0) (void)hipEventRecord(g.ev0, st);
  if (bload == B_BF16_NT && epi == EPI_CE_STATS)
    hipLaunchKernelGGL((big_kernel<B_BF16_NT, EPI_CE_STATS>), grid, dim3(NT), 0, st, g, cb);
  else if (bload == B_BF16_NT)
    hipLaunchKernelGGL((big_kernel<B_BF16_NT, EPI_CE_GRAD>), grid, dim3(NT), 0, st, g, cb);
  else if (bload == B_BF16_NN && epi == EPI_F32)
    hipLaunchKernelGGL((big_kernel<B_BF16_NN, EPI_F32>), grid, dim3(NT), 0, st, g, cb);
  else if (bload == B_BF16_NN)
    hipLaunchKernelGGL((big_kernel<B_BF16_NN, EPI_F32_ACC>), grid, dim3(NT), 0, st, g, cb);
  else if (bload == B_NF4_NT)
    hipLaunchKernelGGL((big_kernel<B_NF4_NT, EPI_BF16>), grid, dim3(NT), 0, st, g, cb);
  else if (epi == EPI_F32)
    hipLaunchKernelGGL((big_kernel<B_NF4_NN, EPI_F32>), grid, dim3(NT), 0, st, g, cb);
  else if (epi == EPI_BF16)
    hipLaunchKernelGGL((big_kernel<B_NF4_NN, EPI_BF16>), grid, dim3(NT), 0, st, g, cb);
  else
    hipLaunchKernelGGL((big_kernel<B_NF4_NN, EPI_SWIGLU_BWD>), grid, dim3(NT), 0, st, g, cb);
  if (g.ev1) (void)hipEventRecord(g.ev1, st);
  if (ks > 1 && bload != B_BF16_NT) gemm_reduce_epi(g, epi, st);
  return 0;
}
