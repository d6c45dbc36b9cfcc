// Causal grouped-query attention for gfx950 with v_mfma_f32_16x16x32_bf16.
//
// Operand tiles (64 rows x head_dim bf16) go from global memory straight into
// LDS with buffer_load ... lds, double-buffered, in unpadded rows whose
// 16-byte chunks are XOR-swizzled by row.  Every product reads its operands
// from row-major tiles: 16-byte fragments where the contraction runs along a
// row, ds_read_b64_tr_b16 (the transposing LDS read of gfx950) where it runs
// down a column, so no tile is ever staged transposed.
//
// Forward: one workgroup per (32 query rows, kv head, sequence); wave w is the
// w-th query head of the kv head, so each K / V block is staged once for the
// heads that share it.  Scores are formed transposed, S^T = K Q^T, so a
// lane's accumulator column is its query row: the softmax statistics stay per
// lane (online max / sum in fp32) and the probabilities feed the P V product
// directly as the B operand.  P is rounded to bf16 for the product; the final
// division by the fp32 row sum follows it.  The log-sum-exp per row is saved.
//
// Backward (no atomics, fixed summation order):
//   dq kernel  -- per (32 query rows, kv head) as the forward: recompute P
//                 from the saved LSE, dP^T = V dO^T, dS = P (dP - D),
//                 dQ = dS K / sqrt(hd).
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

// 2^x with v_exp_f32 alone.  Every argument here is a logit minus a running
// maximum or the row's log-sum-exp (<= 0 up to rounding), so a result below
// 2^-126 is negligible next to the row's other terms and flushes to zero;
// exp2f would wrap each call in a range-scaling sequence for that case.
QLS_DEV float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32,
// l ^ 48) with gfx950's row-swap moves, which stay in the VALU: the 16-lane
// swap pairs rows 0-1 and 2-3, the 32-lane swap the two halves, and every lane
// ends with the same value, (r0 op r1) op (r2 op r3).
QLS_DEV float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
QLS_DEV float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

QLS_DEV u32x4 pack8(const f32x4& a, const f32x4& b) {
  return u32x4{pack2_bf16(a[0], a[1]), pack2_bf16(a[2], a[3]), pack2_bf16(b[0], b[1]),
               pack2_bf16(b[2], b[3])};
}

// ---- Unpadded swizzled tiles, filled by LDS-DMA.
// A tile is 64 rows x HD bf16 with rows of HD*2 bytes; the 16-byte chunk c of
// row r sits at chunk c ^ tswz(r).  gfx950's LDS has 64 banks, and a chunk's
// banks are fixed by its 16-byte granule index mod 16.  Measured: a 16-byte
// read runs at full rate when lanes 0-15 (and 32-47) cover 16 distinct
// granules and lane l + 16 hits the granule of lane l; the MFMA fragment
// reads here give lanes l and l + 16 adjacent chunks of one row, which no key
// can align, so they run at half rate whatever the key.  The key makes the 16
// rows read by each 16-lane group (one chunk index) distinct granules, which
// removed a further 2-way conflict: over 16 rows it is a bijection onto the
// 16 granules, and within each aligned 8 rows it sends the chunk pairs {2p,
// 2p+1} of the transposing reads to 8 different pairs.  HD = 128 (16 chunks
// per row): 2 (r mod 8) + bit 3 of r; HD = 64 (8 chunks per 128-byte row, two
// rows per 256 bytes): 2 ((r / 2) mod 4) + bit 3 of r.
template <int HD>
QLS_DEV int tswz(int r) {
  static_assert(HD == 64 || HD == 128, "head_dim 64 or 128");
  return HD == 128 ? (2 * (r & 7)) | ((r >> 3) & 1) : (2 * ((r >> 1) & 3)) | ((r >> 3) & 1);
}
template <int HD>
QLS_DEV int tpos(int r, int col) { return r * HD + 8 * ((col >> 3) ^ tswz<HD>(r)) + (col & 7); }

// Rows [r0, r0 + 64) of a [S x ld] operand (columns [0, HD) at base) into a
// tile: one 16-byte DMA per lane, 1 KB per instruction, the instructions of
// the tile spread over the workgroup's nw waves.  Rows at or past S read 0
// (the resource ends at row S).
template <int HD>
QLS_DEV void dma_tile(uint16_t* tile, const uint16_t* base, int64_t ld, int r0, int S, int wave, int nw, int lane) {
  constexpr int CH = HD / 8, RPI = 64 / CH, NI = 64 / RPI;   // chunks per row, rows and instructions per tile
  const int64_t rows = S - r0 > 0 ? S - r0 : 0;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(base + (int64_t)r0 * ld), (short)0,
      (int)(rows * ld * 2 > 0x7fffffffLL ? 0x7fffffffLL : rows * ld * 2), 0x00020000);
  if (nw == 4) {
    // Four waves (the 8B shape's 32 / 8 heads, and the dK / dV kernel):
    // unrolled, wave w issues instructions w, w + 4, ...; the swizzle key of
    // a lane's row is the same in all of them (the rows are 4 RPI apart, a
    // multiple of 16), so only the scalar row offset changes.
    const int r = RPI * wave + lane / CH;
    const uint32_t v = (uint32_t)((r * ld + 8 * ((lane % CH) ^ tswz<HD>(r))) * 2);
#pragma unroll
    for (int u = 0; u < NI / 4; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(tile + (wave + 4 * u) * 512),
                                               16, v, (uint32_t)(4 * RPI * u * ld * 2), 0, 0);
    return;
  }
  for (int i = wave; i < NI; i += nw) {
    const int r = RPI * i + lane / CH;
    const int c = (lane % CH) ^ tswz<HD>(r);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(tile + i * 512), 16,
                                             (uint32_t)((r * ld + 8 * c) * 2), 0, 0, 0);
  }
}

// 16-byte MFMA fragment: row r, columns [col, col + 8).
template <int HD>
QLS_DEV u32x4 frag(const uint16_t* tile, int r, int col) {
  return *reinterpret_cast<const u32x4*>(tile + tpos<HD>(r, col));
}

// Transposed fragment from a row-major tile with ds_read_b64_tr_b16: within
// each 16-lane group, lane j receives element i from the lane 4i + j/4 of
// its group, element j % 4 of that lane's 8-byte read.  A lane of group g4
// reading row kb + c16/4, columns col0 + 4 (c16 % 4) therefore returns
// tile[kb + i][col0 + c16], i = 0..3.  Two reads give the 8 contraction
// slots {k0 + 4 g4 + 0..3, k0 + 16 + 4 g4 + 0..3} of column col0 + c16.
template <int HD>
QLS_DEV u32x4 frag_t(const uint16_t* tile, int k0, int col0, int g4, int c16) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const int r = k0 + 4 * g4 + (c16 >> 2), col = col0 + 4 * (c16 & 3);
  const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(tile + tpos<HD>(r, col)));
  const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(tile + tpos<HD>(r + 16, col)));
  const u32x2 x = __builtin_bit_cast(u32x2, a), y = __builtin_bit_cast(u32x2, b);
  return u32x4{x.x, x.y, y.x, y.y};
}

// Work order over the grid's x (rank: 0 = the most key / query blocks to
// walk) and y (heads): workgroups are dispatched in linear (x, y) order, so
// rank r of every head goes before rank r + 1 of any, and the longest
// workgroups start first instead of those of the last heads starting last.
QLS_DEV void rank_major(int* rank, int* y) {
  const int id = (int)(blockIdx.x + gridDim.x * blockIdx.y);
  *rank = id / (int)gridDim.y;
  *y = id % (int)gridDim.y;
}

QLS_DEV void wait_dma() {
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (0 << 8) | (0 << 14));   // vmcnt(0) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Forward, one workgroup per (32 query rows, kv head, sequence): wave w is
// query head kv * G + w (the G heads that share the kv head), so each K / V
// block is staged once for all of them.  Key blocks of 64 are double-buffered
// in LDS by DMA; a wave's 32 rows are two 16-row groups that share every K
// and V fragment it reads.
template <int HD>
__global__ void __launch_bounds__(512) attn_fwd_k(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK0[64 * HD];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[64 * HD];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[64 * HD];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[64 * HD];
  const int G = a.H / a.KV;
  const int nqb = (a.S + 31) / 32;
  int rank, g;
  rank_major(&rank, &g);
  const int qb = nqb - 1 - rank;                  // long rows first
  const int b = blockIdx.z;
  const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6), g4 = lane >> 4, c16 = lane & 15;
  const int h = g * G + w;
  const int q0 = qb * 32;
  const int64_t tb = (int64_t)b * a.S;
  const uint16_t* Q = a.qkv + tb * a.ld + a.q_off + (int64_t)h * HD;
  const uint16_t* K = a.qkv + tb * a.ld + a.k_off + (int64_t)g * HD;
  const uint16_t* V = a.qkv + tb * a.ld + a.v_off + (int64_t)g * HD;
  const int nkb = min((q0 + 31) / 64 + 1, (a.S + 63) / 64);

  dma_tile<HD>(sK0, K, a.ld, 0, a.S, w, G, lane);
  dma_tile<HD>(sV0, V, a.ld, 0, a.S, w, G, lane);

  int myq[2];
  u32x4 qf[2][HD / 32];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
    myq[qg] = q0 + 16 * qg + c16;
#pragma unroll
    for (int s = 0; s < HD / 32; ++s)
      qf[qg][s] = myq[qg] < a.S ? *reinterpret_cast<const u32x4*>(Q + (int64_t)myq[qg] * a.ld + 32 * s + 8 * g4)
                                : u32x4{0, 0, 0, 0};
  }
  f32x4 o[2][HD / 16];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg)
#pragma unroll
    for (int i = 0; i < HD / 16; ++i) o[qg][i] = f32x4{0, 0, 0, 0};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  const float c = a.scale * kLog2e;

  auto block = [&](const uint16_t* sK, const uint16_t* sV, int k0) {
    f32x4 sc[2][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[0][j] = f32x4{0, 0, 0, 0};
      sc[1][j] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < HD / 32; ++s) {
        const u32x4 ka = frag<HD>(sK, 16 * j + c16, 32 * s + 8 * g4);
        sc[0][j] = mfma16(ka, qf[0][s], sc[0][j]);
        sc[1][j] = mfma16(ka, qf[1][s], sc[1][j]);
      }
    }
    // Running statistics in the log2 domain of the scaled scores: the
    // maximum is taken on the raw scores (the scale is positive) and each
    // probability is exp2(fma(score, scale log2 e, -max)).
    u32x4 pf[2][2];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
      float mloc = -INFINITY;
      // Only the block that holds the diagonal (the last one) has keys to mask;
      // every earlier block lies wholly at or below the workgroup's first row.
      if (k0 + 63 > q0) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = k0 + 16 * j + 4 * g4 + i;
            if (!(key <= myq[qg] && key < a.S)) sc[qg][j][i] = -INFINITY;
          }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, sc[qg][j][i]);
      mloc = rows_max(mloc);
      const float m_new = fmaxf(m_run[qg], mloc * c);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fexp2(m_run[qg] - m_use);
      float ls = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = fexp2(fmaf(sc[qg][j][i], c, -m_use));
          sc[qg][j][i] = p;
          ls += p;
        }
      l_run[qg] = l_run[qg] * alpha + ls;
      // alpha is exactly 1 on every row whose maximum did not move; the
      // rescale of the output accumulators is skipped when that holds for
      // the whole wave (the usual case once a row has seen a few blocks).
      if (__builtin_amdgcn_ballot_w64(m_new != m_run[qg])) {
#pragma unroll
        for (int i = 0; i < HD / 16; ++i) o[qg][i] *= alpha;
      }
      m_run[qg] = m_new;
      pf[qg][0] = pack8(sc[qg][0], sc[qg][1]);
      pf[qg][1] = pack8(sc[qg][2], sc[qg][3]);
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int hb = 0; hb < HD / 16; ++hb) {
        const u32x4 va = frag_t<HD>(sV, 32 * tt, 16 * hb, g4, c16);
        o[0][hb] = mfma16(va, pf[0][tt], o[0][hb]);
        o[1][hb] = mfma16(va, pf[1][tt], o[1][hb]);
      }
  };

  for (int kb = 0; kb < nkb; kb += 2) {
    wait_dma();                                       // block kb in stage 0; stage 1 free
    if (kb + 1 < nkb) {
      dma_tile<HD>(sK1, K, a.ld, 64 * (kb + 1), a.S, w, G, lane);
      dma_tile<HD>(sV1, V, a.ld, 64 * (kb + 1), a.S, w, G, lane);
    }
    block(sK0, sV0, 64 * kb);
    if (kb + 1 >= nkb) break;
    wait_dma();                                       // block kb+1 in stage 1; stage 0 free
    if (kb + 2 < nkb) {
      dma_tile<HD>(sK0, K, a.ld, 64 * (kb + 2), a.S, w, G, lane);
      dma_tile<HD>(sV0, V, a.ld, 64 * (kb + 2), a.S, w, G, lane);
    }
    block(sK1, sV1, 64 * (kb + 1));
  }
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
    const float lt = rows_sum(l_run[qg]);
    if (myq[qg] < a.S) {
      const float inv = 1.f / lt;
      uint16_t* O = a.out + (tb + myq[qg]) * a.ldo + (int64_t)h * HD;
#pragma unroll
      for (int hb = 0; hb < HD / 16; ++hb) {
        const u32x2 v = {pack2_bf16(o[qg][hb][0] * inv, o[qg][hb][1] * inv),
                         pack2_bf16(o[qg][hb][2] * inv, o[qg][hb][3] * inv)};
        *reinterpret_cast<u32x2*>(O + 16 * hb + 4 * g4) = v;
      }
      if (g4 == 0) a.lse[((int64_t)b * a.H + h) * a.S + myq[qg]] = m_run[qg] * kLn2 + logf(lt);
    }
  }
}

// D[b,h,q] = sum_j dO[q, h, j] * O[q, h, j]; HD/8 lanes per (row, head), 8
// elements (16 bytes) of each operand per lane.
template <int HD>
__global__ void attn_pre_k(const uint16_t* __restrict__ dO, const uint16_t* __restrict__ O,
                           int64_t ld, int S, int H, int T, float* __restrict__ D) {
  constexpr int L = HD / 8;                       // lanes per (row, head): 16 or 8
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t pair = gid / L;
  const int c = (int)(gid % L);
  const bool ok = pair < (int64_t)T * H;
  const int tok = ok ? (int)(pair / H) : 0, h = ok ? (int)(pair % H) : 0;
  float acc = 0.f;
  if (ok) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(dO + (int64_t)tok * ld + h * HD + 8 * c);
    const u32x4 o = *reinterpret_cast<const u32x4*>(O + (int64_t)tok * ld + h * HD + 8 * c);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc += bflo(a[q]) * bflo(o[q]) + bfhi(a[q]) * bfhi(o[q]);
  }
#pragma unroll
  for (int off = 1; off < L; off <<= 1) acc += __shfl_xor(acc, off, 64);
  if (ok && c == 0) {
    const int b = tok / S, s = tok % S;
    D[((int64_t)b * H + h) * S + s] = acc;
  }
}

// dQ, one workgroup per (32 query rows, kv head, sequence), wave w = query head
// kv * G + w; K and V blocks of 64 keys double-buffered by DMA and shared by
// the G heads.  Per block: S^T = K Q^T and dP^T = V dO^T from row fragments,
// P from the saved LSE, dS = P (dP - D), dQ += dS K with K read transposed.
template <int HD>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) attn_dq_k(AttnBwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK0[64 * HD];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[64 * HD];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[64 * HD];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[64 * HD];
  const int G = a.H / a.KV;
  const int nqb = (a.S + 31) / 32;
  int rank, g;
  rank_major(&rank, &g);
  const int qb = nqb - 1 - rank;                  // long rows first
  const int b = blockIdx.z;
  const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6), g4 = lane >> 4, c16 = lane & 15;
  const int h = g * G + w;
  const int q0 = qb * 32;
  const int64_t tb = (int64_t)b * a.S;
  const uint16_t* Q = a.qkv + tb * a.ld + a.q_off + (int64_t)h * HD;
  const uint16_t* K = a.qkv + tb * a.ld + a.k_off + (int64_t)g * HD;
  const uint16_t* V = a.qkv + tb * a.ld + a.v_off + (int64_t)g * HD;
  const uint16_t* dO = a.dO + tb * a.lddo + (int64_t)h * HD;
  const int nkb = min((q0 + 31) / 64 + 1, (a.S + 63) / 64);

  dma_tile<HD>(sK0, K, a.ld, 0, a.S, w, G, lane);
  dma_tile<HD>(sV0, V, a.ld, 0, a.S, w, G, lane);

  int myq[2];
  float lse2[2], Dq[2];
  u32x4 qf[2][HD / 32], df[2][HD / 32];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
    myq[qg] = q0 + 16 * qg + c16;
    const bool ok = myq[qg] < a.S;
#pragma unroll
    for (int s = 0; s < HD / 32; ++s) {
      qf[qg][s] = ok ? *reinterpret_cast<const u32x4*>(Q + (int64_t)myq[qg] * a.ld + 32 * s + 8 * g4) : u32x4{0, 0, 0, 0};
      df[qg][s] = ok ? *reinterpret_cast<const u32x4*>(dO + (int64_t)myq[qg] * a.lddo + 32 * s + 8 * g4) : u32x4{0, 0, 0, 0};
    }
    const int64_t rid = ((int64_t)b * a.H + h) * a.S + myq[qg];
    lse2[qg] = ok ? a.lse[rid] * kLog2e : 0.f;
    Dq[qg] = ok ? a.D[rid] : 0.f;
  }
  const float c = a.scale * kLog2e;
  f32x4 dq[2][HD / 16];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg)
#pragma unroll
    for (int i = 0; i < HD / 16; ++i) dq[qg][i] = f32x4{0, 0, 0, 0};

  auto block = [&](const uint16_t* sK, const uint16_t* sV, int k0) {
    f32x4 sc[2][4], dp[2][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int qg = 0; qg < 2; ++qg) { sc[qg][j] = f32x4{0, 0, 0, 0}; dp[qg][j] = f32x4{0, 0, 0, 0}; }
#pragma unroll
      for (int s = 0; s < HD / 32; ++s) {
        const u32x4 ka = frag<HD>(sK, 16 * j + c16, 32 * s + 8 * g4);
        const u32x4 va = frag<HD>(sV, 16 * j + c16, 32 * s + 8 * g4);
#pragma unroll
        for (int qg = 0; qg < 2; ++qg) {
          sc[qg][j] = mfma16(ka, qf[qg][s], sc[qg][j]);
          dp[qg][j] = mfma16(va, df[qg][s], dp[qg][j]);
        }
      }
    }
    u32x4 dsf[2][2];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + 16 * j + 4 * g4 + i;
          const float p = (key <= myq[qg] && key < a.S && myq[qg] < a.S) ? fexp2(sc[qg][j][i] * c - lse2[qg]) : 0.f;
          sc[qg][j][i] = p * (dp[qg][j][i] - Dq[qg]);     // dS (rounded to bf16 below)
        }
      dsf[qg][0] = pack8(sc[qg][0], sc[qg][1]);
      dsf[qg][1] = pack8(sc[qg][2], sc[qg][3]);
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int hb = 0; hb < HD / 16; ++hb) {
        const u32x4 kt = frag_t<HD>(sK, 32 * tt, 16 * hb, g4, c16);
        dq[0][hb] = mfma16(dsf[0][tt], kt, dq[0][hb]);
        dq[1][hb] = mfma16(dsf[1][tt], kt, dq[1][hb]);
      }
  };

  for (int kb = 0; kb < nkb; kb += 2) {
    wait_dma();
    if (kb + 1 < nkb) {
      dma_tile<HD>(sK1, K, a.ld, 64 * (kb + 1), a.S, w, G, lane);
      dma_tile<HD>(sV1, V, a.ld, 64 * (kb + 1), a.S, w, G, lane);
    }
    block(sK0, sV0, 64 * kb);
    if (kb + 1 >= nkb) break;
    wait_dma();
    if (kb + 2 < nkb) {
      dma_tile<HD>(sK0, K, a.ld, 64 * (kb + 2), a.S, w, G, lane);
      dma_tile<HD>(sV0, V, a.ld, 64 * (kb + 2), a.S, w, G, lane);
    }
    block(sK1, sV1, 64 * (kb + 1));
  }
  // dq[qg][hb][i] = dQ[q0 + 16 qg + 4 g4 + i][16 hb + c16]
#pragma unroll
  for (int qg = 0; qg < 2; ++qg)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = q0 + 16 * qg + 4 * g4 + i;
      if (q >= a.S) continue;
      float* dst = a.dq + (tb + q) * a.lddq + (int64_t)h * HD;
#pragma unroll
      for (int hb = 0; hb < HD / 16; ++hb) dst[16 * hb + c16] = dq[qg][hb][i] * a.scale;
    }
}

// dK, dV: one workgroup per (64 keys, query head, sequence), wave w owns keys
// k0 + 16 w .. + 15 and walks the query blocks on or below the diagonal; Q and
// dO blocks of 64 rows double-buffered by DMA (with their LSE and D values),
// read as row fragments for S = Q K^T, dP = dO V^T and transposed for
// dV += P^T dO and dK += dS^T Q.  One float partial per query head; the sum
// over the heads that share a kv head is taken in head order by the RoPE
// backward that consumes dK and dV.
template <int HD>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) attn_dkv_k(AttnBwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sQ0[64 * HD];
  __shared__ __attribute__((aligned(16))) uint16_t sQ1[64 * HD];
  __shared__ __attribute__((aligned(16))) uint16_t sO0[64 * HD];
  __shared__ __attribute__((aligned(16))) uint16_t sO1[64 * HD];
  __shared__ __attribute__((aligned(16))) float sL[2][64];
  __shared__ __attribute__((aligned(16))) float sD[2][64];
  const int nqb = (a.S + BQ - 1) / BQ;
  int kb, h;
  rank_major(&kb, &h);                            // key block 0 walks the most query blocks
  const int b = blockIdx.z;
  const int g = h / (a.H / a.KV);
  const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6), g4 = lane >> 4, c16 = lane & 15;
  const int k0 = kb * BQ;
  const int myk = k0 + 16 * w + c16;
  const int64_t tb = (int64_t)b * a.S;
  const uint16_t* K = a.qkv + tb * a.ld + a.k_off + (int64_t)g * HD;
  const uint16_t* V = a.qkv + tb * a.ld + a.v_off + (int64_t)g * HD;
  const uint16_t* Q = a.qkv + tb * a.ld + a.q_off + (int64_t)h * HD;
  const uint16_t* dO = a.dO + tb * a.lddo + (int64_t)h * HD;
  const int64_t rid0 = ((int64_t)b * a.H + h) * a.S;

  // The LSE and D rows of a query block are loaded into registers one block
  // ahead (wave 0, one row per lane) and written to LDS when the block is
  // staged, so no wave waits on their latency.
  float nl = 0.f, nd = 0.f;
  auto load_ld = [&](int q0) {
    const int q = q0 + t;
    if (t < BQ && q < a.S) {
      nl = a.lse[rid0 + q];
      nd = a.D[rid0 + q];
    } else {
      nl = 0.f;
      nd = 0.f;
    }
  };
  auto stage = [&](uint16_t* sq, uint16_t* so, int st, int q0) {
    if (t < BQ) {
      sL[st][t] = nl * kLog2e;
      sD[st][t] = nd;
    }
    load_ld(q0 + BQ);
    asm volatile("" ::: "memory");
    dma_tile<HD>(sq, Q, a.ld, q0, a.S, w, NT / 64, lane);
    dma_tile<HD>(so, dO, a.lddo, q0, a.S, w, NT / 64, lane);
  };
  load_ld(k0);
  stage(sQ0, sO0, 0, k0);

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

  auto block = [&](const uint16_t* sq, const uint16_t* so, int st, int q0) {
    f32x4 sc[4], dp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[j] = f32x4{0, 0, 0, 0};
      dp[j] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < HD / 32; ++s) {
        sc[j] = mfma16(frag<HD>(sq, 16 * j + c16, 32 * s + 8 * g4), kf[s], sc[j]);
        dp[j] = mfma16(frag<HD>(so, 16 * j + c16, 32 * s + 8 * g4), vf[s], dp[j]);
      }
    }
    // The fragments of row block j+1 are read while the MFMAs of block j
    // run, and no further ahead: reading all 32 up front would hold 128
    // registers and spill.
    constexpr int NRD = HD / 16;                 // fragment reads per row block
    __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, NRD, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NRD, 0);
    // Scheduling barriers between the phases keep the compiler from hoisting
    // the next phase's LDS reads across them, which raises register pressure.
    __builtin_amdgcn_sched_barrier(0);
    // sc[j][i] = S[q = q0 + 16j + 4g4 + i][key = myk]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sL[st][16 * j + 4 * g4]);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sD[st][16 * j + 4 * g4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = q0 + 16 * j + 4 * g4 + i;
        const float p = (myk <= q && q < a.S && myk < a.S) ? fexp2(sc[j][i] * c - l4[i]) : 0.f;
        sc[j][i] = p;
        dp[j][i] = p * (dp[j][i] - d4[i]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const u32x4 pf = pack8(sc[2 * tt], sc[2 * tt + 1]);
      const u32x4 dsf = pack8(dp[2 * tt], dp[2 * tt + 1]);
#pragma unroll
      for (int hb = 0; hb < HD / 16; ++hb) {
        dv[hb] = mfma16(pf, frag_t<HD>(so, 32 * tt, 16 * hb, g4, c16), dv[hb]);
        dk[hb] = mfma16(dsf, frag_t<HD>(sq, 32 * tt, 16 * hb, g4, c16), dk[hb]);
      }
      // Transposed fragments (4 reads per column block) two blocks ahead.
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int hb = 0; hb < HD / 16 - 2; ++hb) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  for (int qb = kb; qb < nqb; qb += 2) {
    wait_dma();
    if (qb + 1 < nqb) stage(sQ1, sO1, 1, BQ * (qb + 1));
    block(sQ0, sO0, 0, BQ * qb);
    if (qb + 1 >= nqb) break;
    wait_dma();
    if (qb + 2 < nqb) stage(sQ0, sO0, 0, BQ * (qb + 2));
    block(sQ1, sO1, 1, BQ * (qb + 1));
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

// out[t][g hd + j] = sum over i < G, in order, of part[t][(g G + i) hd + j].
__global__ void group_sum_k(const float* __restrict__ part, float* __restrict__ out, int64_t n, int H, int KV,
                            int hd) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int kvd = KV * hd, G = H / KV;
  const int64_t t = idx / kvd;
  const int e = (int)(idx % kvd), g = e / hd, j = e % hd;
  const float* src = part + t * (int64_t)H * hd + (int64_t)g * G * hd + j;
  float acc = 0.f;
  for (int i = 0; i < G; ++i) acc += src[(int64_t)i * hd];
  out[idx] = acc;
}

}  // namespace

void attn_group_sum(const float* part, float* out, int T, int H, int KV, int hd, hipStream_t st) {
  const int64_t n = (int64_t)T * KV * hd;
  if (n <= 0) return;
  hipLaunchKernelGGL(group_sum_k, dim3((unsigned)ceil_div64(n, 256)), dim3(256), 0, st, part, out, n, H, KV, hd);
}

// Heads per kv head the kernels take: one wave each, up to 8 per workgroup.
static bool group_ok(int H, int KV) { return KV > 0 && H % KV == 0 && H / KV <= 8; }

int attn_fwd(const AttnArgs& a, int B, hipStream_t st) {
  if (!group_ok(a.H, a.KV) || a.ld % 8 || a.q_off % 8 || a.k_off % 8 || a.v_off % 8) return -1;
  const dim3 grid((a.S + 31) / 32, a.KV, B), block(64 * (a.H / a.KV));
  if (a.hd == 128) hipLaunchKernelGGL(attn_fwd_k<128>, grid, block, 0, st, a);
  else if (a.hd == 64) hipLaunchKernelGGL(attn_fwd_k<64>, grid, block, 0, st, a);
  else return -1;
  return 0;
}

int attn_bwd(const AttnBwdArgs& a, int B, hipStream_t st) {
  const int T = B * a.S;
  const int64_t waves = (int64_t)T * a.H;
  if (!group_ok(a.H, a.KV) || a.ld % 8 || a.lddo % 8 || a.q_off % 8 || a.k_off % 8 || a.v_off % 8) return -1;
  const dim3 gq((a.S + 31) / 32, a.KV, B), gk((a.S + BQ - 1) / BQ, a.H, B), bq(64 * (a.H / a.KV));
  if (a.hd == 128) {
    hipLaunchKernelGGL(attn_pre_k<128>, dim3((unsigned)ceil_div64(waves * 16, 256)), dim3(256), 0, st,
                       a.dO, a.O, a.lddo, a.S, a.H, T, a.D);
    hipLaunchKernelGGL(attn_dq_k<128>, gq, bq, 0, st, a);
    hipLaunchKernelGGL(attn_dkv_k<128>, gk, dim3(NT), 0, st, a);
  } else if (a.hd == 64) {
    hipLaunchKernelGGL(attn_pre_k<64>, dim3((unsigned)ceil_div64(waves * 8, 256)), dim3(256), 0, st,
                       a.dO, a.O, a.lddo, a.S, a.H, T, a.D);
    hipLaunchKernelGGL(attn_dq_k<64>, gq, bq, 0, st, a);
    hipLaunchKernelGGL(attn_dkv_k<64>, gk, dim3(NT), 0, st, a);
  } else {
    return -1;
  }
  return 0;
}
