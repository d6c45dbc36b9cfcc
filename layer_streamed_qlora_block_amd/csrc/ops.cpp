// Host-side orchestration of GEMM launches for the QLoRA linears.
#include <algorithm>

#include "gemm.h"
#include "internal.h"
#include "ops.h"

namespace {

constexpr int kSkinnyTarget = 1024;  // workgroups to aim for with split-K
constexpr int kMaxSplit = 64;
constexpr int64_t kBigPartial = 512LL * 4096 * 8;    // floats available to a split big GEMM (64 MB)

// Skinny products (one side is the LoRA rank): each k-tile iteration of a
// 64 x 64 tile is latency-bound, so the contraction is split into slices of at
// least 4 k-tiles, up to ~1024 workgroups (partials <= 1024 * 64 * 64 floats).
int pick_split(int M, int N, int K) {
  const int64_t tiles = cdiv(M, 64) * cdiv(N, 64);
  const int nk = (int)cdiv(K, 64);
  const int64_t by_tiles = std::max<int64_t>(1, kSkinnyTarget / std::max<int64_t>(tiles, 1));
  return (int)std::max<int64_t>(1, std::min<int64_t>({(int64_t)nk / 4, by_tiles, (int64_t)kMaxSplit}));
}

int skinny(int aload, const uint16_t* A, int64_t lda, int bload, const uint16_t* B, int64_t ldb,
           int M, int N, int K, float alpha, int mode, void* C, int64_t ldc, float* part,
           hipStream_t st) {
  GemmArgs g{};
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda;
  g.Bh = B; g.ldb = ldb;
  g.ksplit = pick_split(M, N, K);
  if (g.ksplit == 1) {
    g.alpha = alpha;
    g.C = C; g.ldc = ldc;
    return gemm_launch(g, aload, bload, mode == 0 ? EPI_BF16 : EPI_F32, 64, st);
  }
  g.partial = part;
  if (gemm_launch(g, aload, bload, EPI_PARTIAL, 64, st)) return -1;
  gemm_reduce(part, g.ksplit, M, N, alpha, mode, C, ldc, st);
  return 0;
}

}  // namespace

// Split-K for the 128 x 128 GEMMs: aim for ~512 workgroups when M is small,
// keep at least 8 k-tiles per split and the partials within kBigPartial.
int big_split(int M, int N, int K) {
  const int64_t tiles = cdiv(M, 128) * cdiv(N, 128);
  if (tiles >= 384) return 1;
  const int nk = (int)cdiv(K, 64);
  int ks = (int)std::min<int64_t>(cdiv(512, tiles), nk / 8);
  while (ks > 1 && (int64_t)M * N * ks > kBigPartial) --ks;
  return std::max(1, std::min(ks, 16));
}

// One 256 x 256 workgroup (512 threads, ~138 KB of LDS) fills a CU, so a
// launch of at least 192 of them (one wave over the 256 CUs, >= 75% of them
// busy) runs the big kernels.  With fewer output tiles the contraction is
// split into up to 256 / tiles slices of at least 12 steps of 64, partials
// within kBigPartial; when that still leaves fewer than 192 workgroups the
// 128 x 128 kernels (several workgroups per CU) take the GEMM.
GemmPlan plan_nf4(int M, int N, int K, bool can_split) {
  const int64_t tiles = cdiv(M, 256) * cdiv(N, 256);
  if (tiles >= 192) return {true, 1};
  if (can_split) {
    const int nk = K / 64;
    for (int ks = (int)std::min<int64_t>(256 / std::max<int64_t>(tiles, 1), nk / 12); ks >= 2; --ks)
      if (tiles * ks >= 192 && (int64_t)M * N * ks <= kBigPartial) return {true, ks};
  }
  return {false, can_split ? big_split(M, N, K) : 1};
}

int64_t skinny_partial_floats(int64_t max_mn) {
  return std::max<int64_t>({max_mn, (int64_t)kSkinnyTarget * 64 * 64, kBigPartial});
}

int64_t linear_ws_bytes(int T, int N, int K, int r) {
  const int64_t du = align_up((int64_t)T * r * 2, 256);
  const int64_t mn = std::max({(int64_t)T * r, (int64_t)N * r, (int64_t)r * K});
  return du + 4 * skinny_partial_floats(mn);
}

int skinny_U(const uint16_t* x, int64_t ldx, int T, int K, const uint16_t* A, int n, uint16_t* U,
             int64_t ldu, float* part, hipStream_t st) {
  return skinny(A_ROW, x, ldx, B_BF16_NT, A, K, T, n, K, 1.f, 0, U, ldu, part, st);
}

int skinny_du(const uint16_t* dy, int64_t lddy, int T, int N, const uint16_t* B, int r, float s,
              uint16_t* du, int64_t lddu, float* part, hipStream_t st) {
  return skinny(A_ROW, dy, lddy, B_BF16_NN, B, r, T, r, N, s, 0, du, lddu, part, st);
}

int skinny_dB(const uint16_t* dy, int64_t lddy, int T, int N, const uint16_t* u, int64_t ldu,
              float s, float* dB, float* part, hipStream_t st, int r) {
  const int rr = r > 0 ? r : (int)ldu;
  return skinny(A_COL, dy, lddy, B_BF16_NN, u, ldu, N, rr, T, s, 1, dB, rr, part, st);
}

int skinny_dA(const uint16_t* du, int64_t lddu, int T, int r, const uint16_t* x, int64_t ldx, int K,
              float* dA, float* part, hipStream_t st) {
  return skinny(A_COL, du, lddu, B_BF16_NN, x, ldx, r, K, T, 1.f, 1, dA, K, part, st);
}

int skinny_dA_multi(const uint16_t* du, int64_t lddu, int T, int r, int nmod, const uint16_t* x, int64_t ldx,
                    int K, float* const* dA, float* part, int64_t part_floats, hipStream_t st) {
  if (nmod < 1 || nmod > 4) return -1;
  GemmArgs g{};
  g.M = nmod * r; g.N = K; g.K = T;
  g.A = du; g.lda = lddu;
  g.Bh = x; g.ldb = ldx;
  g.ksplit = pick_split(g.M, g.N, g.K);
  if (gemm_partial_elems(g.M, g.N, g.ksplit) > part_floats) return -1;
  g.partial = part;
  if (gemm_launch(g, A_COL, B_BF16_NN, EPI_PARTIAL, 64, st)) return -1;
  return gemm_reduce_rows(part, g.ksplit, g.M, g.N, 1.f, dA, r, K, st);
}

SkinnyProd sk_du(const uint16_t* dy, int64_t lddy, int T, int N, const uint16_t* B, int r, float s, uint16_t* du,
                 int64_t lddu) {
  SkinnyProd p{};
  p.aload = A_ROW; p.bload = B_BF16_NN;
  p.A = dy; p.lda = lddy; p.B = B; p.ldb = r;
  p.M = T; p.N = r; p.K = N;
  p.alpha = s; p.mode = 0; p.C = du; p.ldc = lddu;
  return p;
}

SkinnyProd sk_dB(const uint16_t* dy, int64_t lddy, int T, int N, const uint16_t* u, int64_t ldu, float s, float* dB,
                 int r) {
  SkinnyProd p{};
  p.aload = A_COL; p.bload = B_BF16_NN;
  p.A = dy; p.lda = lddy; p.B = u; p.ldb = ldu;
  p.M = N; p.N = r; p.K = T;
  p.alpha = s; p.mode = 1; p.C = dB; p.ldc = r;
  return p;
}

SkinnyProd sk_dA_multi(const uint16_t* du, int64_t lddu, int T, int r, int nmod, const uint16_t* x, int64_t ldx,
                       int K, float* const* dA) {
  SkinnyProd p{};
  p.aload = A_COL; p.bload = B_BF16_NN;
  p.A = du; p.lda = lddu; p.B = x; p.ldb = ldx;
  p.M = nmod * r; p.N = K; p.K = T;
  p.alpha = 1.f; p.mode = 1; p.ldc = K;
  p.rows = r;
  for (int i = 0; i < nmod && i < 4; ++i) p.Crows[i] = dA[i];
  return p;
}

int64_t skinny_group_floats(const SkinnyProd* p, int n) {
  int64_t off = 0;
  for (int i = 0; i < n; ++i)
    off += align_up(gemm_partial_elems(p[i].M, p[i].N, pick_split(p[i].M, p[i].N, p[i].K)), 64);
  return off;
}

int skinny_group(const SkinnyProd* p, int n, float* part, int64_t part_floats, hipStream_t st) {
  if (n < 1 || n > kMaxGroup) return -1;
  static const int kinds[3][2] = {{A_ROW, B_BF16_NN}, {A_COL, B_BF16_NN}, {A_ROW, B_BF16_NT}};
  GemmArgs args[kMaxGroup];
  ReduceGroup rg{};
  int64_t off = 0;
  for (int i = 0; i < n; ++i) {
    const SkinnyProd& q = p[i];
    if (q.rows > 0 && (q.M % q.rows || q.M / q.rows > 4)) return -1;
    GemmArgs& g = args[i];
    g = GemmArgs{};
    g.M = q.M; g.N = q.N; g.K = q.K;
    g.A = q.A; g.lda = q.lda;
    g.Bh = q.B; g.ldb = q.ldb;
    g.ksplit = pick_split(q.M, q.N, q.K);
    g.partial = part + off;
    off += align_up(gemm_partial_elems(q.M, q.N, g.ksplit), 64);
    ReduceJob& j = rg.j[i];
    j.P = g.partial; j.ks = g.ksplit; j.M = q.M; j.N = q.N; j.alpha = q.alpha; j.mode = q.mode;
    j.C = q.C; j.ldc = q.ldc; j.rows = q.rows;
    for (int c = 0; c < 4; ++c) j.Cr[c] = q.Crows[c];
    rg.end[i] = (i ? rg.end[i - 1] : 0) + (int64_t)q.M * q.N;
  }
  rg.n = n;
  if (off > part_floats) return -1;
  for (const auto& kd : kinds) {
    GemmGroup gg{};
    int wg = 0;
    for (int i = 0; i < n; ++i) {
      if (p[i].aload != kd[0] || p[i].bload != kd[1]) continue;
      const GemmArgs& g = args[i];
      wg += (int)(cdiv(g.M, 64) * cdiv(g.N, 64)) * g.ksplit;
      gg.g[gg.n] = g;
      gg.end[gg.n] = wg;
      ++gg.n;
    }
    if (gg.n && gemm_group_launch(gg, kd[0], kd[1], st)) return -1;
  }
  return reduce_group_launch(rg, st);
}

int linear_fwd(LinearFwd& f, hipStream_t st) {
  const int64_t ldx = f.ldx ? f.ldx : f.K;
  const bool lora = f.A != nullptr && f.r > 0;
  if (lora) {
    if (skinny_U(f.x, ldx, f.T, f.K, f.A, f.nmod * f.r, f.u, f.nmod * f.r, f.ws, st)) return -1;
  }
  GemmArgs g{};
  g.M = f.T; g.N = f.N; g.K = f.K;
  g.A = f.x; g.lda = ldx;
  g.Bq = f.codes; g.Bs = f.absmax; g.ldq = f.K;
  g.alpha = 1.f;
  g.C = f.y; g.ldc = f.ldy ? f.ldy : f.N;
  g.R = f.res; g.ldr = f.ldres ? f.ldres : f.N;
  if (lora) {
    g.lora = LORA_FWD;
    g.A2 = f.u; g.lda2 = f.nmod * f.r;
    g.K2 = f.r;
    g.nmod = f.nmod;
    for (int i = 0; i < f.nmod; ++i) { g.mod_end[i] = f.mod_end[i]; g.modB[i] = f.Bm[i]; }
    g.s2 = f.s;
  }
  g.ev0 = f.ev0;
  g.ev1 = f.ev1;
  // Split-K needs the workspace for its partials; without one the GEMM runs unsplit.
  const GemmPlan pl = plan_nf4(f.T, f.N, f.K, f.ws != nullptr);
  g.partial = f.ws;
  int rc;
  g.ksplit = pl.ksplit;
  if (pl.big && gemm_big_ok(g, B_NF4_NT, EPI_BF16)) {
    f.tile = 256;
    rc = gemm_big_launch(g, B_NF4_NT, EPI_BF16, st);
  } else {
    f.tile = 128;
    g.ksplit = f.ws ? big_split(f.T, f.N, f.K) : 1;
    rc = gemm_launch(g, A_ROW, B_NF4_NT, EPI_BF16, 128, st);
  }
  f.ksplit = g.ksplit;
  if (!rc && f.ev2 && g.ksplit > 1) (void)hipEventRecord(f.ev2, st);
  return rc;
}

int linear_dx(LinearDx& d, hipStream_t st) {
  GemmArgs g{};
  g.M = d.T; g.N = d.Nout; g.K = d.Kc;
  g.A = d.dy; g.lda = d.lddy;
  g.Bq = d.codes; g.Bs = d.absmax; g.ldq = d.ldq;
  g.alpha = 1.f;
  g.C = d.out; g.ldc = d.ldo;
  if (d.du && d.rc > 0) {
    g.lora = LORA_DX;
    g.A2 = d.du; g.lda2 = d.lddu;
    g.B2 = d.Acat; g.ldb2 = d.Nout;
    g.K2 = d.rc;
  }
  g.gu = d.gu; g.ldgu = d.ldgu; g.I = d.I;
  g.ev0 = d.ev0;
  g.ev1 = d.ev1;
  const GemmPlan pl = plan_nf4(d.T, d.Nout, d.Kc, d.ws != nullptr);
  g.partial = d.ws;
  int rc;
  g.ksplit = pl.ksplit;
  if (pl.big && gemm_big_ok(g, B_NF4_NN, d.epi)) {
    d.tile = 256;
    rc = gemm_big_launch(g, B_NF4_NN, d.epi, st);
  } else {
    d.tile = 128;
    g.ksplit = d.ws ? big_split(d.T, d.Nout, d.Kc) : 1;
    rc = gemm_launch(g, A_ROW, B_NF4_NN, d.epi, 128, st);
  }
  d.ksplit = g.ksplit;
  if (!rc && d.ev2 && g.ksplit > 1) (void)hipEventRecord(d.ev2, st);
  return rc;
}
