// Launch interface of the bf16 / NF4 MFMA GEMM family.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// How operand A (M x K) is stored.
enum ALoad { A_ROW = 0,    // A[m * lda + k]
             A_COL = 1 };  // A[k * lda + m]
// How operand B (contraction k, output column n) is stored.
enum BLoad { B_BF16_NT = 0,  // bf16 B[n * ldb + k]
             B_BF16_NN = 1,  // bf16 B[k * ldb + n]
             B_NF4_NT = 2,   // NF4 W, flat element n * ldq + k
             B_NF4_NN = 3 }; // NF4 W, flat element k * ldq + n
enum Epi {
  EPI_BF16 = 0,       // C bf16 = alpha*acc (+ s2*acc2 LoRA) (+ R residual)
  EPI_F32 = 1,        // C f32 = alpha*acc
  EPI_F32_ACC = 2,    // C f32 += alpha*acc
  EPI_PARTIAL = 3,    // split-K partial sums (reduced by gemm_reduce)
  EPI_SWIGLU_BWD = 4, // acc = dL/da; writes bf16 dg (col n) and du (col I + n)
  EPI_CE_STATS = 5,   // per-row (max, sum exp) over the tile's columns + target logit
  EPI_CE_GRAD = 6     // C bf16 = w_m (exp(acc - lse_m) - [n == tgt_m])
};
enum LoraMode { LORA_NONE = 0, LORA_FWD = 1, LORA_DX = 2 };

struct GemmArgs {
  int M, N, K;
  const uint16_t* A; int64_t lda;
  const uint16_t* Bh; int64_t ldb;
  const uint8_t* Bq; const float* Bs; int64_t ldq;
  // LoRA second contraction
  int lora;
  const uint16_t* A2; int64_t lda2;  // U_cat [M, nmod*r] (FWD) or du_cat [M, K2] (DX)
  const uint16_t* B2; int64_t ldb2;  // A_cat [K2, N] row-major (DX)
  int K2;                            // r (FWD) or total contraction (DX)
  int nmod;                          // FWD: modules along N
  int mod_end[4];                    // FWD: cumulative column end of each module
  const uint16_t* modB[4];           // FWD: B_g [N_g, r] row-major
  float s2;                          // FWD: LoRA scale
  // epilogue
  float alpha;
  void* C; int64_t ldc;
  const uint16_t* R; int64_t ldr;
  const uint16_t* gu; int64_t ldgu; int I;
  const int32_t* tgt; const float* lse; const float* roww;
  float* stats; int stats_ld; float* tgt_logit; int col0;
  int ksplit; float* partial;
  hipEvent_t ev0, ev1;   // optional: recorded around the GEMM kernel itself (not the split-K reduce)
};

// Returns 0, or -1 when the (tile, loaders, epilogue) combination is not built.
int gemm_launch(const GemmArgs& g, int aload, int bload, int epi, int tile, hipStream_t st);
// Large GEMMs (256 x 256 tiles, 512 threads): B_NF4_NT with EPI_BF16
// (LORA_FWD allowed), B_NF4_NN with EPI_F32 / EPI_BF16 (no residual) /
// EPI_SWIGLU_BWD (LORA_DX allowed), B_BF16_NT with EPI_CE_STATS /
// EPI_CE_GRAD (statistics per 128-column half, no split), and B_BF16_NN with
// EPI_F32 / EPI_F32_ACC (N % 256 == 0, no LoRA); split-K (ksplit > 1) writes
// float partials to g.partial (ksplit * M * N floats) and then runs
// gemm_reduce_epi.  gemm_big_ok checks the shape and alignment conditions;
// gemm_big_launch returns -1 when they do not hold.
bool gemm_big_ok(const GemmArgs& g, int bload, int epi);
int gemm_big_launch(const GemmArgs& g, int bload, int epi, hipStream_t st);
// out = epilogue(sum_z partial[z]) for split-K: mode 0 -> bf16 alpha*sum, 1 -> f32 alpha*sum.
void gemm_reduce(const float* partial, int ksplit, int M, int N, float alpha, int mode,
                 void* C, int64_t ldc, hipStream_t st);
// gemm_reduce with mode 1 (float), row block i (rows i*rows .. +rows-1 of the
// M x N sum) written to C[i] (ldc); M / rows <= 4 blocks, else -1.
int gemm_reduce_rows(const float* partial, int ksplit, int M, int N, float alpha, float* const* C, int rows,
                     int64_t ldc, hipStream_t st);
int64_t gemm_partial_elems(int M, int N, int ksplit);
// Sums the ksplit partials of g (in split order) and applies epilogue epi to g.C
// (N % 4 == 0).
void gemm_reduce_epi(const GemmArgs& g, int epi, hipStream_t st);

// Grouped skinny products: up to kMaxGroup products of one loader combination
// in one launch, each writing split-K float partials (g[i].partial, its
// g[i].ksplit slices); end[i] = cumulative workgroup count (tiles x slices of
// 64 x 64) through product i.
constexpr int kMaxGroup = 6;
struct GemmGroup { GemmArgs g[kMaxGroup]; int end[kMaxGroup]; int n; };
int gemm_group_launch(const GemmGroup& gg, int aload, int bload, hipStream_t st);
// The sums of those partials in split order, one job per product: alpha * sum
// to C (mode 0 bf16, 1 float) or, with rows > 0, row block m / rows to Cr[m /
// rows] (float); end[i] = cumulative M * N through job i.
struct ReduceJob {
  const float* P; int ks, M, N; float alpha; int mode;
  void* C; int64_t ldc; int rows; float* Cr[4];
};
struct ReduceGroup { ReduceJob j[kMaxGroup]; int64_t end[kMaxGroup]; int n; };
int reduce_group_launch(const ReduceGroup& rg, hipStream_t st);
