// Kernel argument structs and host-side launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace poetx {

// ---- Cayley builder (build.hip)
struct GJSeg {
  const float* theta;   // theta mode: [blk][b(b-1)/2]; nullptr selects matrix mode
  float* q32;           // optional Q = 2M - I outputs, [blk][B][B]
  uint16_t* qbf;
  uint16_t* qtbf;
};
constexpr int GJ_MAXSEG = 64;
struct GJArgs {
  GJSeg seg[GJ_MAXSEG]; // workgroup w uses the segment s with start[s] <= w < start[s+1]
  int start[GJ_MAXSEG + 1];
  int nseg;
  const float* in;      // matrix mode input (one segment)
  int64_t in_stride;
  int in_ld;
  float* out;           // optional M output (strided)
  int64_t out_stride;
  int out_ld;
  const int* skip;      // optional: workgroup w does nothing when skip[w] != 0
};
// mode 0: fp32 MFMA trailing updates; mode 6: split bf16 x6 (fp32-level accuracy)
void launch_gj(int B, int mode, int nblk, const GJArgs& g, hipStream_t s);

struct BGemmArgs {
  int M, N, K;
  const float* A; int64_t sA; int lda; int transA; int addIA;
  const float* B; int64_t sB; int ldb; int transB; int addIB;
  float* C; int64_t sC; int ldc;
  float alpha, beta;
  // optional second segment: batch items z >= nb0 use A1 / B1 / C1 (when set)
  // at index z - nb0 instead of A / B / C at index z, with the leading
  // dimensions and batch strides lda1 .. sC1 where those are nonzero
  const float* A1; const float* B1; float* C1; int nb0;
  int lda1, ldb1, ldc1; int64_t sA1, sB1, sC1;
  // optional: batch item z is computed only when run[z] != 0
  const int* run;
};
// mode 0: fp32 MFMA; 3 / 6: split bf16 x3 / x6
void launch_bgemm(int mode, int batch, const BGemmArgs& a, hipStream_t s);
void launch_unpack_eye_minus_s(const float* theta, int b, int nblk, float* A, hipStream_t s);
void launch_finalize_q(const float* M, int b, int nblk, float* q32, uint16_t* qbf, uint16_t* qtbf, hipStream_t s);
// truncated Neumann (CNP) builder pieces (cnp.hip)
void launch_cnp_unpack_s(const float* theta, int b, int nblk, float* S, hipStream_t s);
void launch_cnp_guard(const float* S, int b, int nblk, int terms, float tol, int* use, hipStream_t s);
void launch_cnp_finalize(const float* T, const int* use, int b, int nblk, float* q32, uint16_t* qbf, uint16_t* qtbf,
                         hipStream_t s);
// chain rule over blocks from up to CH_MAXSEG sources: block z of a launch
// belongs to the segment s with start[s] <= z < start[s+1] and is block
// z - start[s] of that segment's arrays (q: fp32 Q, g: dL/dQ, dth: output).
constexpr int CH_MAXSEG = 64;
struct ChainSeg {
  const float* q;
  const float* g;
  float* dth;
};
struct ChainSegs {
  ChainSeg seg[CH_MAXSEG];
  int start[CH_MAXSEG + 1];
  int nseg;
};
// fp32-accurate chain-rule products on split bf16 operands (chain.hip):
// C1[z] = (I + Q) G^T / 2 and GS[z] = (I + Q^T) C1[z]^T; C1 and GS are
// contiguous [nblk][b][b] fp32 and GS may alias the segments' g arrays when
// those are contiguous in block order (G is dead once C1 is formed).
void launch_chain_products(const ChainSegs& cs, int nblk, int b, float* C1, float* GS, hipStream_t s);
// dth of block z = (GS[z] - GS[z]^T) on the strict upper triangle (GS contiguous)
void launch_skew_project(const float* GS, int b, int nblk, const ChainSegs& cs, int accumulate, hipStream_t s);
// ---- block transforms (transform.hip)
// bf16 row permutations of a token-major [N][W] matrix:
//   gather : out[t][j] = in[t][perm[j]]; if tail_out, also tail_out[t][j] for j >= tail0
//   scatter: out[t][perm[j]] = src[t][j], src = in (j < tail0) or tail_in (j >= tail0; NULL = in)
struct PermArgs {
  const uint16_t* in;
  const uint16_t* tail_in;
  uint16_t* out;
  uint16_t* tail_out;
  const int32_t* perm;
  int64_t N;
  int W, tail0;
};
void launch_permute_bf16(bool gather, const PermArgs& a, hipStream_t s);
// fp32 transforms, permutation and block product in one pass:
// gather-in : out[t][l*B+i] = sum_kk in[t][perm[l*B+kk]] * Mq(kk, i); tail copies in[t][perm[j]]
// scatter-out: out[t][perm[l*B+i]] = sum_kk in[t][l*B+kk] * Mq(kk, i); tail copies in[t][j]
// with Mq(kk, i) = q[l][i][kk] (trans=0) / q[l][kk][i] (trans=1)
struct XformArgs {
  const void* in;
  void* out;
  void* emit;           // gather-in only: gathered copy of in (nullable)
  const int32_t* perm;
  const void* bq;
  int64_t N;
  int W, B, k;
  int trans;
};
void launch_gather_in_f32(const XformArgs& a, hipStream_t s);
void launch_scatter_out_f32(const XformArgs& a, hipStream_t s);

// ---- block-diagonal products (blockdiag.hip)
// out[t][l*b + i] = sum_kk in[t][l*b + kk] * q[l][i][kk] for l < k, t < N (bf16,
// fp32 accumulation; row strides lda, ldc; columns from k*b on untouched).
// Returns false, launching nothing, where the streaming kernel does not apply
// (b not in {32, 64, 128, 256}, rows or pointers not 16-byte aligned, or
// offsets beyond 32 bits); the caller then uses the batched GEMM.
bool launch_blockdiag_bf16(const uint16_t* in, const uint16_t* q, uint16_t* out, int64_t N, int64_t lda,
                           int64_t ldc, int b, int k, hipStream_t s);

// gather and block product in one pass (blockdiag.hip):
//   out[t][l*b + i] = sum_kk q[l][i][kk] in[t][perm[l*b + kk]], l < k, W = k b
//   emit (nullable) [t][l*b + kk] = in[t][perm[l*b + kk]]
// false (nothing launched) where it does not apply (b != 256, W > 2048, ...)
struct GatherBdArgs {
  const uint16_t* in;
  const int32_t* perm;
  const uint16_t* q;
  uint16_t* out;
  uint16_t* emit;
  int64_t N;
  int W, k, runs, tpr;
  int64_t lda, ldc, lde;
};
bool gather_blockdiag_applies(const void* in, const int32_t* perm, const void* q, const void* out, const void* emit,
                              int64_t N, int W, int b, int k, int64_t lda, int64_t ldc, int64_t lde);
bool launch_gather_blockdiag_bf16(const uint16_t* in, const int32_t* perm, const uint16_t* q, uint16_t* out,
                                  uint16_t* emit, int64_t N, int W, int b, int k, int64_t lda, int64_t ldc,
                                  int64_t lde, hipStream_t s);

// ---- dense GEMMs (gemm.hip): C[M][N] = A[M][K] * op(B)
// nt: B is [N][K] (C = A B^T); nn: B is [K][N] (C = A B)
// Batched bf16 GEMM with strides (elements): for z < batch,
//   NT: C_z[M][N] = A_z[M][K] * B_z[N][K]^T,  NN: C_z[M][N] = A_z[M][K] * B_z[K][N]
// with X_z = X + z * sX and row strides lda, ldb, ldc.
struct GemmArgs {
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* C;

  int M, N, K;
  int64_t lda, ldb, ldc;
  int64_t sA, sB, sC;
  int batch;
  // INT8 weight operand (launch_gemm_q8): codes in place of B, one fp32
  // scale per weight row
  const int8_t* Bq;
  const float* Bs;
  // R-side blocks (launch_gemm_rside): bf16 [N / qb][qb][qb]
  const uint16_t* Qr;
  int qb;
};
void launch_gemm_bf16(bool nn, const GemmArgs& g, hipStream_t s);
// C = Z with every b-column block l of Z = A op(W) (W^T for NT, W for NN)
// multiplied by block l of Q (C[:, L] = bf16(Z[:, L]) Q_l^T): the forward
// GEMM and the R-side block product in one launch.  Bit-identical to
// launch_gemm_bf16 followed by the block product.  Takes b in {64, 128,
// 256}, K a multiple of 64 of at least 2048, N a multiple of 256 and 16-byte
// aligned operands (gemm_rside_applies).
bool gemm_rside_applies(bool nn, const void* A, const void* W, const void* Q, const void* C, int64_t M, int64_t N,
                        int64_t K, int b);
void launch_gemm_rside(bool nn, const uint16_t* A, const uint16_t* W, const uint16_t* Q, uint16_t* C, int64_t M,
                       int64_t N, int64_t K, int b, hipStream_t s);
// out [n][m] = in [m][n]^T, bf16 (the transposed weight copy)
void launch_transpose_bf16(const uint16_t* in, uint16_t* out, int64_t m, int64_t n, hipStream_t s);
// out [n][m] = the dequantized INT8 weight [m][n], transposed
void launch_dequant_transpose(const int8_t* q, const float* sc, uint16_t* out, int64_t m, int64_t n, hipStream_t s);
// C = A op(W) with W = bf16(s_i q_ij) formed inside the GEMM from INT8 codes
// q [rows][cols] and scales s [rows] (NT: W [N][K], rows = N; NN: W [K][N],
// rows = K).  Returns false (nothing launched) where the tiled kernel does not
// apply: K % 16 (NT) or N % 16 (NN), K or N not a multiple of 8, or
// misaligned operands.
bool launch_gemm_q8(bool nn, const uint16_t* A, const int8_t* codes, const float* scales, uint16_t* C, int64_t M,
                    int64_t N, int64_t K, hipStream_t s);
void launch_gemm_bf16(bool nn, const uint16_t* A, const uint16_t* Bm, uint16_t* C, int64_t M, int64_t N,
                      int64_t K, hipStream_t s);
void launch_gemm_f32(bool nn, const float* A, const float* Bm, float* C, int64_t M, int64_t N, int64_t K,
                     hipStream_t s);

// ---- block Gram reduction (gram.hip): G[l][i][j] = sum_t A[t][l*B+i] * C[t][l*B+j]
size_t gram_partials_bytes(int64_t N, int B, int k, bool f32);
void launch_gram(bool f32, const void* A, const void* C, int64_t N, int W, int B, int k, float* G, void* partials,
                 hipStream_t s);

// ---- merge (merge.hip)
// V = D_R W D_P on b x b tiles of the working-layout weight W [m][n]:
//   bf16: qr = Q_R bf16 row-major [kR][b][b], qpt = Q_P^T bf16 [kP][b][b]
//   f32 : qr = Q_R fp32, qpt = Q_P fp32 (row-major, not transposed)
void launch_merge_tiles(bool f32, const void* W, void* V, const void* qr, const void* qpt, int64_t m, int64_t n, int b,
                        int kR, int kP, hipStream_t s);
void launch_perm_keys_rank(uint64_t seed, uint64_t merge_index, int side, int64_t n, uint64_t* keys, int32_t* out,
                           hipStream_t s);
void launch_invert_perm(const int32_t* p, int64_t n, int32_t* inv, hipStream_t s);
void launch_relayout(bool f32, const void* V, void* W, const int32_t* sinv_old, const int32_t* snew,
                     const int32_t* tinv_old, const int32_t* tnew, int64_t m, int64_t n, hipStream_t s);
void launch_copy_i32(const int32_t* src, int32_t* dst, int64_t n, hipStream_t s);
// The permutation step of a merge, both sides: snew / tnew <- new draws,
// sinv / tinv <- inverses of the old sigma / tau, sigma / tau <- the new draws,
// and snew / tnew <- sinv(snew), tinv(tnew) (the relayout's source maps).
void launch_merge_permutations(uint64_t seed, uint64_t merge_index, int32_t* sigma, int32_t* tau, int64_t m, int64_t n,
                               int32_t* snew, int32_t* tnew, int32_t* sinv, int32_t* tinv, hipStream_t s);
// rows [0, rows) of a bf16 [.][n] matrix, n a multiple of 8, 16-byte aligned
void launch_copy_rows_bf16(const uint16_t* src, uint16_t* dst, int64_t rows, int64_t n, hipStream_t s);
// W[i][j] = V[rmap[i]][cmap[j]] (bf16; V and W distinct).  Returns false,
// launching nothing, unless n is a multiple of 8 up to 32768 and V, W, cmap are
// 16-byte aligned.
bool launch_relayout_rows_bf16(const uint16_t* V, uint16_t* W, const int32_t* rmap, const int32_t* cmap, int64_t m,
                               int64_t n, hipStream_t s);
void launch_fill_f32(float* p, float v, int64_t n, hipStream_t s);
void launch_fill2_f32(float* p0, int64_t n0, float* p1, int64_t n1, float v, hipStream_t s);
// In-place merge products: W <- W D_P (full column groups), then W <- D_R W
// (full row groups); bf16 through MFMA, fp32 with FMA sums.
void launch_merge_products_inplace(bool f32, void* W, const void* qr, const void* qpt, int64_t m, int64_t n, int b,
                                   int kR, int kP, hipStream_t s);
// In-place relayout W[i][j] <- W[rho(i)][kappa(j)] along the cycles of rho
// (m <= 32768), cut into segments of at most L <= 64 rows; saved receives up
// to max_saved rows (max_saved >= 2 ceil(m / L) suffices); dist, hlist,
// slot, nxt ([m] each), slist ([max_saved]) and counts ([2]) are scratch.
void launch_relayout_inplace(bool f32, void* W, void* saved, const int32_t* rho, const int32_t* kappa, int64_t m,
                             int64_t n, int L, int32_t* dist, int32_t* hlist, int32_t* slot, int32_t* slist,
                             int32_t* counts, int32_t* nxt, int64_t max_saved, hipStream_t s);
// The permutation step and the in-place relayout of several merges in one
// launch per stage.  One item per matrix, its buffers disjoint from the other
// items': W (bf16 [m][n]), saved (rows set aside), the current permutations
// sigma / tau, the merge scratch (snew, tnew, sinv, tinv, dist, hlist, slot,
// nxt: [m] or [n]; slist [max_saved]; counts [2]) and the generators thR / thP
// (nthR, nthP entries), zeroed by launch_zero_generators_batch.
struct MergeItem {
  void* W;
  void* saved;
  int32_t *sigma, *tau, *snew, *tnew, *sinv, *tinv;
  int32_t *dist, *hlist, *slot, *slist, *counts, *nxt;
  float *thR, *thP;
  int64_t nthR, nthP, m, n, max_saved;
  uint64_t seed, merge_index;
};
constexpr int MERGE_BATCH = 16;   // items per launch (the batch travels as a kernel argument)
struct MergeBatch {
  MergeItem it[MERGE_BATCH];
  int count;
  int start[MERGE_BATCH + 1];     // first workgroup of each item (set by the launchers)
};
// launch_merge_permutations for every item
void launch_merge_permutations_batch(const MergeBatch& b, hipStream_t s);
// the relayout plans (cycle heads and segments) of every item, rho = snew
void launch_cycle_plans_batch(const MergeBatch& b, int L, hipStream_t s);
// head rows set aside and the segment walks of every item (bf16 W with rows
// of a multiple of 8 columns, W, saved and tnew 16-byte aligned:
// walk_staged_ok), kappa = tnew
void launch_relayout_staged_batch(const MergeBatch& b, int L, hipStream_t s);
bool walk_staged_ok(int64_t n, int L, const void* W, const void* saved, const int32_t* kappa);
// thR, thP <- 0 for every item
void launch_zero_generators_batch(const MergeBatch& b, hipStream_t s);
// INT8 weight codes with per-row fp32 scales (quant.hip)
void launch_dequant_rows(const int8_t* q, const float* sc, uint16_t* w, int64_t m, int64_t n, hipStream_t s);
void launch_quantize_rows(const uint16_t* w, int8_t* q, float* sc, int64_t m, int64_t n, hipStream_t s);
void launch_adam(float* theta, const float* grad, float* m, float* v, int64_t n, float lr, float b1, float b2,
                 float eps, float bc1, float bc2, hipStream_t s);

}  // namespace poetx
