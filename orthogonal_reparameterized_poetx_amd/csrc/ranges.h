// Buffer-resource ranges of the streaming kernels, shared by the kernels and
// by a host-side check.  Each range starts at the first element a
// workgroup's tile may read and ends at its last: a tile of `rows` rows of
// `width` elements from (r0, c0) of a row-major operand with leading
// dimension ld covers ((rows - 1) ld + width) elements.  Loads whose offset
// falls past the range read zero, so with exact ranges no load can touch
// memory past the operand, whatever the lane arithmetic does.  Plain C++
// (no HIP types), so that the check compiles with a host compiler.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define POETX_HD __host__ __device__
#else
#define POETX_HD
#endif

namespace poetx {

struct BufRange {
  int64_t first;   // first element, counted from the operand's base
  int64_t bytes;   // byte extent (the descriptor's record count)
};

// rows [r0, r0 + rows) and columns [c0, c0 + width) of a row-major operand
POETX_HD inline BufRange tile_range(int64_t r0, int64_t rows, int64_t c0, int64_t width, int64_t ld, int es) {
  return BufRange{r0 * ld + c0, rows > 0 ? ((rows - 1) * ld + width) * es : 0};
}

// GEMM (256 x 256 output tiles, bf16): the A tile [min(M - m0, 256) rows][K];
// the NT B tile [min(N - n0, 256) rows][K]; the NN B tile, all K rows from
// column n0 to the last column N - 1
constexpr int GEMM_TILE = 256;
// shapes the tiled GEMM kernels take (whole 16-byte chunks along K and N);
// others go to a generic kernel without buffer resources
POETX_HD inline bool gemm_tiled_shape(int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t sA, int64_t sB) {
  return K > 0 && K % 8 == 0 && N % 8 == 0 && lda % 8 == 0 && ldb % 8 == 0 && sA % 8 == 0 && sB % 8 == 0;
}
POETX_HD inline BufRange gemm_range_a(int64_t m0, int64_t M, int64_t K, int64_t lda) {
  return tile_range(m0, (M - m0 < GEMM_TILE ? M - m0 : GEMM_TILE), 0, K, lda, 2);
}
POETX_HD inline BufRange gemm_range_b_nt(int64_t n0, int64_t N, int64_t K, int64_t ldb) {
  return tile_range(n0, (N - n0 < GEMM_TILE ? N - n0 : GEMM_TILE), 0, K, ldb, 2);
}
POETX_HD inline BufRange gemm_range_b_nn(int64_t n0, int64_t N, int64_t K, int64_t ldb) {
  return tile_range(0, K, n0, N - n0, ldb, 2);
}

// the R-side blocks multiplying output column tile bn of the fused forward
// GEMM: the 256 / b blocks of b x b from block 256 bn / b on, which form
// rows [256 bn, 256 bn + 256) of the blocks viewed as a [N][b] matrix
POETX_HD inline BufRange gemm_range_q(int64_t bn, int64_t b) { return tile_range(bn * GEMM_TILE, GEMM_TILE, 0, b, b, 2); }

// the same tiles of an INT8 weight (one byte per code)
POETX_HD inline BufRange gemm_range_bq_nt(int64_t n0, int64_t N, int64_t K, int64_t ldb) {
  return tile_range(n0, (N - n0 < GEMM_TILE ? N - n0 : GEMM_TILE), 0, K, ldb, 1);
}
POETX_HD inline BufRange gemm_range_bq_nn(int64_t n0, int64_t N, int64_t K, int64_t ldb) {
  return tile_range(0, K, n0, N - n0, ldb, 1);
}

// Gram product of token runs (tiles of 32 tokens): runs and tiles per run
constexpr int GRAM_T = 32, GRAM_TI = 128, GRAM_STAGES = 7;
struct GramRuns { int runs; int tpc; };
POETX_HD inline GramRuns gram_stream_runs(int64_t N, int B, int k) {
  const int q = (B / GRAM_TI) * (B / GRAM_TI);
  const int64_t ntiles = (N + GRAM_T - 1) / GRAM_T;
  int64_t r = 256 / ((int64_t)k * q);
  if (r < 1) r = 1;
  if (r > ntiles) r = ntiles;
  const int64_t tpc = (ntiles + r - 1) / r;
  r = (ntiles + tpc - 1) / tpc;
  return GramRuns{(int)r, (int)tpc};
}

// Block product over token runs (tiles of 32 tokens, a ring of 7 stages):
// workgroups per block and tiles per run.  Runs are cut so that every
// per-lane offset, including the ring's loads of up to 6 tiles past a run's
// end (which read zero), stays below 2^31.  runs == 0: no such cut exists.
// (Nine stages, the most the LDS holds at b = 256, measured no faster.)
constexpr int BDIAG_T = 32, BDIAG_STAGES = 7, BDIAG_PP_STAGES = 7;
// ring loads reach this many tiles past a run (the deeper ring of the two)
constexpr int BDIAG_REACH = BDIAG_STAGES > BDIAG_PP_STAGES ? BDIAG_STAGES : BDIAG_PP_STAGES;
struct BdiagRuns { int64_t runs; int64_t tpc; };
POETX_HD inline BdiagRuns blockdiag_runs(int64_t N, int64_t lda, int64_t ldc, int b, int k) {
  const int lds = (BDIAG_STAGES + 1) * BDIAG_T * b * 2;
  const int occ_lds = (160 * 1024) / lds, occ_w = 16 / (b / 32 > 0 ? b / 32 : 1);
  const int occ = occ_lds < occ_w ? occ_lds : occ_w;
  const int64_t ntiles = (N + BDIAG_T - 1) / BDIAG_T;
  int64_t runs = (256LL * occ) / k;
  if (runs < 1) runs = 1;
  if (runs > ntiles) runs = ntiles;
  int64_t tpc = (ntiles + runs - 1) / runs;
  const int64_t ld = lda > ldc ? lda : ldc;
  const int64_t maxt = (0x7fffffffLL / (BDIAG_T * ld * 2)) - BDIAG_REACH;
  if (maxt < 1) return BdiagRuns{0, 0};
  if (tpc > maxt) tpc = maxt;
  runs = (ntiles + tpc - 1) / tpc;
  return BdiagRuns{runs, tpc};
}

}  // namespace poetx
