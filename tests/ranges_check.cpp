// Host-side check of the buffer ranges the GEMM, block-product and Gram
// kernels build (ranges.h, the same functions the kernels call), for the
// launches listed on stdin, one per line:
//   gemm nt|nn M N K lda ldb       every 256 x 256 output tile
//   bdiag N lda ldc b k            every (token run, block) workgroup
//   gram N W B k                   every (block, quadrant, token run) workgroup
// A range must start inside its operand, end at or before the operand's last
// element, and fit the 32-bit record count; the block product's per-lane
// offsets, including the ring's loads past a run, must stay below 2^31.
// Prints "ok <launches> <ranges>" or the first failure.
#include <cstdio>
#include <cstring>
#include <string>

#include "../orthogonal_reparameterized_poetx_amd/csrc/ranges.h"

using namespace poetx;

static long long checked = 0;

static bool within(const BufRange& r, long long extent_elems, const char* what, const char* line) {
  ++checked;
  const long long end = r.first + r.bytes / 2;   // bf16 operands
  if (r.first < 0 || r.bytes < 0 || end > extent_elems || r.bytes > 0xffffffffLL || (r.bytes & 1)) {
    std::printf("FAIL %s: first %lld bytes %lld extent %lld | %s\n", what, (long long)r.first, (long long)r.bytes,
                extent_elems, line);
    return false;
  }
  return true;
}

int main() {
  char buf[512];
  long long launches = 0;
  while (std::fgets(buf, sizeof buf, stdin)) {
    char kind[16] = {0}, op[8] = {0};
    long long a[6] = {0};
    if (std::sscanf(buf, "%15s", kind) != 1) continue;
    buf[std::strcspn(buf, "\n")] = 0;
    ++launches;
    if (!std::strcmp(kind, "gemm")) {
      if (std::sscanf(buf, "%*s %7s %lld %lld %lld %lld %lld", op, &a[0], &a[1], &a[2], &a[3], &a[4]) != 6) return 2;
      const long long M = a[0], N = a[1], K = a[2], lda = a[3], ldb = a[4];
      const bool nn = !std::strcmp(op, "nn");
      const long long extA = (M - 1) * lda + K;
      const long long extB = nn ? (K - 1) * ldb + N : (N - 1) * ldb + K;
      // batch strides: a multiple of 8 in every launch of the library
      if (!gemm_tiled_shape(N, K, lda, ldb, 8, 8)) continue;   // the generic kernel, no buffer resources
      for (long long m0 = 0; m0 < M; m0 += GEMM_TILE)
        if (!within(gemm_range_a(m0, M, K, lda), extA, "gemm A", buf)) return 1;
      for (long long n0 = 0; n0 < N; n0 += GEMM_TILE)
        if (!within(nn ? gemm_range_b_nn(n0, N, K, ldb) : gemm_range_b_nt(n0, N, K, ldb), extB, "gemm B", buf))
          return 1;
      // the fused forward (NT, N a multiple of 256): the blocks of column
      // tile n0 / 256 among the R-side blocks [N / b][b][b]
      if (!nn && N % GEMM_TILE == 0)
        for (long long b = 64; b <= GEMM_TILE; b *= 2)
          for (long long n0 = 0; n0 < N; n0 += GEMM_TILE)
            if (!within(gemm_range_q(n0 / GEMM_TILE, b), N * b, "gemm Q", buf)) return 1;
    } else if (!std::strcmp(kind, "bdiag")) {
      if (std::sscanf(buf, "%*s %lld %lld %lld %lld %lld", &a[0], &a[1], &a[2], &a[3], &a[4]) != 5) return 2;
      const long long N = a[0], lda = a[1], ldc = a[2];
      const int b = (int)a[3], k = (int)a[4];
      const BdiagRuns br = blockdiag_runs(N, lda, ldc, b, k);
      if (br.runs < 1) continue;   // the launcher takes the GEMM path instead
      const long long ld = lda > ldc ? lda : ldc;
      if ((br.tpc + BDIAG_REACH) * BDIAG_T * ld * 2 >= 0x7fffffffLL) {
        std::printf("FAIL bdiag 32-bit offsets | %s\n", buf);
        return 1;
      }
      for (long long run = 0; run < br.runs; ++run) {
        const long long t0 = run * br.tpc * BDIAG_T;
        if (t0 >= N) break;
        const long long rows = (br.tpc * BDIAG_T < N - t0) ? br.tpc * BDIAG_T : N - t0;
        for (int l = 0; l < k; ++l) {
          if (!within(tile_range(t0, rows, (long long)l * b, b, lda, 2), (N - 1) * lda + (long long)k * b, "bdiag in",
                      buf) ||
              !within(tile_range(t0, rows, (long long)l * b, b, ldc, 2), (N - 1) * ldc + (long long)k * b, "bdiag out",
                      buf))
            return 1;
        }
      }
    } else if (!std::strcmp(kind, "gram")) {
      if (std::sscanf(buf, "%*s %lld %lld %lld %lld", &a[0], &a[1], &a[2], &a[3]) != 4) return 2;
      const long long N = a[0], W = a[1];
      const int B = (int)a[2], k = (int)a[3];
      const long long ntiles = (N + GRAM_T - 1) / GRAM_T;
      if ((ntiles + GRAM_STAGES) * GRAM_T * W * 2 >= 0x7fffffffLL) continue;   // the launcher falls back
      const GramRuns gr = gram_stream_runs(N, B, k);
      for (int l = 0; l < k; ++l)
        for (int run = 0; run < gr.runs; ++run) {
          const long long t0 = (long long)run * gr.tpc * GRAM_T;
          if (t0 >= N) continue;
          const long long rows = ((long long)gr.tpc * GRAM_T < N - t0) ? (long long)gr.tpc * GRAM_T : N - t0;
          for (int ti = 0; ti < B / GRAM_TI; ++ti)
            if (!within(tile_range(t0, rows, (long long)l * B + ti * GRAM_TI, GRAM_TI, W, 2), (N - 1) * W + (long long)k * B,
                        "gram", buf))
              return 1;
        }
    } else {
      std::printf("FAIL unknown launch | %s\n", buf);
      return 2;
    }
  }
  std::printf("ok %lld %lld\n", launches, checked);
  return 0;
}
