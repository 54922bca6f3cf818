// C ABI of the POET-X layer hot path: validation, workspace planning and the
// launch sequences of forward, backward, merge and the Cayley builder.
// See include/poetx.h for the contract of every entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/poetx.h"
#include "kernels.h"

using namespace poetx;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(POETX_EHIP, "%s: %s", what, hipGetErrorString(e));
  return POETX_OK;
}

// ---- optional per-launch timing (diagnostics)
struct TimingRec {
  const char* name;
  hipEvent_t a, b;
  double flops, bytes;
};
bool g_timing = false;
std::vector<TimingRec> g_recs;

void clear_timing() {
  for (auto& r : g_recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_recs.clear();
}

// Records an event pair around the launches issued during its lifetime.
struct Tm {
  bool on;
  size_t idx;
  hipStream_t s;
  Tm(hipStream_t st, const char* name, double flops, double bytes) : on(g_timing), idx(0), s(st) {
    if (!on) return;
    TimingRec r{name, nullptr, nullptr, flops, bytes};
    if (hipEventCreate(&r.a) != hipSuccess || hipEventCreate(&r.b) != hipSuccess) { on = false; return; }
    (void)hipEventRecord(r.a, s);
    g_recs.push_back(r);
    idx = g_recs.size() - 1;
  }
  ~Tm() {
    if (on) (void)hipEventRecord(g_recs[idx].b, s);
  }
};

constexpr int64_t kMaxDim = 32768;
constexpr size_t kAlign = 256;
// tolerance of the truncated Cayley series: bound on the spectral norm of its
// dropped tail, two fp32 ulps of 1, so that even summed over a 256-wide block
// (sqrt(256) times) it stays below the 1e-5 fp32 tolerance of the outputs
constexpr float kCnpTol = 1.0f / (1 << 22);

bool valid_b(int32_t b) { return b == 32 || b == 64 || b == 128 || b == 256 || b == 512; }

int validate_layer(const poetx_layer* L) {
  if (!L) return fail(POETX_EINVAL, "layer is NULL");
  if (L->reserved != 0) return fail(POETX_EINVAL, "layer.reserved must be 0");
  if (L->dtype != POETX_F32 && L->dtype != POETX_BF16) return fail(POETX_EDTYPE, "unsupported dtype %d", L->dtype);
  if (!valid_b(L->b)) return fail(POETX_EINVAL, "block size b=%d not in {32,64,128,256,512}", L->b);
  if (L->m < 1 || L->m > kMaxDim || L->n < 1 || L->n > kMaxDim)
    return fail(POETX_ESHAPE, "m=%lld n=%lld out of range [1, %lld]", (long long)L->m, (long long)L->n,
                (long long)kMaxDim);
  if (L->flags & ~(POETX_ACCUMULATE_GRAD | POETX_W0_INT8 | POETX_SEPARATE_BLOCK_PRODUCTS | POETX_W0_TRANSPOSED |
                   POETX_X_PERMUTED))
    return fail(POETX_EINVAL, "unknown flags 0x%x", L->flags);
  if ((L->flags & POETX_X_PERMUTED) && L->dtype != POETX_BF16)
    return fail(POETX_EDTYPE, "POETX_X_PERMUTED applies to bf16 layers");
  if ((L->flags & POETX_W0_INT8) && L->dtype != POETX_BF16)
    return fail(POETX_EDTYPE, "POETX_W0_INT8 applies to bf16 layers");
  if ((L->flags & POETX_W0_TRANSPOSED) && L->dtype != POETX_BF16)
    return fail(POETX_EDTYPE, "POETX_W0_TRANSPOSED applies to bf16 layers");
  if ((L->flags & POETX_W0_TRANSPOSED) && (L->flags & POETX_W0_INT8))
    return fail(POETX_EINVAL, "POETX_W0_TRANSPOSED and POETX_W0_INT8 exclude each other");
  return POETX_OK;
}

int validate_N(int64_t N) {
  if (N < 0 || N >= (int64_t(1) << 31)) return fail(POETX_ESHAPE, "N=%lld out of range [0, 2^31)", (long long)N);
  return POETX_OK;
}

// bump allocator over the caller's workspace (base == nullptr: sizing only)
struct Arena {
  char* base;
  size_t off = 0;
  explicit Arena(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

size_t build_ws_bytes(int64_t nblk, int b) {
  if (b != 512 || nblk <= 0) return 0;
  Arena a(nullptr);
  a.take<float>((size_t)nblk * 512 * 512);  // I - S, then the Schur complement in place
  a.take<float>((size_t)nblk * 512 * 512);  // M = (I - S)^-1
  a.take<float>((size_t)nblk * 256 * 256);  // T = A11^-1 A12
  a.take<float>((size_t)nblk * 256 * 256);  // V = A21 A11^-1
  return a.off + kAlign;
}

// Output layouts wanted for one batch of Cayley blocks.
struct QOut {
  float* q32;
  uint16_t* qbf;
  uint16_t* qtbf;
};

int build_schur512(const float* const* theta, const int64_t* nblks, const QOut* outs, int nsets, void* ws, int mode,
                   hipStream_t s) {
  // 2x2 block inverse with 256-wide Schur complement:
  //   [A B; C D]^-1 = [Ai + Ai B Si C Ai, -Ai B Si; -Si C Ai, Si], Si = (D - C Ai B)^-1
  // over the blocks of every set at once (one pass of launches for all)
  int64_t nblk = 0;
  for (int i = 0; i < nsets; ++i) nblk += nblks[i];
  if (nblk <= 0) return POETX_OK;
  Arena a(ws);
  float* Af = a.take<float>((size_t)nblk * 512 * 512);
  float* Mf = a.take<float>((size_t)nblk * 512 * 512);
  float* Tm = a.take<float>((size_t)nblk * 256 * 256);
  float* Vm = a.take<float>((size_t)nblk * 256 * 256);
  const int64_t SB = 512 * 512, SH = 256 * 256;
  {
    int64_t off = 0;
    for (int i = 0; i < nsets; ++i) {
      if (nblks[i] <= 0) continue;
      launch_unpack_eye_minus_s(theta[i], 512, (int)nblks[i], Af + off * SB, s);
      off += nblks[i];
    }
  }
  auto gj = [&](float* in, float* out) {
    GJArgs g{};
    g.nseg = 1;
    g.start[0] = 0;
    g.start[1] = (int)nblk;
    g.in = in; g.in_stride = SB; g.in_ld = 512;
    g.out = out; g.out_stride = SB; g.out_ld = 512;
    launch_gj(256, mode, (int)nblk, g, s);
  };
  auto gemm = [&](const float* A, int lda, const float* B, int ldb, float* C, int ldc, float alpha, float beta,
                  int64_t sA, int64_t sB, int64_t sC) {
    BGemmArgs q{};
    q.M = q.N = q.K = 256;
    q.A = A; q.sA = sA; q.lda = lda;
    q.B = B; q.sB = sB; q.ldb = ldb;
    q.C = C; q.sC = sC; q.ldc = ldc;
    q.alpha = alpha; q.beta = beta;
    launch_bgemm(mode, (int)nblk, q, s);
  };
  float* A12 = Af + 256;
  float* A21 = Af + 256 * 512;
  float* A22 = Af + 256 * 512 + 256;
  float* M11 = Mf;
  float* M12 = Mf + 256;
  float* M21 = Mf + 256 * 512;
  float* M22 = Mf + 256 * 512 + 256;
  // two independent products with the same alpha and beta in one launch
  // (batch items nblk .. 2 nblk - 1 take the second)
  auto gemm_pair = [&](const float* A, int lda, int64_t sA, const float* B, int ldb, int64_t sB, float* C, int ldc,
                       int64_t sC, const float* A1, int lda1, int64_t sA1, const float* B1, int ldb1, int64_t sB1,
                       float* C1, int ldc1, int64_t sC1, float alpha) {
    BGemmArgs q{};
    q.M = q.N = q.K = 256;
    q.A = A; q.sA = sA; q.lda = lda;
    q.B = B; q.sB = sB; q.ldb = ldb;
    q.C = C; q.sC = sC; q.ldc = ldc;
    q.A1 = A1; q.sA1 = sA1; q.lda1 = lda1;
    q.B1 = B1; q.sB1 = sB1; q.ldb1 = ldb1;
    q.C1 = C1; q.sC1 = sC1; q.ldc1 = ldc1;
    q.nb0 = (int)nblk;
    q.alpha = alpha; q.beta = 0.f;
    launch_bgemm(mode, 2 * (int)nblk, q, s);
  };
  gj(Af, M11);                                                    // Ai = A^-1 into M11
  gemm_pair(M11, 512, SB, A12, 512, SB, Tm, 256, SH,              // T = Ai B
            A21, 512, SB, M11, 512, SB, Vm, 256, SH, 1.f);        // V = C Ai
  gemm(A21, 512, Tm, 256, A22, 512, -1.f, 1.f, SB, SH, SB);       // Sc = D - C T
  gj(A22, M22);                                                   // Si
  gemm_pair(Tm, 256, SH, M22, 512, SB, M12, 512, SB,              // M12 = -T Si
            M22, 512, SB, Vm, 256, SH, M21, 512, SB, -1.f);       // M21 = -Si V
  gemm(M12, 512, Vm, 256, M11, 512, -1.f, 1.f, SB, SH, SB);       // M11 = Ai - M12 V
  {
    int64_t off = 0;
    for (int i = 0; i < nsets; ++i) {
      if (nblks[i] <= 0) continue;
      launch_finalize_q(Mf + off * SB, 512, (int)nblks[i], outs[i].q32, outs[i].qbf, outs[i].qtbf, s);
      off += nblks[i];
    }
  }
  return check_launch("cayley builder (b=512)");
}

// Cayley blocks of several independent batches (layers, sides) with as few
// launches as possible: up to GJ_MAXSEG batches share one Gauss-Jordan launch,
// so the grid covers the blocks of all of them.  mode 6: split-bf16 x6 MFMA
// products (fp32-level accuracy); mode 0: fp32 MFMA.  Both give Q accurate
// to fp32 rounding.  b = 512 takes the blocks of all batches through one pass
// of the Schur path (ws sized for all of them together).
// skip (b <= 256): blocks in the order of the sets (empty sets left out)
// whose flag is set are not built here
int build_sets(const float* const* theta, const int64_t* nblk, const QOut* out, int nsets, int b, void* ws, int mode,
               hipStream_t s, const int* skip = nullptr) {
  int64_t total = 0;
  for (int i = 0; i < nsets; ++i) total += nblk[i];
  if (total <= 0) return POETX_OK;
  Tm tm(s, "cayley_build", 2.0 * b * (double)b * b * total, 0.0);
  if (b <= 256) {
    int i = 0;
    int64_t first = 0;   // index of this launch's first block among all
    while (i < nsets) {
      GJArgs g{};
      g.skip = skip ? skip + first : nullptr;
      int launched = 0;
      for (; i < nsets && g.nseg < GJ_MAXSEG; ++i) {
        if (nblk[i] <= 0) continue;
        g.seg[g.nseg] = GJSeg{theta[i], out[i].q32, out[i].qbf, out[i].qtbf};
        g.start[g.nseg] = launched;
        launched += (int)nblk[i];
        ++g.nseg;
      }
      g.start[g.nseg] = launched;
      if (launched > 0) launch_gj(b, mode, launched, g, s);
      first += launched;
    }
    return check_launch("cayley builder");
  }
  return build_schur512(theta, nblk, out, nsets, ws, mode, s);
}

// a layer's R and P blocks
int build2(const float* th0, int64_t n0, QOut o0, const float* th1, int64_t n1, QOut o1, int b, void* ws, int mode,
           hipStream_t s) {
  const float* th[2] = {th0, th1};
  const int64_t nb[2] = {n0, n1};
  const QOut o[2] = {o0, o1};
  return build_sets(th, nb, o, 2, b, ws, mode, s);
}

// dtheta from G = dL/dQ:  G_S = 1/2 (I + Q^T) G (I + Q^T);  dtheta_p = G_S[i][j] - G_S[j][i].
// G holds the R blocks then the P blocks contiguously; the fp32 blocks of the
// two sides may live apart (q32R, q32P).  Both sides in one pass.
// bf16 layers: fp32-accurate products on split bf16 operands (chain.hip);
// fp32 layers: fp32 MFMA products.
// split-operand chain rule over nblk blocks described by cs; T ([nblk][b][b]
// fp32) is scratch; GS (fp32 [nblk][b][b], contiguous) receives G_S and may
// alias the g arrays only when they are contiguous in block order.
void chain_bf16(const ChainSegs& cs, int nblk, int b, float* T, float* GS, int accumulate, hipStream_t s) {
  launch_chain_products(cs, nblk, b, T, GS, s);
  launch_skew_project(GS, b, nblk, cs, accumulate, s);
}

int chain(float* G, const float* q32R, const float* q32P, float* tmp, int64_t nR, int64_t nP,
          int b, float* dthR, float* dthP, bool accumulate, bool f32, hipStream_t s) {
  const int64_t nblk = nR + nP;
  if (nblk <= 0) return POETX_OK;
  Tm tm(s, "chain_rule", 4.0 * b * (double)b * b * nblk, 0.0);
  const int64_t sb = (int64_t)b * b;
  ChainSegs cs{};
  cs.nseg = 0;
  if (nR > 0) { cs.seg[cs.nseg] = ChainSeg{q32R, G, dthR}; cs.start[cs.nseg] = 0; ++cs.nseg; }
  if (nP > 0) { cs.seg[cs.nseg] = ChainSeg{q32P, G + nR * sb, dthP}; cs.start[cs.nseg] = (int)nR; ++cs.nseg; }
  cs.start[cs.nseg] = (int)nblk;
  if (!f32) {
    chain_bf16(cs, (int)nblk, b, tmp, G, accumulate ? 1 : 0, s);
  } else {
    BGemmArgs q{};
    q.M = q.N = q.K = b;
    q.A = G; q.sA = sb; q.lda = b;
    q.B = q32R; q.sB = sb; q.ldb = b; q.transB = 1; q.addIB = 1;
    q.B1 = q32P; q.nb0 = (int)nR;
    q.C = tmp; q.sC = sb; q.ldc = b;
    q.alpha = 1.f; q.beta = 0.f;
    launch_bgemm(0, (int)nblk, q, s);
    BGemmArgs r{};
    r.M = r.N = r.K = b;
    r.A = q32R; r.sA = sb; r.lda = b; r.transA = 1; r.addIA = 1;
    r.A1 = q32P; r.nb0 = (int)nR;
    r.B = tmp; r.sB = sb; r.ldb = b;
    r.C = G; r.sC = sb; r.ldc = b;
    r.alpha = 0.5f; r.beta = 0.f;
    launch_bgemm(0, (int)nblk, r, s);
    launch_skew_project(G, b, (int)nblk, cs, accumulate ? 1 : 0, s);
  }
  return check_launch("chain rule");
}

// blocks per chunk of poetx_chain_rule_sets and its workspace
constexpr int64_t kChainChunk = 512;
size_t chain_ws_bytes(int64_t total, int b) {
  const int64_t c = std::min<int64_t>(total, kChainChunk);
  if (c <= 0) return 0;
  Arena a(nullptr);
  const size_t bb = (size_t)b * b;
  a.take<float>(c * bb);   // T
  a.take<float>(c * bb);   // G_S
  return a.off + kAlign;
}

// block-product flops of one transform: N tokens x k blocks x 2 b^2
double xf_flops(int64_t N, int k, int b) { return 2.0 * N * k * (double)b * b; }

struct Shape {
  int64_t m, n, N;
  int b, kR, kP;
  bool f32;
  bool q8;    // W0p holds INT8 codes and per-row scales (POETX_W0_INT8)
  bool sep;   // POETX_SEPARATE_BLOCK_PRODUCTS
  bool tr;    // W0p followed by its transpose (POETX_W0_TRANSPOSED)
  bool xp;    // X given as x' = Pi_tau x (POETX_X_PERMUTED)
  size_t es;  // element size of activations / weight
};

Shape shape_of(const poetx_layer* L, int64_t N) {
  Shape S;
  S.m = L->m; S.n = L->n; S.N = N; S.b = L->b;
  S.kR = (int)(L->m / L->b);
  S.kP = (int)(L->n / L->b);
  S.f32 = L->dtype == POETX_F32;
  S.q8 = (L->flags & POETX_W0_INT8) != 0;
  S.sep = (L->flags & POETX_SEPARATE_BLOCK_PRODUCTS) != 0;
  S.tr = (L->flags & POETX_W0_TRANSPOSED) != 0;
  S.xp = (L->flags & POETX_X_PERMUTED) != 0;
  S.es = S.f32 ? 4 : 2;
  return S;
}

// INT8 weight format: codes [m][n], then fp32 scales [m] at this byte offset
size_t w0_scale_offset(int64_t m, int64_t n) { return ((size_t)m * n + kAlign - 1) / kAlign * kAlign; }
// transposed weight format: bf16 [m][n], then bf16 [n][m] at this byte offset
size_t w0t_offset(int64_t m, int64_t n) { return ((size_t)m * n * 2 + kAlign - 1) / kAlign * kAlign; }

// INT8 layers whose shapes the fused GEMM takes: the weight products can read
// the codes and scales directly (bf16(s q) formed inside the GEMM)
bool q8_direct(const Shape& S) { return S.q8 && S.n % 16 == 0 && S.m % 8 == 0; }
// K at which the bf16 GEMM takes its wide kernel (gemm.hip)
bool gemm_wide_k(int64_t K) { return K % 64 == 0 && K >= 2048; }
// INT8 layers whose passes read the codes directly by default: those whose
// GEMMs would not take the wide bf16 kernel in either direction.  Where they
// would, dequantizing into the workspace and running the wide kernel measured
// faster than the fused GEMM (whose weight tile is fed from registers), so
// those layers keep the dequantized copy
bool q8_fused(const Shape& S) { return q8_direct(S) && !gemm_wide_k(S.n) && !gemm_wide_k(S.m); }

// the weight operand of a pass's products: bf16 (W0p itself, or an INT8
// layer's codes dequantized into the workspace buffer w0) or INT8 codes and
// scales read by the fused GEMM
struct Wop {
  const void* bf;
  const int8_t* q;
  const float* sc;
  const void* bt;   // bf16 [n][m], the transposed copy (POETX_W0_TRANSPOSED), or null
  // INT8 layers dequantized per pass with bt the dequantized copy, transposed,
  // in buf: the codes (W0p) and buf, for the [m][n] copy the backward product
  // takes afterwards in the same buffer
  const void* q8src;
  void* q8buf;
};

// the bf16 weight a pass reads: W0p itself, or (INT8 layers) its codes
// dequantized into the pass's workspace buffer w0
const void* weight_for_pass(const Shape& S, const void* W0p, void* w0, hipStream_t s) {
  if (!S.q8) return W0p;
  const int8_t* q = static_cast<const int8_t*>(W0p);
  const float* sc = reinterpret_cast<const float*>(static_cast<const char*>(W0p) + w0_scale_offset(S.m, S.n));
  Tm tm(s, "dequant", 0.0, (double)S.m * S.n * 3);
  launch_dequant_rows(q, sc, static_cast<uint16_t*>(w0), S.m, S.n, s);
  return w0;
}

// w0 == nullptr: no room for a dequantized copy (the layer then reads its
// codes directly; callers check q8_direct first).  fwd_product: the pass runs
// the forward product z1' W0p^T, which an INT8 layer dequantized per pass
// then reads from a transposed copy as an NN GEMM, as a layer with
// POETX_W0_TRANSPOSED does (bit-identical either way)
Wop weight_operand(const Shape& S, const void* W0p, void* w0, hipStream_t s, bool fwd_product = true) {
  if (S.tr) return Wop{W0p, nullptr, nullptr, static_cast<const char*>(W0p) + w0t_offset(S.m, S.n)};
  if (S.q8 && w0 && fwd_product && !q8_fused(S)) {
    const int8_t* q = static_cast<const int8_t*>(W0p);
    const float* sc = reinterpret_cast<const float*>(static_cast<const char*>(W0p) + w0_scale_offset(S.m, S.n));
    {
      Tm tm(s, "dequant", 0.0, (double)S.m * S.n * 3);
      launch_dequant_transpose(q, sc, static_cast<uint16_t*>(w0), S.m, S.n, s);
    }
    return Wop{nullptr, nullptr, nullptr, w0, W0p, w0};
  }
  if (!(q8_fused(S) || (!w0 && q8_direct(S)))) return Wop{weight_for_pass(S, W0p, w0, s), nullptr, nullptr};
  const int8_t* q = static_cast<const int8_t*>(W0p);
  const float* sc = reinterpret_cast<const float*>(static_cast<const char*>(W0p) + w0_scale_offset(S.m, S.n));
  return Wop{nullptr, q, sc};
}

// C = A W^T (NT: M x N, K) or C = A W (NN) with the pass's weight operand
int weight_gemm(bool nn, const uint16_t* A, const Wop& W, uint16_t* C, int64_t M, int64_t N, int64_t K,
                hipStream_t s) {
  if (!W.q) {
    launch_gemm_bf16(nn, A, static_cast<const uint16_t*>(W.bf), C, M, N, K, s);
    return POETX_OK;
  }
  if (!launch_gemm_q8(nn, A, W.q, W.sc, C, M, N, K, s))
    return fail(POETX_EINVAL, "INT8 weight operand not usable by the fused GEMM (alignment)");
  return POETX_OK;
}

// Cayley blocks one forward / backward consumes (built by the call itself,
// or handed in by the caller).  fp32 layers use q32R / q32P only; bf16
// forward uses qbR, qbP; bf16 backward uses q32R, q32P (chain rule), qbP,
// qtR and qtP.
struct Blk {
  const float *q32R, *q32P;
  const uint16_t *qbR, *qbP, *qtR, *qtP;
};

// ---- workspace plans (same code sizes and carves).  own = the call builds
// its own blocks into the workspace.
struct FwdWs {
  float *q32R, *q32P;
  uint16_t *qbR, *qbP;
  void* bws;
  void *z1, *z2, *sc;
  void* w0;
};
// w0copy false: no dequantized weight for INT8 layers (their GEMMs read the
// codes; the no-allocation forward)
FwdWs plan_fwd(const Shape& S, bool own, void* base, size_t* bytes, bool w0copy = true) {
  Arena a(base);
  FwdWs w{};
  if (own) {
    if (S.f32) {
      w.q32R = a.take<float>((size_t)S.kR * S.b * S.b);
      w.q32P = a.take<float>((size_t)S.kP * S.b * S.b);
    } else {
      w.qbR = a.take<uint16_t>((size_t)S.kR * S.b * S.b);
      w.qbP = a.take<uint16_t>((size_t)S.kP * S.b * S.b);
    }
    w.bws = a.take<char>(build_ws_bytes(S.kR + S.kP, S.b));
  }
  w.z1 = a.take<char>((size_t)S.N * S.n * S.es);
  w.z2 = a.take<char>((size_t)S.N * S.m * S.es);
  if (!S.f32) w.sc = a.take<char>((size_t)S.N * std::max(S.n, S.m) * S.es);   // permuted rows / block products
  if (S.q8 && !q8_fused(S) && w0copy) w.w0 = a.take<char>((size_t)S.m * S.n * 2);   // dequantized weight
  *bytes = a.off + kAlign;
  return w;
}

struct BwdWs {
  float *q32R, *q32P;
  uint16_t *qbP, *qtR, *qtP;
  void* bws;
  void *z1, *xg, *z2, *gyg, *gz2;
  float *GR, *GP, *tmp;
  void* part;
  void* w0;
};
BwdWs plan_bwd(const Shape& S, bool own, void* base, size_t* bytes, bool dq = false) {
  Arena a(base);
  BwdWs w{};
  const size_t bb = (size_t)S.b * S.b;
  if (own) {
    w.q32R = a.take<float>((S.kR + S.kP) * bb);   // R blocks, then P blocks
    w.q32P = w.q32R ? w.q32R + S.kR * bb : nullptr;
    if (!S.f32) {
      w.qbP = a.take<uint16_t>(S.kP * bb);
      w.qtR = a.take<uint16_t>(S.kR * bb);
      w.qtP = a.take<uint16_t>(S.kP * bb);
    }
    w.bws = a.take<char>(build_ws_bytes(S.kR + S.kP, S.b));
  }
  w.z1 = a.take<char>((size_t)S.N * S.n * S.es);
  w.xg = a.take<char>((size_t)S.N * S.n * S.es);
  w.z2 = a.take<char>((size_t)S.N * S.m * S.es);
  w.gyg = a.take<char>((size_t)S.N * S.m * S.es);
  w.gz2 = a.take<char>((size_t)S.N * S.m * S.es);
  if (!dq) {   // dL/dQ and the chain rule stay inside the call
    w.GR = a.take<float>((S.kR + S.kP) * bb);     // R blocks, then P blocks
    w.GP = w.GR ? w.GR + S.kR * bb : nullptr;
    w.tmp = a.take<float>((S.kR + S.kP) * bb);
  }
  const size_t pb = std::max(gram_partials_bytes(S.N, S.b, S.kR, S.f32), gram_partials_bytes(S.N, S.b, S.kP, S.f32));
  w.part = a.take<char>(pb);
  if (S.q8 && !q8_fused(S)) w.w0 = a.take<char>((size_t)S.m * S.n * 2);   // dequantized weight
  *bytes = a.off + kAlign;
  return w;
}

// rows per segment of the in-place relayout: the rows saved aside number
// at most 2 ceil(m / L)
constexpr int kRelayoutL = 16;
int64_t relayout_max_saved(int64_t m) { return 2 * ((m + kRelayoutL - 1) / kRelayoutL) + 1; }

struct MrgWs {
  float *q32R, *q32P;
  uint16_t *qbR, *qtP;
  void* bws;
  int32_t *snew, *tnew, *sinv, *tinv;
  int32_t *dist, *hlist, *slot, *slist, *counts, *nxt;
  void* saved;
  int64_t max_saved;
  void* w0;
};
MrgWs plan_merge(const Shape& S, bool own, void* base, size_t* bytes) {
  Arena a(base);
  MrgWs w{};
  const size_t bb = (size_t)S.b * S.b;
  if (own) {
    if (S.f32) {
      w.q32R = a.take<float>(S.kR * bb);
      w.q32P = a.take<float>(S.kP * bb);
    } else {
      w.qbR = a.take<uint16_t>(S.kR * bb);
      w.qtP = a.take<uint16_t>(S.kP * bb);
    }
    w.bws = a.take<char>(build_ws_bytes(S.kR + S.kP, S.b));
  }
  w.snew = a.take<int32_t>(S.m);
  w.tnew = a.take<int32_t>(S.n);
  w.sinv = a.take<int32_t>(S.m);
  w.tinv = a.take<int32_t>(S.n);
  w.dist = a.take<int32_t>(S.m);
  w.hlist = a.take<int32_t>(S.m);
  w.slot = a.take<int32_t>(S.m);
  w.nxt = a.take<int32_t>(S.m);
  w.max_saved = relayout_max_saved(S.m);
  w.slist = a.take<int32_t>(w.max_saved);
  w.counts = a.take<int32_t>(2);
  w.saved = a.take<char>((size_t)w.max_saved * S.n * S.es);   // rows saved aside by the relayout
  if (S.q8) w.w0 = a.take<char>((size_t)S.m * S.n * 2);       // dequantized weight, merged in place
  *bytes = a.off + kAlign;
  return w;
}

int check_ws(const void* ws, size_t have, size_t need) {
  if (need == 0) return POETX_OK;
  if (!ws) return fail(POETX_EWORKSPACE, "workspace is NULL but %zu bytes are needed", need);
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(POETX_EWORKSPACE, "workspace not %zu-byte aligned", kAlign);
  if (have < need) return fail(POETX_EWORKSPACE, "workspace has %zu bytes, needs %zu", have, need);
  return POETX_OK;
}

uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// bf16 row permutation of an [N][W] token matrix (see PermArgs)
int permute(bool gather, const void* in, const void* tail_in, void* out, void* tail_out, const int32_t* perm,
            int64_t N, int W, int tail0, size_t es, hipStream_t s) {
  PermArgs p{};
  p.in = static_cast<const uint16_t*>(in);
  p.tail_in = static_cast<const uint16_t*>(tail_in);
  p.out = static_cast<uint16_t*>(out);
  p.tail_out = static_cast<uint16_t*>(tail_out);
  p.perm = perm;
  p.N = N; p.W = W; p.tail0 = tail0;
  Tm tm(s, "xform_permute", 0.0, 2.0 * N * W * es);
  launch_permute_bf16(gather, p, s);
  return check_launch(gather ? "row gather" : "row scatter");
}

// block products over contiguous columns: out[t][l*b+i] = sum_kk in[t][l*b+kk] * q[l][i][kk]
// for l < k (bf16, fp32 accumulation); columns from k*b on are not touched
int blockmul(const void* in, const uint16_t* q, void* out, int64_t N, int W, int b, int k, hipStream_t s) {
  if (k <= 0 || N <= 0) return POETX_OK;
  GemmArgs g{};
  g.A = static_cast<const uint16_t*>(in);
  g.B = q;
  g.C = static_cast<uint16_t*>(out);
  g.M = (int)N; g.N = b; g.K = b;
  g.lda = W; g.ldb = b; g.ldc = W;
  g.sA = b; g.sB = (int64_t)b * b; g.sC = b;
  g.batch = k;
  Tm tm(s, "xform_blockmul", xf_flops(N, k, b), 2.0 * N * (double)k * b * 2);
  if (!launch_blockdiag_bf16(g.A, q, g.C, N, W, W, b, k, s)) launch_gemm_bf16(false, g, s);
  return check_launch("block product");
}

// gather-in transform z = D (Pi in) over all W = k b columns, with x' = Pi in
// also written to emit (nullable) for a later Gram product: one fused pass
// where the kernel applies and measured faster (b = 256, no identity tail, up
// to 6 blocks per row), else the permutation into sc (emit, if given) and the
// block product.
int gather_blockmul(const void* in, const int32_t* perm, const uint16_t* q, void* sc, void* out, void* emit,
                    int64_t N, int W, int b, int k, size_t es, hipStream_t s) {
  if (gather_blockdiag_applies(in, perm, q, out, emit, N, W, b, k, W, W, W)) {
    {
      Tm tm(s, "xform_gather", xf_flops(N, k, b), (emit ? 6.0 : 4.0) * N * W);
      launch_gather_blockdiag_bf16(static_cast<const uint16_t*>(in), perm, q, static_cast<uint16_t*>(out),
                                   static_cast<uint16_t*>(emit), N, W, b, k, W, W, W, s);
    }
    return check_launch("gather and block product");
  }
  void* xg = emit ? emit : sc;
  int rc;
  if ((rc = permute(true, in, nullptr, xg, out, perm, N, W, k * b, es, s))) return rc;
  return blockmul(xg, q, out, N, W, b, k, s);
}

// z = D x' for an x' the caller gathered (POETX_X_PERMUTED): the block
// product over the k b block columns, and the identity tail (columns from
// k b on) copied from x'
int blockmul_permuted(const void* xp, const uint16_t* q, void* out, int64_t N, int W, int b, int k, size_t es,
                      hipStream_t s) {
  int rc;
  if ((rc = blockmul(xp, q, out, N, W, b, k, s))) return rc;
  const int t0 = k * b;
  if (t0 >= W || N <= 0) return POETX_OK;
  const size_t pitch = (size_t)W * es;
  if (hipMemcpy2DAsync(static_cast<char*>(out) + t0 * es, pitch, static_cast<const char*>(xp) + t0 * es, pitch,
                       (size_t)(W - t0) * es, (size_t)N, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return fail(POETX_EHIP, "identity-tail copy failed");
  return POETX_OK;
}

// forward after the blocks exist: a3, a4, a5
// z2out non-null (bf16): z2' goes there instead of the workspace (kept for
// the backward pass)
int fwd_core(const Shape& S, const Wop& W0, const Blk& q, const int32_t* sigma, const int32_t* tau, const void* X,
             void* Y, const FwdWs& w, hipStream_t s, void* z2out = nullptr) {
  const int64_t N = S.N;
  const int n = (int)S.n, m = (int)S.m;
  int rc;
  if (S.f32) {
    // z1' = D_P (Pi_tau x), z2' = z1' W0p^T, y = Pi_sigma^T (D_R z2'), each in one pass
    XformArgs p{};
    p.in = X; p.out = w.z1; p.perm = tau; p.N = N; p.W = n; p.B = S.b; p.k = S.kP; p.bq = q.q32P; p.trans = 0;
    {
      Tm tm(s, "xform_fp32", xf_flops(N, S.kP, S.b), 2.0 * N * n * S.es);
      launch_gather_in_f32(p, s);
    }
    {
      Tm tm(s, "gemm_fp32", 2.0 * N * S.m * S.n, (double)(N * S.n + S.m * S.n + N * S.m) * S.es);
      launch_gemm_f32(false, (const float*)w.z1, (const float*)W0.bf, (float*)w.z2, N, S.m, S.n, s);
    }
    XformArgs r{};
    r.in = w.z2; r.out = Y; r.perm = sigma; r.N = N; r.W = m; r.B = S.b; r.k = S.kR; r.bq = q.q32R; r.trans = 0;
    {
      Tm tm(s, "xform_fp32", xf_flops(N, S.kR, S.b), 2.0 * N * m * S.es);
      launch_scatter_out_f32(r, s);
    }
    return check_launch("fp32 forward");
  }
  // z1' = D_P x' with x' = Pi_tau x (the identity tail of x' goes straight to
  // z1'); with POETX_X_PERMUTED, X is x' already
  if (S.xp) rc = blockmul_permuted(X, q.qbP, w.z1, N, n, S.b, S.kP, S.es, s);
  else rc = gather_blockmul(X, tau, q.qbP, w.sc, w.z1, nullptr, N, n, S.b, S.kP, S.es, s);
  if (rc) return rc;
  // z2' = z1' W0p^T
  void* const z2 = z2out ? z2out : w.z2;
  // with the transposed copy the product is NN, z2' = z1' (W0p^T) with the
  // weight's output features along its contiguous rows; else NT on W0p.
  // b of 64 to 256 without an identity tail, z2' not kept: the R-side block
  // product in the GEMM's epilogue, r = D_R z2' straight into sc
  // (bit-identical to the two passes below)
  const bool tn = W0.bt != nullptr;
  const uint16_t* const Wf = static_cast<const uint16_t*>(tn ? W0.bt : W0.bf);
  if (!z2out && !S.sep && !W0.q && (int64_t)S.kR * S.b == m &&
      gemm_rside_applies(tn, w.z1, Wf, q.qbR, w.sc, N, S.m, S.n, S.b)) {
    {
      Tm tm(s, tn ? "gemm_nn_rside" : "gemm_nt_rside", 2.0 * N * S.m * S.n + xf_flops(N, S.kR, S.b),
            (double)(N * S.n + S.m * S.n + N * S.m) * S.es);
      launch_gemm_rside(tn, (const uint16_t*)w.z1, Wf, q.qbR, (uint16_t*)w.sc, N, S.m, S.n, S.b, s);
    }
    if ((rc = check_launch("forward GEMM with the R-side blocks"))) return rc;
    return permute(false, w.sc, z2, Y, nullptr, sigma, N, m, S.kR * S.b, S.es, s);
  }
  {
    Tm tm(s, tn ? "gemm_nn" : "gemm_nt", 2.0 * N * S.m * S.n, (double)(N * S.n + S.m * S.n + N * S.m) * S.es);
    if (tn) launch_gemm_bf16(true, (const uint16_t*)w.z1, Wf, (uint16_t*)z2, N, S.m, S.n, s);
    else if ((rc = weight_gemm(false, (const uint16_t*)w.z1, W0, (uint16_t*)z2, N, S.m, S.n, s))) return rc;
  }
  if ((rc = check_launch("forward GEMM"))) return rc;
  // y = Pi_sigma^T r with r = D_R z2' (the tail of r is the tail of z2')
  if ((rc = blockmul(z2, q.qbR, w.sc, N, m, S.b, S.kR, s))) return rc;
  return permute(false, w.sc, z2, Y, nullptr, sigma, N, m, S.kR * S.b, S.es, s);
}

// backward after the blocks exist: a0 (recompute), a6, a7, a8, a9
// gR / gP non-null: write dL/dQ there and stop before the chain rule
// z2in non-null (bf16): z2' kept from the forward pass, so a0 reduces to
// gathering x' again (no P-side block product, no forward GEMM)
int bwd_core(const Shape& S, const Wop& W0, const Blk& q, const int32_t* sigma, const int32_t* tau, const void* X,
             const void* dY, void* dX, float* dthR, float* dthP, bool accum, const BwdWs& w, hipStream_t s,
             float* gR = nullptr, float* gP = nullptr, const void* z2in = nullptr) {
  float* const GR = gR ? gR : w.GR;
  float* const GP = gR ? gP : w.GP;
  const int64_t N = S.N;
  const int n = (int)S.n, m = (int)S.m;
  int rc;
  if (S.f32) {
    // recompute z1' (keeping x' = Pi_tau x for dL/dQ_P) and z2'
    XformArgs p{};
    p.in = X; p.out = w.z1; p.emit = w.xg; p.perm = tau; p.N = N; p.W = n; p.B = S.b; p.k = S.kP; p.bq = q.q32P;
    p.trans = 0;
    {
      Tm tm(s, "xform_fp32", xf_flops(N, S.kP, S.b), 2.0 * N * n * S.es);
      launch_gather_in_f32(p, s);
    }
    {
      Tm tm(s, "gemm_fp32", 2.0 * N * S.m * S.n, (double)(N * S.n + S.m * S.n + N * S.m) * S.es);
      launch_gemm_f32(false, (const float*)w.z1, (const float*)W0.bf, (float*)w.z2, N, S.m, S.n, s);
    }
    // R side: gY' = Pi_sigma gY (kept), gz2' = D_R^T gY'
    XformArgs r{};
    r.in = dY; r.out = w.gz2; r.emit = w.gyg; r.perm = sigma; r.N = N; r.W = m; r.B = S.b; r.k = S.kR;
    r.bq = q.q32R; r.trans = 1;
    {
      Tm tm(s, "xform_fp32", xf_flops(N, S.kR, S.b), 2.0 * N * m * S.es);
      launch_gather_in_f32(r, s);
    }
  } else {
    // recompute x' = Pi_tau x (kept for dL/dQ_P), z1' = D_P x', z2' = z1' W0p^T;
    // with POETX_X_PERMUTED, X is x' already
    if (z2in) {
      if (!S.xp && (rc = permute(true, X, nullptr, w.xg, w.z1, tau, N, n, S.kP * S.b, S.es, s))) return rc;
    } else {
      if (S.xp) rc = blockmul_permuted(X, q.qbP, w.z1, N, n, S.b, S.kP, S.es, s);
      else rc = gather_blockmul(X, tau, q.qbP, nullptr, w.z1, w.xg, N, n, S.b, S.kP, S.es, s);
      if (rc) return rc;
      // NN on the transposed copy when there is one, as in the forward pass
      Tm tm(s, W0.bt ? "gemm_nn" : "gemm_nt", 2.0 * N * S.m * S.n, (double)(N * S.n + S.m * S.n + N * S.m) * S.es);
      if (W0.bt)
        launch_gemm_bf16(true, (const uint16_t*)w.z1, static_cast<const uint16_t*>(W0.bt), (uint16_t*)w.z2, N, S.m,
                         S.n, s);
      else if ((rc = weight_gemm(false, (const uint16_t*)w.z1, W0, (uint16_t*)w.z2, N, S.m, S.n, s))) return rc;
    }
    if ((rc = check_launch("recompute"))) return rc;
    // R side: gY' = Pi_sigma gY (kept), gz2' = D_R^T gY' (blocks Q_R^T)
    if ((rc = gather_blockmul(dY, sigma, q.qtR, nullptr, w.gz2, w.gyg, N, m, S.b, S.kR, S.es, s))) return rc;
  }
  // G_R = gY'^T z2' per block
  {
    // algorithmic bytes: the reads of gY' and z2'
    Tm tm(s, "gram", xf_flops(N, S.kR, S.b), 2.0 * N * S.m * S.es);
    launch_gram(S.f32, w.gyg, z2in ? z2in : w.z2, N, m, S.b, S.kR, GR, w.part, s);
  }
  if ((rc = check_launch("R-side backward"))) return rc;
  // gz1' = gz2' W0p (into the z1' buffer)
  void* gz1 = w.z1;
  {
    // an INT8 layer whose buffer held the transposed copy for the recompute
    // takes its [m][n] dequantized copy there now
    Wop Wn = W0;
    if (W0.q8src) {
      Wn.bf = weight_for_pass(S, W0.q8src, W0.q8buf, s);
      Wn.bt = nullptr;
    }
    Tm tm(s, S.f32 ? "gemm_fp32" : "gemm_nn", 2.0 * N * S.m * S.n, (double)(N * S.n + S.m * S.n + N * S.m) * S.es);
    if (S.f32) launch_gemm_f32(true, (const float*)w.gz2, (const float*)W0.bf, (float*)gz1, N, S.n, S.m, s);
    else if ((rc = weight_gemm(true, (const uint16_t*)w.gz2, Wn, (uint16_t*)gz1, N, S.n, S.m, s))) return rc;
  }
  // G_P = gz1'^T x' per block
  {
    Tm tm(s, "gram", xf_flops(N, S.kP, S.b), 2.0 * N * S.n * S.es);
    launch_gram(S.f32, gz1, S.xp ? X : w.xg, N, n, S.b, S.kP, GP, w.part, s);
  }
  if ((rc = check_launch("P-side gradient"))) return rc;
  // dX = Pi_tau^T D_P^T gz1'
  if (dX) {
    if (S.f32) {
      XformArgs t{};
      t.in = gz1; t.out = dX; t.perm = tau; t.N = N; t.W = n; t.B = S.b; t.k = S.kP; t.bq = q.q32P; t.trans = 1;
      Tm tm(s, "xform_fp32", xf_flops(N, S.kP, S.b), 2.0 * N * n * S.es);
      launch_scatter_out_f32(t, s);
    } else {
      // x' is no longer needed: its buffer takes the block products
      if ((rc = blockmul(gz1, q.qtP, w.xg, N, n, S.b, S.kP, s))) return rc;
      if ((rc = permute(false, w.xg, gz1, dX, nullptr, tau, N, n, S.kP * S.b, S.es, s))) return rc;
    }
  }
  if ((rc = check_launch("P-side backward"))) return rc;
  if (gR) return POETX_OK;
  // chain rule through the Cayley map onto the stored upper triangle
  return chain(w.GR, q.q32R, q.q32P, w.tmp, S.kR, S.kP, S.b, dthR, dthP, accum, S.f32, s);
}

// INT8 weights read by the fused GEMM: 16 codes per load
int check_w0_int8_align(const Shape& S, const void* W0p) {
  if (S.N > 0 && q8_direct(S) && reinterpret_cast<uintptr_t>(W0p) % 16)
    return fail(POETX_EINVAL, "INT8 W0p not 16-byte aligned");
  return POETX_OK;
}

// shared argument checks of forward / forward_blocks
int check_fwd_args(const poetx_layer* layer, int64_t N, const void* W0p, const int32_t* sigma, const int32_t* tau,
                   const void* X, const void* Y) {
  int rc = validate_layer(layer);
  if (rc) return rc;
  if ((rc = validate_N(N))) return rc;
  if (N > 0 && (!W0p || !sigma || !tau || !X || !Y)) return fail(POETX_EINVAL, "NULL tensor argument");
  return check_w0_int8_align(shape_of(layer, N), W0p);
}

int check_bwd_args(const poetx_layer* layer, int64_t N, const void* W0p, const int32_t* sigma, const int32_t* tau,
                   const void* X, const void* dY, const float* dthR, const float* dthP) {
  int rc = validate_layer(layer);
  if (rc) return rc;
  if ((rc = validate_N(N))) return rc;
  const Shape S = shape_of(layer, N);
  if (N > 0 && (!W0p || !sigma || !tau || !X || !dY)) return fail(POETX_EINVAL, "NULL tensor argument");
  if ((S.kR > 0 && !dthR) || (S.kP > 0 && !dthP)) return fail(POETX_EINVAL, "NULL generator gradient");
  return check_w0_int8_align(S, W0p);
}

// gradient reset of an empty backward
int zero_grads(const Shape& S, bool accum, float* dthR, float* dthP, hipStream_t s) {
  if (!accum) {
    launch_fill_f32(dthR, 0.f, (int64_t)S.kR * (S.b * (S.b - 1) / 2), s);
    launch_fill_f32(dthP, 0.f, (int64_t)S.kP * (S.b * (S.b - 1) / 2), s);
  }
  return check_launch("zero gradients");
}

int check_merge_blocks(const Shape& S, const poetx_blocks* q) {
  if (!q) return fail(POETX_EINVAL, "blocks is NULL");
  const bool R = S.kR > 0, P = S.kP > 0;
  if (S.f32 && ((R && !q->Q32R) || (P && !q->Q32P))) return fail(POETX_EINVAL, "NULL fp32 blocks (Q32R / Q32P)");
  if (!S.f32 && ((R && !q->QR) || (P && !q->QTP))) return fail(POETX_EINVAL, "NULL bf16 blocks (QR / QTP)");
  return POETX_OK;
}

int check_blocks(const Shape& S, const poetx_blocks* q, bool backward) {
  if (!q) return fail(POETX_EINVAL, "blocks is NULL");
  const bool R = S.kR > 0, P = S.kP > 0;
  if (S.f32 || backward) {
    if ((R && !q->Q32R) || (P && !q->Q32P)) return fail(POETX_EINVAL, "NULL fp32 blocks (Q32R / Q32P)");
  }
  if (!S.f32 && !backward && ((R && !q->QR) || (P && !q->QP)))
    return fail(POETX_EINVAL, "NULL bf16 blocks (QR / QP)");
  if (!S.f32 && backward && ((P && !q->QP) || (R && !q->QTR) || (P && !q->QTP)))
    return fail(POETX_EINVAL, "NULL bf16 blocks (QP / QTR / QTP)");
  return POETX_OK;
}

// merge after the blocks exist: tile products, new permutations, relayout,
// generator reset (a10, a11), all on W0p in place.
// bf16 products on the streaming kernels, where they apply (b <= 256, rows of
// a multiple of 8 columns up to 32768, 16-byte aligned operands):
//   W0p <- W0p D_P        block product, row by row
//   W0p[I] <- Q_R,I W0p[I] batched NN GEMM over the kR row blocks with C = B:
//                         at b <= 256 one 256-row output tile covers a row
//                         block, so each workgroup reads exactly the slab
//                         columns it writes, and no other workgroup touches
//                         them; tail rows stay
// otherwise: the staged tile kernels of launch_merge_products_inplace.
// One bf16 rounding after each product.  Then the new permutations, and
// W0p[i][j] <- W0p[sinv(snew(i))][tinv(tnew(j))] along the cycles of the
// row map, with at most relayout_max_saved(m) rows saved aside.
bool merge_fast_products_bf16(const Shape& S, void* W0p, const Blk& q, hipStream_t s) {
  const int64_t m = S.m, n = S.n;
  const int b = S.b;
  if (S.f32 || b > 256 || (n & 7) || n > 32768 || !q.qbR || !q.qtP) return false;
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  if (!al(W0p) || !al(q.qbR) || !al(q.qtP)) return false;
  uint16_t* W = static_cast<uint16_t*>(W0p);
  if (S.kP > 0 && !launch_blockdiag_bf16(W, q.qtP, W, m, n, n, b, S.kP, s)) return false;
  if (S.kR > 0) {
    GemmArgs g{};
    g.A = q.qbR; g.B = W; g.C = W;
    g.M = b; g.N = (int)n; g.K = b;
    g.lda = b; g.ldb = n; g.ldc = n;
    g.sA = (int64_t)b * b; g.sB = (int64_t)b * n; g.sC = (int64_t)b * n;
    g.batch = S.kR;
    launch_gemm_bf16(true, g, s);
  }
  return true;
}

// W0p <- R W0p P where it lies (the merge's block products)
int merge_products(const Shape& S, void* W0p, const Blk& q, hipStream_t s) {
  {
    Tm tm(s, "merge_tiles", 4.0 * S.m * S.n * S.b, 2.0 * S.m * S.n * S.es);
    if (!merge_fast_products_bf16(S, W0p, q, s)) {
      if (S.f32) launch_merge_products_inplace(true, W0p, q.q32R, q.q32P, S.m, S.n, S.b, S.kR, S.kP, s);
      else launch_merge_products_inplace(false, W0p, q.qbR, q.qtP, S.m, S.n, S.b, S.kR, S.kP, s);
    }
  }
  return check_launch("merge products");
}

int merge_core(const Shape& S, void* W0p, const Blk& q, float* thR, float* thP, int32_t* sigma, int32_t* tau,
               uint64_t perm_seed, uint64_t merge_index, const MrgWs& w, hipStream_t s) {
  int rc;
  if ((rc = merge_products(S, W0p, q, s))) return rc;
  {
    // new permutations, old inverses; then the composed maps in place of the new ones
    Tm tm(s, "merge_permutations", 0.0, 0.0);
    launch_merge_permutations(perm_seed, merge_index, sigma, tau, S.m, S.n, w.snew, w.tnew, w.sinv, w.tinv, s);
  }
  {
    Tm tm(s, "merge_relayout", 0.0, 2.0 * S.m * S.n * S.es);
    launch_relayout_inplace(S.f32, W0p, w.saved, w.snew, w.tnew, S.m, S.n, kRelayoutL, w.dist, w.hlist, w.slot,
                            w.slist, w.counts, w.nxt, w.max_saved, s);
  }
  launch_fill2_f32(thR, (int64_t)S.kR * (S.b * (S.b - 1) / 2), thP, (int64_t)S.kP * (S.b * (S.b - 1) / 2), 0.f, s);
  return check_launch("merge relayout");
}

// merge of the layer's stored weight: INT8 layers merge their dequantized
// weight in the workspace and store its new codes and scales
// the transposed copy of a merged weight (POETX_W0_TRANSPOSED)
int refresh_transpose(const Shape& S, void* W0p, hipStream_t s) {
  if (!S.tr) return POETX_OK;
  {
    Tm tm(s, "transpose", 0.0, 4.0 * S.m * S.n);
    launch_transpose_bf16(static_cast<const uint16_t*>(W0p),
                          reinterpret_cast<uint16_t*>(static_cast<char*>(W0p) + w0t_offset(S.m, S.n)), S.m, S.n, s);
  }
  return check_launch("weight transpose");
}

int merge_w0(const Shape& S, void* W0p, const Blk& q, float* thR, float* thP, int32_t* sigma, int32_t* tau,
             uint64_t seed, uint64_t merge_index, const MrgWs& w, hipStream_t s) {
  if (!S.q8) {
    const int rc = merge_core(S, W0p, q, thR, thP, sigma, tau, seed, merge_index, w, s);
    return rc ? rc : refresh_transpose(S, W0p, s);
  }
  weight_for_pass(S, W0p, w.w0, s);
  int rc = merge_core(S, w.w0, q, thR, thP, sigma, tau, seed, merge_index, w, s);
  if (rc) return rc;
  int8_t* codes = static_cast<int8_t*>(W0p);
  float* sc = reinterpret_cast<float*>(static_cast<char*>(W0p) + w0_scale_offset(S.m, S.n));
  {
    Tm tm(s, "quantize", 0.0, (double)S.m * S.n * 3);
    launch_quantize_rows(static_cast<const uint16_t*>(w.w0), codes, sc, S.m, S.n, s);
  }
  return check_launch("weight quantization");
}

Blk blk_of(const poetx_blocks* q) {
  return Blk{q->Q32R, q->Q32P, static_cast<const uint16_t*>(q->QR), static_cast<const uint16_t*>(q->QP),
             static_cast<const uint16_t*>(q->QTR), static_cast<const uint16_t*>(q->QTP)};
}

// poetx_forward_blocks(_z2): Z2 non-null keeps z2' for the backward pass
int forward_blocks_impl(const poetx_layer* layer, const void* W0p, const poetx_blocks* blocks, const int32_t* sigma,
                        const int32_t* tau, const void* X, int64_t N, void* Y, void* Z2, void* ws, size_t ws_bytes,
                        void* stream) {
  int rc = check_fwd_args(layer, N, W0p, sigma, tau, X, Y);
  if (rc) return rc;
  const Shape S = shape_of(layer, N);
  if ((rc = check_blocks(S, blocks, false))) return rc;
  if (N == 0) return POETX_OK;
  size_t need = 0;
  plan_fwd(S, false, nullptr, &need);
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  const FwdWs w = plan_fwd(S, false, ws, &need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return fwd_core(S, weight_operand(S, W0p, w.w0, s), blk_of(blocks), sigma, tau, X, Y, w, s, Z2);
}

// poetx_backward_blocks_dq(_z2): Z2 non-null is z2' kept from the forward pass
int backward_dq_impl(const poetx_layer* layer, const void* W0p, const poetx_blocks* blocks, const int32_t* sigma,
                     const int32_t* tau, const void* X, const void* dY, const void* Z2, int64_t N, void* dX,
                     float* GR, float* GP, void* ws, size_t ws_bytes, void* stream, const char* fn) {
  int rc = check_bwd_args(layer, N, W0p, sigma, tau, X, dY, GR, GP);
  if (rc) return rc;
  if (layer->flags & POETX_ACCUMULATE_GRAD)
    return fail(POETX_EINVAL, "POETX_ACCUMULATE_GRAD applies to poetx_chain_rule_sets, not to dL/dQ");
  const Shape S = shape_of(layer, N);
  if (S.f32) return fail(POETX_EDTYPE, "%s takes bf16 layers", fn);
  if ((rc = check_blocks(S, blocks, true))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N == 0) {
    launch_fill_f32(GR, 0.f, (int64_t)S.kR * S.b * S.b, s);
    launch_fill_f32(GP, 0.f, (int64_t)S.kP * S.b * S.b, s);
    return check_launch("zero dL/dQ");
  }
  size_t need = 0;
  plan_bwd(S, false, nullptr, &need, true);
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  const BwdWs w = plan_bwd(S, false, ws, &need, true);
  return bwd_core(S, weight_operand(S, W0p, w.w0, s, Z2 == nullptr), blk_of(blocks), sigma, tau, X, dY, dX, nullptr,
                  nullptr, false, w, s, GR, GP, Z2);
}

// ---- allocation-free forward: intermediates in a file-scope device array
// (one per GPU, held until the process ends) instead of a caller workspace.
// Host code never passes the array's name to a kernel: its device address is
// taken once per device with hipGetSymbolAddress and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of `scratch` on the current device
int scratch_on_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(POETX_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(POETX_EHIP, "device %d out of range [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(POETX_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return POETX_OK;
}

// tokens per chunk of the allocation-free forward: the largest multiple of
// 128 whose forward workspace fits the scratch (128 rows keep every chunk's
// row starts at the alignment of the first, so chunks take the same kernels
// as one call over all tokens); 0 if not even 128 tokens fit
int64_t noalloc_chunk(const poetx_layer* layer) {
  const Shape S1 = shape_of(layer, 1);
  const int64_t per_token = (S1.n + S1.m + (S1.f32 ? 0 : std::max(S1.n, S1.m))) * (int64_t)S1.es;
  int64_t c = ((int64_t)kScratchBytes - 8 * (int64_t)kAlign) / per_token / 128 * 128;
  for (; c >= 128; c -= 128) {
    size_t need = 0;
    plan_fwd(shape_of(layer, c), false, nullptr, &need, false);
    if (need <= kScratchBytes) return c;
  }
  return 0;
}

}  // namespace

extern "C" {

const char* poetx_last_error(void) { return g_err.c_str(); }

size_t poetx_build_workspace_bytes(int64_t nblocks, int32_t b) {
  if (!valid_b(b) || nblocks < 0) {
    fail(POETX_EINVAL, "bad build request nblocks=%lld b=%d", (long long)nblocks, b);
    return 0;
  }
  return build_ws_bytes(nblocks, b);
}

size_t poetx_workspace_bytes(const poetx_layer* layer, int64_t N, int op) {
  if (validate_layer(layer) != POETX_OK) return 0;
  const bool merge_op = op == POETX_OP_MERGE || op == POETX_OP_MERGE_BLOCKS;
  if (!merge_op && validate_N(N) != POETX_OK) return 0;
  const Shape S = shape_of(layer, merge_op ? 0 : N);
  size_t bytes = 0;
  switch (op) {
    case POETX_OP_FORWARD: plan_fwd(S, true, nullptr, &bytes); break;
    case POETX_OP_BACKWARD: plan_bwd(S, true, nullptr, &bytes); break;
    case POETX_OP_FORWARD_BLOCKS: plan_fwd(S, false, nullptr, &bytes); break;
    case POETX_OP_BACKWARD_BLOCKS: plan_bwd(S, false, nullptr, &bytes); break;
    case POETX_OP_BACKWARD_DQ: plan_bwd(S, false, nullptr, &bytes, true); break;
    case POETX_OP_MERGE: plan_merge(S, true, nullptr, &bytes); break;
    case POETX_OP_MERGE_BLOCKS: plan_merge(S, false, nullptr, &bytes); break;
    default: fail(POETX_EINVAL, "unknown op %d", op); return 0;
  }
  return bytes;
}

int poetx_build_blocks(const float* theta, int64_t nblocks, int32_t b, float* Q32, void* Qbf16, void* QTbf16,
                       void* ws, size_t ws_bytes, void* stream) {
  poetx_block_set set{theta, nblocks, Q32, Qbf16, QTbf16};
  return poetx_build_block_sets(&set, 1, b, ws, ws_bytes, stream);
}

int poetx_build_block_sets(const poetx_block_set* sets, int32_t count, int32_t b, void* ws, size_t ws_bytes,
                           void* stream) {
  if (!valid_b(b)) return fail(POETX_EINVAL, "block size b=%d not in {32,64,128,256,512}", b);
  if (count < 0 || count > 4096) return fail(POETX_ESHAPE, "count=%d out of range [0, 4096]", count);
  if (count > 0 && !sets) return fail(POETX_EINVAL, "sets is NULL");
  int64_t total = 0;
  for (int i = 0; i < count; ++i) {
    const poetx_block_set& t = sets[i];
    if (t.nblocks < 0 || t.nblocks > (int64_t(1) << 20))
      return fail(POETX_ESHAPE, "set %d: nblocks=%lld", i, (long long)t.nblocks);
    if (t.nblocks == 0) continue;
    if (!t.theta) return fail(POETX_EINVAL, "set %d: theta is NULL", i);
    if (!t.Q32 && !t.Qbf16 && !t.QTbf16) return fail(POETX_EINVAL, "set %d: no output requested", i);
    total += t.nblocks;
  }
  if (total > (int64_t(1) << 24)) return fail(POETX_ESHAPE, "%lld blocks in one call", (long long)total);
  if (total == 0) return POETX_OK;
  const int rc = check_ws(ws, ws_bytes, build_ws_bytes(total, b));
  if (rc) return rc;
  std::vector<const float*> th((size_t)count);
  std::vector<int64_t> nb((size_t)count);
  std::vector<QOut> out((size_t)count);
  for (int i = 0; i < count; ++i) {
    th[(size_t)i] = sets[i].theta;
    nb[(size_t)i] = sets[i].nblocks;
    out[(size_t)i] = QOut{sets[i].Q32, static_cast<uint16_t*>(sets[i].Qbf16), static_cast<uint16_t*>(sets[i].QTbf16)};
  }
  return build_sets(th.data(), nb.data(), out.data(), count, b, ws, 6, static_cast<hipStream_t>(stream));
}

size_t poetx_build_cnp_workspace_bytes(int64_t total_blocks, int32_t b) {
  if (!valid_b(b) || b > 256 || total_blocks < 0) {
    fail(POETX_EINVAL, "bad CNP request total_blocks=%lld b=%d", (long long)total_blocks, b);
    return 0;
  }
  const size_t bb = (size_t)b * b;
  Arena a(nullptr);
  a.take<float>((size_t)total_blocks * bb);   // S
  a.take<float>((size_t)total_blocks * bb);   // Horner buffers
  a.take<float>((size_t)total_blocks * bb);
  a.take<int>((size_t)total_blocks);          // per-block choice
  return a.off + kAlign;
}

int poetx_build_block_sets_cnp(const poetx_block_set* sets, int32_t count, int32_t b, int32_t terms, void* ws,
                               size_t ws_bytes, void* stream) {
  if (!valid_b(b) || b > 256) return fail(POETX_EINVAL, "block size b=%d not in {32,64,128,256}", b);
  if (terms < 1 || terms > 16) return fail(POETX_EINVAL, "terms=%d out of range [1, 16]", terms);
  if (count < 0 || count > 4096) return fail(POETX_ESHAPE, "count=%d out of range [0, 4096]", count);
  if (count > 0 && !sets) return fail(POETX_EINVAL, "sets is NULL");
  int64_t total = 0;
  for (int i = 0; i < count; ++i) {
    const poetx_block_set& t = sets[i];
    if (t.nblocks < 0 || t.nblocks > 65535) return fail(POETX_ESHAPE, "set %d: nblocks=%lld", i, (long long)t.nblocks);
    if (t.nblocks == 0) continue;
    if (!t.theta) return fail(POETX_EINVAL, "set %d: theta is NULL", i);
    if (!t.Q32 && !t.Qbf16 && !t.QTbf16) return fail(POETX_EINVAL, "set %d: no output requested", i);
    total += t.nblocks;
  }
  if (total > 65535) return fail(POETX_ESHAPE, "%lld blocks in one call (at most 65535)", (long long)total);
  if (total == 0) return POETX_OK;
  int rc = check_ws(ws, ws_bytes, poetx_build_cnp_workspace_bytes(total, b));
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t bb = (size_t)b * b;
  Arena a(ws);
  float* S = a.take<float>((size_t)total * bb);
  float* T[2] = {a.take<float>((size_t)total * bb), a.take<float>((size_t)total * bb)};
  int* use = a.take<int>((size_t)total);
  std::vector<const float*> th;
  std::vector<int64_t> nb;
  std::vector<QOut> out;
  for (int i = 0; i < count; ++i) {
    if (sets[i].nblocks == 0) continue;
    th.push_back(sets[i].theta);
    nb.push_back(sets[i].nblocks);
    out.push_back(QOut{sets[i].Q32, static_cast<uint16_t*>(sets[i].Qbf16), static_cast<uint16_t*>(sets[i].QTbf16)});
  }
  {
    Tm tm(s, "cayley_cnp", 4.0 * (terms - 1) * (double)b * bb * total, 0.0);
    int64_t off = 0;
    for (size_t i = 0; i < th.size(); ++i) {
      launch_cnp_unpack_s(th[i], b, (int)nb[i], S + off * bb, s);
      off += nb[i];
    }
    launch_cnp_guard(S, b, (int)total, terms, kCnpTol, use, s);
    // Horner: T_1 = S, T_j = S (I + T_{j-1}), fp32-accurate split products,
    // only for the blocks that take the series
    const float* cur = S;
    for (int j = 2; j <= terms; ++j) {
      BGemmArgs q{};
      q.M = q.N = q.K = b;
      q.A = S; q.sA = (int64_t)bb; q.lda = b;
      q.B = cur; q.sB = (int64_t)bb; q.ldb = b; q.addIB = 1;
      q.C = T[j & 1]; q.sC = (int64_t)bb; q.ldc = b;
      q.alpha = 1.f; q.beta = 0.f;
      q.nb0 = (int)total;
      q.run = use;
      launch_bgemm(6, (int)total, q, s);
      cur = q.C;
    }
    off = 0;
    for (size_t i = 0; i < th.size(); ++i) {
      launch_cnp_finalize(cur + off * bb, use + off, b, (int)nb[i], out[i].q32, out[i].qbf, out[i].qtbf, s);
      off += nb[i];
    }
    if ((rc = check_launch("truncated-series builder"))) return rc;
  }
  // every other block: the exact solve (nothing else in the workspace is
  // needed for b <= 256)
  return build_sets(th.data(), nb.data(), out.data(), (int)th.size(), b, nullptr, 6, s, use);
}

int poetx_forward(const poetx_layer* layer, const void* W0p, const float* thR, const float* thP,
                  const int32_t* sigma, const int32_t* tau, const void* X, int64_t N, void* Y, void* ws,
                  size_t ws_bytes, void* stream) {
  int rc = check_fwd_args(layer, N, W0p, sigma, tau, X, Y);
  if (rc) return rc;
  if (N == 0) return POETX_OK;
  const Shape S = shape_of(layer, N);
  if ((S.kR > 0 && !thR) || (S.kP > 0 && !thP)) return fail(POETX_EINVAL, "NULL generator");
  size_t need = 0;
  plan_fwd(S, true, nullptr, &need);
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  const FwdWs w = plan_fwd(S, true, ws, &need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int bmode = S.f32 ? 0 : 6;
  // Cayley blocks (recomputed every call; nothing is cached between calls)
  if (S.f32) rc = build2(thR, S.kR, QOut{w.q32R, nullptr, nullptr}, thP, S.kP, QOut{w.q32P, nullptr, nullptr}, S.b,
                       w.bws, bmode, s);
  else rc = build2(thR, S.kR, QOut{nullptr, w.qbR, nullptr}, thP, S.kP, QOut{nullptr, w.qbP, nullptr}, S.b, w.bws,
                   bmode, s);
  if (rc) return rc;
  return fwd_core(S, weight_operand(S, W0p, w.w0, s), Blk{w.q32R, w.q32P, w.qbR, w.qbP, nullptr, nullptr}, sigma,
                  tau, X, Y, w, s);
}

int poetx_forward_blocks(const poetx_layer* layer, const void* W0p, const poetx_blocks* blocks,
                         const int32_t* sigma, const int32_t* tau, const void* X, int64_t N, void* Y, void* ws,
                         size_t ws_bytes, void* stream) {
  return forward_blocks_impl(layer, W0p, blocks, sigma, tau, X, N, Y, nullptr, ws, ws_bytes, stream);
}

int poetx_forward_blocks_z2(const poetx_layer* layer, const void* W0p, const poetx_blocks* blocks,
                            const int32_t* sigma, const int32_t* tau, const void* X, int64_t N, void* Y, void* Z2,
                            void* ws, size_t ws_bytes, void* stream) {
  if (layer && layer->dtype == POETX_F32) return fail(POETX_EDTYPE, "poetx_forward_blocks_z2 takes bf16 layers");
  if (N > 0 && !Z2) return fail(POETX_EINVAL, "Z2 is NULL");
  return forward_blocks_impl(layer, W0p, blocks, sigma, tau, X, N, Y, Z2, ws, ws_bytes, stream);
}

int poetx_permute_input(const poetx_layer* layer, const int32_t* tau, const void* X, int64_t N, void* Xp,
                        void* stream) {
  int rc = validate_layer(layer);
  if (rc) return rc;
  if ((rc = validate_N(N))) return rc;
  const Shape S = shape_of(layer, N);
  if (S.f32) return fail(POETX_EDTYPE, "poetx_permute_input takes bf16 layers");
  if (N > 0 && (!tau || !X || !Xp)) return fail(POETX_EINVAL, "NULL tensor argument");
  if (N == 0) return POETX_OK;
  return permute(true, X, nullptr, Xp, Xp, tau, N, (int)S.n, S.kP * S.b, S.es, static_cast<hipStream_t>(stream));
}

int poetx_forward_blocks_noalloc(const poetx_layer* layer, const void* W0p, const poetx_blocks* blocks,
                                 const int32_t* sigma, const int32_t* tau, const void* X, int64_t N, void* Y,
                                 void* stream) {
  int rc = check_fwd_args(layer, N, W0p, sigma, tau, X, Y);
  if (rc) return rc;
  const Shape S0 = shape_of(layer, N);
  if (S0.q8 && !q8_direct(S0))
    return fail(POETX_EINVAL, "poetx_forward_blocks_noalloc: POETX_W0_INT8 layers with n %% 16 or m %% 8 nonzero "
                              "need a dequantized weight (m*n*2 bytes) beside the scratch; use poetx_forward_blocks");
  if ((rc = check_blocks(S0, blocks, false))) return rc;
  if (N == 0) return POETX_OK;
  const int64_t chunk = noalloc_chunk(layer);
  if (chunk <= 0)
    return fail(POETX_ESHAPE, "poetx_forward_blocks_noalloc: 128 tokens of m=%lld n=%lld exceed the %zu-byte scratch",
                (long long)S0.m, (long long)S0.n, kScratchBytes);
  void* base = nullptr;
  if ((rc = scratch_on_device(&base))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Blk q = blk_of(blocks);
  for (int64_t t0 = 0; t0 < N; t0 += chunk) {
    const Shape S = shape_of(layer, std::min(chunk, N - t0));
    size_t need = 0;
    const FwdWs w = plan_fwd(S, false, base, &need, false);
    if (need > kScratchBytes) return fail(POETX_EWORKSPACE, "scratch plan of %zu bytes", need);
    // INT8 layers here read their codes in the GEMM (no dequantized copy)
    const Wop W0 = weight_operand(S, W0p, nullptr, s);
    rc = fwd_core(S, W0, q, sigma, tau, static_cast<const char*>(X) + t0 * S.n * (int64_t)S.es,
                  static_cast<char*>(Y) + t0 * S.m * (int64_t)S.es, w, s);
    if (rc) return rc;
  }
  return POETX_OK;
}

int poetx_backward(const poetx_layer* layer, const void* W0p, const float* thR, const float* thP,
                   const int32_t* sigma, const int32_t* tau, const void* X, const void* dY, int64_t N, void* dX,
                   float* dthR, float* dthP, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_bwd_args(layer, N, W0p, sigma, tau, X, dY, dthR, dthP);
  if (rc) return rc;
  const Shape S = shape_of(layer, N);
  if ((S.kR > 0 && !thR) || (S.kP > 0 && !thP)) return fail(POETX_EINVAL, "NULL generator");
  const bool accum = (layer->flags & POETX_ACCUMULATE_GRAD) != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N == 0) return zero_grads(S, accum, dthR, dthP, s);
  size_t need = 0;
  plan_bwd(S, true, nullptr, &need);
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  const BwdWs w = plan_bwd(S, true, ws, &need);
  const int bmode = S.f32 ? 0 : 6;   // Cayley builder
  // recompute the blocks (not stored between forward and backward)
  if (S.f32) rc = build2(thR, S.kR, QOut{w.q32R, nullptr, nullptr}, thP, S.kP, QOut{w.q32P, nullptr, nullptr}, S.b,
                       w.bws, bmode, s);
  else rc = build2(thR, S.kR, QOut{w.q32R, nullptr, w.qtR}, thP, S.kP, QOut{w.q32P, w.qbP, w.qtP}, S.b, w.bws,
                   bmode, s);
  if (rc) return rc;
  return bwd_core(S, weight_operand(S, W0p, w.w0, s), Blk{w.q32R, w.q32P, nullptr, w.qbP, w.qtR, w.qtP}, sigma,
                  tau, X, dY, dX, dthR, dthP,
                  accum, w, s);
}

int poetx_backward_blocks(const poetx_layer* layer, const void* W0p, const poetx_blocks* blocks,
                          const int32_t* sigma, const int32_t* tau, const void* X, const void* dY, int64_t N,
                          void* dX, float* dthR, float* dthP, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_bwd_args(layer, N, W0p, sigma, tau, X, dY, dthR, dthP);
  if (rc) return rc;
  const Shape S = shape_of(layer, N);
  if ((rc = check_blocks(S, blocks, true))) return rc;
  const bool accum = (layer->flags & POETX_ACCUMULATE_GRAD) != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N == 0) return zero_grads(S, accum, dthR, dthP, s);
  size_t need = 0;
  plan_bwd(S, false, nullptr, &need);
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  const BwdWs w = plan_bwd(S, false, ws, &need);
  return bwd_core(S, weight_operand(S, W0p, w.w0, s), blk_of(blocks), sigma, tau, X, dY, dX, dthR, dthP, accum,
                  w, s);
}

int poetx_backward_blocks_dq(const poetx_layer* layer, const void* W0p, const poetx_blocks* blocks,
                             const int32_t* sigma, const int32_t* tau, const void* X, const void* dY, int64_t N,
                             void* dX, float* GR, float* GP, void* ws, size_t ws_bytes, void* stream) {
  return backward_dq_impl(layer, W0p, blocks, sigma, tau, X, dY, nullptr, N, dX, GR, GP, ws, ws_bytes, stream,
                          "poetx_backward_blocks_dq");
}

int poetx_backward_blocks_dq_z2(const poetx_layer* layer, const void* W0p, const poetx_blocks* blocks,
                                const int32_t* sigma, const int32_t* tau, const void* X, const void* dY,
                                const void* Z2, int64_t N, void* dX, float* GR, float* GP, void* ws,
                                size_t ws_bytes, void* stream) {
  if (N > 0 && !Z2) return fail(POETX_EINVAL, "Z2 is NULL");
  return backward_dq_impl(layer, W0p, blocks, sigma, tau, X, dY, Z2, N, dX, GR, GP, ws, ws_bytes, stream,
                          "poetx_backward_blocks_dq_z2");
}

size_t poetx_chain_workspace_bytes(int64_t total_blocks, int32_t b) {
  if (!valid_b(b) || total_blocks < 0) {
    fail(POETX_EINVAL, "bad chain request total_blocks=%lld b=%d", (long long)total_blocks, b);
    return 0;
  }
  return chain_ws_bytes(total_blocks, b);
}

int poetx_chain_rule_sets(const poetx_chain_set* sets, int32_t count, int32_t b, uint32_t flags, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!valid_b(b)) return fail(POETX_EINVAL, "block size b=%d not in {32,64,128,256,512}", b);
  if (count < 0 || count > 65536) return fail(POETX_ESHAPE, "count=%d out of range [0, 65536]", count);
  if (count > 0 && !sets) return fail(POETX_EINVAL, "sets is NULL");
  if (flags & ~POETX_ACCUMULATE_GRAD) return fail(POETX_EINVAL, "unknown flags 0x%x", flags);
  int64_t total = 0;
  for (int i = 0; i < count; ++i) {
    const poetx_chain_set& t = sets[i];
    if (t.nblocks < 0 || t.nblocks > (int64_t(1) << 20))
      return fail(POETX_ESHAPE, "set %d: nblocks=%lld", i, (long long)t.nblocks);
    if (t.nblocks > 0 && (!t.Q32 || !t.G || !t.dtheta)) return fail(POETX_EINVAL, "set %d: NULL array", i);
    total += t.nblocks;
  }
  if (total > (int64_t(1) << 24)) return fail(POETX_ESHAPE, "%lld blocks in one call", (long long)total);
  if (total == 0) return POETX_OK;
  const int rc = check_ws(ws, ws_bytes, chain_ws_bytes(total, b));
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t chunk = std::min<int64_t>(total, kChainChunk);
  const size_t bb = (size_t)b * b;
  Arena a(ws);
  float* T = a.take<float>(chunk * bb);
  float* GS = a.take<float>(chunk * bb);
  Tm tm(s, "chain_rule", 4.0 * b * (double)b * b * total, 0.0);
  // walk the sets in chunks of at most kChainChunk blocks and CH_MAXSEG pieces
  int si = 0;
  int64_t off = 0;   // blocks of set si already done
  while (si < count) {
    ChainSegs cs{};
    int n = 0;
    while (si < count && cs.nseg < CH_MAXSEG && n < chunk) {
      const poetx_chain_set& t = sets[si];
      const int64_t left = t.nblocks - off;
      if (left <= 0) { ++si; off = 0; continue; }
      const int take = (int)std::min<int64_t>(left, chunk - n);
      cs.seg[cs.nseg] = ChainSeg{t.Q32 + off * (int64_t)bb, t.G + off * (int64_t)bb,
                                 t.dtheta + off * (int64_t)(b * (b - 1) / 2)};
      cs.start[cs.nseg] = n;
      ++cs.nseg;
      n += take;
      off += take;
      if (off >= t.nblocks) { ++si; off = 0; }
    }
    cs.start[cs.nseg] = n;
    if (n > 0) chain_bf16(cs, n, b, T, GS, (flags & POETX_ACCUMULATE_GRAD) ? 1 : 0, s);
  }
  return check_launch("chain rule");
}

int poetx_merge(const poetx_layer* layer, void* W0p, float* thR, float* thP, int32_t* sigma, int32_t* tau,
                uint64_t perm_seed, uint64_t merge_index, void* ws, size_t ws_bytes, void* stream) {
  int rc = validate_layer(layer);
  if (rc) return rc;
  const Shape S = shape_of(layer, 0);
  if (!W0p || !sigma || !tau) return fail(POETX_EINVAL, "NULL tensor argument");
  if ((S.kR > 0 && !thR) || (S.kP > 0 && !thP)) return fail(POETX_EINVAL, "NULL generator");
  size_t need = 0;
  plan_merge(S, true, nullptr, &need);
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  const MrgWs w = plan_merge(S, true, ws, &need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int bmode = S.f32 ? 0 : 6;
  if (S.f32) rc = build2(thR, S.kR, QOut{w.q32R, nullptr, nullptr}, thP, S.kP, QOut{w.q32P, nullptr, nullptr}, S.b,
                       w.bws, bmode, s);
  else rc = build2(thR, S.kR, QOut{nullptr, w.qbR, nullptr}, thP, S.kP, QOut{nullptr, nullptr, w.qtP}, S.b, w.bws,
                   bmode, s);
  if (rc) return rc;
  return merge_w0(S, W0p, Blk{w.q32R, w.q32P, w.qbR, nullptr, nullptr, w.qtP}, thR, thP, sigma, tau, perm_seed,
                    merge_index, w, s);
}

int poetx_merge_blocks(const poetx_layer* layer, void* W0p, const poetx_blocks* blocks, float* thR, float* thP,
                       int32_t* sigma, int32_t* tau, uint64_t perm_seed, uint64_t merge_index, void* ws,
                       size_t ws_bytes, void* stream) {
  int rc = validate_layer(layer);
  if (rc) return rc;
  const Shape S = shape_of(layer, 0);
  if (!W0p || !sigma || !tau) return fail(POETX_EINVAL, "NULL tensor argument");
  if ((S.kR > 0 && !thR) || (S.kP > 0 && !thP)) return fail(POETX_EINVAL, "NULL generator");
  if ((rc = check_merge_blocks(S, blocks))) return rc;
  size_t need = 0;
  plan_merge(S, false, nullptr, &need);
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  const MrgWs w = plan_merge(S, false, ws, &need);
  return merge_w0(S, W0p, blk_of(blocks), thR, thP, sigma, tau, perm_seed, merge_index, w,
                    static_cast<hipStream_t>(stream));
}

namespace {
// host checks of one merge set (as poetx_merge_blocks makes them) and its
// workspace bytes
int check_merge_set_(const poetx_merge_set& m, Shape* S, size_t* need) {
  int rc = validate_layer(m.layer);
  if (rc) return rc;
  *S = shape_of(m.layer, 0);
  if (!m.W0p || !m.sigma || !m.tau) return fail(POETX_EINVAL, "NULL tensor argument");
  if ((S->kR > 0 && !m.thR) || (S->kP > 0 && !m.thP)) return fail(POETX_EINVAL, "NULL generator");
  if ((rc = check_merge_blocks(*S, m.blocks))) return rc;
  plan_merge(*S, false, nullptr, need);
  *need = (*need + kAlign - 1) / kAlign * kAlign;
  return POETX_OK;
}
// the same, the error message naming the set
int check_merge_set(const poetx_merge_set& m, int32_t k, Shape* S, size_t* need) {
  const int rc = check_merge_set_(m, S, need);
  if (rc) {
    const std::string msg = g_err;
    fail(rc, "merge set %d: %s", (int)k, msg.c_str());
  }
  return rc;
}
}  // namespace

size_t poetx_merge_sets_workspace_bytes(const poetx_merge_set* sets, int32_t count) {
  if (count < 0 || (count > 0 && !sets)) {
    fail(POETX_EINVAL, "bad set list");
    return 0;
  }
  size_t tot = kAlign;
  for (int32_t k = 0; k < count; ++k) {
    Shape S;
    size_t need = 0;
    if (check_merge_set(sets[k], k, &S, &need)) return 0;
    tot += need;
  }
  return tot;
}

int poetx_merge_blocks_sets(const poetx_merge_set* sets, int32_t count, void* ws, size_t ws_bytes, void* stream) {
  if (count < 0 || (count > 0 && !sets)) return fail(POETX_EINVAL, "bad set list");
  if (count == 0) return POETX_OK;
  std::vector<Shape> S(count);
  std::vector<size_t> off(count + 1, 0);
  int rc;
  for (int32_t k = 0; k < count; ++k) {
    size_t need = 0;
    if ((rc = check_merge_set(sets[k], k, &S[k], &need))) return rc;
    off[k + 1] = off[k] + need;
  }
  if ((rc = check_ws(ws, ws_bytes, off[count] + kAlign))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  std::vector<MrgWs> w(count);
  std::vector<int> batched;
  for (int32_t k = 0; k < count; ++k) {
    size_t b = 0;
    w[k] = plan_merge(S[k], false, base + off[k], &b);
    const poetx_merge_set& m = sets[k];
    const Blk q = blk_of(m.blocks);
    if (S[k].q8 || S[k].f32 || !walk_staged_ok(S[k].n, kRelayoutL, m.W0p, w[k].saved, w[k].tnew)) {
      // merged alone (dequantized copy, fp32 or unaligned rows)
      if ((rc = merge_w0(S[k], m.W0p, q, m.thR, m.thP, m.sigma, m.tau, m.perm_seed, m.merge_index, w[k], s)))
        return rc;
      continue;
    }
    if ((rc = merge_products(S[k], m.W0p, q, s))) return rc;
    batched.push_back(k);
  }
  for (size_t c0 = 0; c0 < batched.size(); c0 += MERGE_BATCH) {
    MergeBatch b{};
    b.count = (int)std::min(batched.size() - c0, (size_t)MERGE_BATCH);
    double bytes = 0.0;
    for (int i = 0; i < b.count; ++i) {
      const int k = batched[c0 + i];
      const poetx_merge_set& m = sets[k];
      const MrgWs& x = w[k];
      MergeItem& it = b.it[i];
      it.W = m.W0p; it.saved = x.saved;
      it.sigma = m.sigma; it.tau = m.tau; it.snew = x.snew; it.tnew = x.tnew; it.sinv = x.sinv; it.tinv = x.tinv;
      it.dist = x.dist; it.hlist = x.hlist; it.slot = x.slot; it.slist = x.slist; it.counts = x.counts;
      it.nxt = x.nxt;
      it.thR = m.thR; it.thP = m.thP;
      it.nthR = (int64_t)S[k].kR * (S[k].b * (S[k].b - 1) / 2);
      it.nthP = (int64_t)S[k].kP * (S[k].b * (S[k].b - 1) / 2);
      it.m = S[k].m; it.n = S[k].n; it.max_saved = x.max_saved;
      it.seed = m.perm_seed; it.merge_index = m.merge_index;
      bytes += 2.0 * S[k].m * S[k].n * S[k].es;
    }
    {
      Tm tm(s, "merge_permutations", 0.0, 0.0);
      launch_merge_permutations_batch(b, s);
    }
    {
      Tm tm(s, "merge_relayout", 0.0, bytes);
      launch_cycle_plans_batch(b, kRelayoutL, s);
      launch_relayout_staged_batch(b, kRelayoutL, s);
    }
    launch_zero_generators_batch(b, s);
    if ((rc = check_launch("batched merge"))) return rc;
    for (int i = 0; i < b.count; ++i)
      if ((rc = refresh_transpose(S[batched[c0 + i]], sets[batched[c0 + i]].W0p, s))) return rc;
  }
  return POETX_OK;
}

size_t poetx_w0_bytes(const poetx_layer* layer) {
  if (validate_layer(layer) != POETX_OK) return 0;
  const Shape S = shape_of(layer, 0);
  if (S.q8) return w0_scale_offset(S.m, S.n) + (size_t)S.m * sizeof(float);
  if (S.tr) return w0t_offset(S.m, S.n) + (size_t)S.m * S.n * 2;
  return (size_t)S.m * S.n * S.es;
}

int poetx_transpose_w0(const poetx_layer* layer, void* W0p, void* stream) {
  int rc = validate_layer(layer);
  if (rc) return rc;
  const Shape S = shape_of(layer, 0);
  if (!S.tr) return fail(POETX_EINVAL, "layer.flags lacks POETX_W0_TRANSPOSED");
  if (!W0p) return fail(POETX_EINVAL, "NULL tensor argument");
  return refresh_transpose(S, W0p, static_cast<hipStream_t>(stream));
}

int poetx_quantize_w0(const poetx_layer* layer, const void* W0bf16, void* W0q, void* stream) {
  int rc = validate_layer(layer);
  if (rc) return rc;
  const Shape S = shape_of(layer, 0);
  if (!S.q8) return fail(POETX_EINVAL, "layer.flags lacks POETX_W0_INT8");
  if (!W0bf16 || !W0q) return fail(POETX_EINVAL, "NULL tensor argument");
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch_quantize_rows(static_cast<const uint16_t*>(W0bf16), static_cast<int8_t*>(W0q),
                       reinterpret_cast<float*>(static_cast<char*>(W0q) + w0_scale_offset(S.m, S.n)), S.m, S.n, s);
  return check_launch("weight quantization");
}

int poetx_dequantize_w0(const poetx_layer* layer, const void* W0q, void* W0bf16, void* stream) {
  int rc = validate_layer(layer);
  if (rc) return rc;
  const Shape S = shape_of(layer, 0);
  if (!S.q8) return fail(POETX_EINVAL, "layer.flags lacks POETX_W0_INT8");
  if (!W0bf16 || !W0q) return fail(POETX_EINVAL, "NULL tensor argument");
  weight_for_pass(S, W0q, W0bf16, static_cast<hipStream_t>(stream));
  return check_launch("weight dequantization");
}

int poetx_make_permutation(uint64_t seed, uint64_t merge_index, int32_t side, int64_t n, int32_t* host_out) {
  if (side != 0 && side != 1) return fail(POETX_EINVAL, "side must be 0 or 1");
  if (n < 0 || n > (int64_t(1) << 30)) return fail(POETX_ESHAPE, "n=%lld", (long long)n);
  if (n > 0 && !host_out) return fail(POETX_EINVAL, "host_out is NULL");
  const uint64_t g = 0x9E3779B97F4A7C15ull;
  const uint64_t base = mix64(seed + g * (2 * merge_index + (uint64_t)side + 1));
  std::vector<std::pair<uint64_t, int64_t>> kv((size_t)n);
  for (int64_t i = 0; i < n; ++i) kv[(size_t)i] = {mix64(base + g * (uint64_t)(i + 1)), i};
  std::sort(kv.begin(), kv.end());
  for (int64_t i = 0; i < n; ++i) host_out[i] = (int32_t)kv[(size_t)i].second;
  return POETX_OK;
}

int poetx_adam_step(float* theta, const float* grad, float* m, float* v, int64_t count, int64_t step, float lr,
                    float beta1, float beta2, float eps, void* stream) {
  if (count < 0) return fail(POETX_ESHAPE, "count=%lld", (long long)count);
  if (step < 1) return fail(POETX_EINVAL, "step must be >= 1");
  if (count == 0) return POETX_OK;
  if (!theta || !grad || !m || !v) return fail(POETX_EINVAL, "NULL tensor argument");
  const double bc1 = 1.0 - std::pow((double)beta1, (double)step);
  const double bc2 = 1.0 - std::pow((double)beta2, (double)step);
  {
    Tm tm(static_cast<hipStream_t>(stream), "adam", 0.0, 7.0 * 4.0 * count);
    launch_adam(theta, grad, m, v, count, lr, beta1, beta2, eps, (float)bc1, (float)bc2,
                static_cast<hipStream_t>(stream));
  }
  return check_launch("adam");
}

int poetx_timing_enable(int on) {
  clear_timing();
  g_timing = on != 0;
  return POETX_OK;
}

int poetx_timing_summary(char* buf, size_t len) {
  if (!buf || len == 0) return fail(POETX_EINVAL, "NULL buffer");
  struct Agg { std::string name; int n; double ms, flops, bytes; };
  std::vector<Agg> agg;
  for (auto& r : g_recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return fail(POETX_EHIP, "event synchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return fail(POETX_EHIP, "event elapsed time failed");
    auto it = std::find_if(agg.begin(), agg.end(), [&](const Agg& a) { return a.name == r.name; });
    if (it == agg.end()) { agg.push_back({r.name, 0, 0, 0, 0}); it = agg.end() - 1; }
    it->n += 1; it->ms += ms; it->flops += r.flops; it->bytes += r.bytes;
  }
  std::string out;
  char line[256];
  for (auto& a : agg) {
    snprintf(line, sizeof line, "%s %d %.6f %.6e %.6e\n", a.name.c_str(), a.n, a.ms, a.flops, a.bytes);
    out += line;
  }
  if (out.size() + 1 > len) return fail(POETX_EINVAL, "buffer too small (%zu bytes needed)", out.size() + 1);
  memcpy(buf, out.c_str(), out.size() + 1);
  return (int)agg.size();
}

}  // extern "C"
