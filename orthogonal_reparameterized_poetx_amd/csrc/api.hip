// C ABI of the POET-X layer hot path: validation, workspace planning and the
// launch sequences of forward, backward, merge and the Cayley builder.
// See include/poetx.h for the contract of every entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
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

bool valid_b(int32_t b) { return b == 32 || b == 64 || b == 128 || b == 256 || b == 512; }

int validate_layer(const poetx_layer* L) {
  if (!L) return fail(POETX_EINVAL, "layer is NULL");
  if (L->reserved != 0) return fail(POETX_EINVAL, "layer.reserved must be 0");
  if (L->dtype != POETX_F32 && L->dtype != POETX_BF16) return fail(POETX_EDTYPE, "unsupported dtype %d", L->dtype);
  if (!valid_b(L->b)) return fail(POETX_EINVAL, "block size b=%d not in {32,64,128,256,512}", L->b);
  if (L->m < 1 || L->m > kMaxDim || L->n < 1 || L->n > kMaxDim)
    return fail(POETX_ESHAPE, "m=%lld n=%lld out of range [1, %lld]", (long long)L->m, (long long)L->n,
                (long long)kMaxDim);
  if (L->flags & ~POETX_ACCUMULATE_GRAD) return fail(POETX_EINVAL, "unknown flags 0x%x", L->flags);
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

// Cayley blocks.  mode 6: split-bf16 x6 MFMA products (fp32-level accuracy);
// mode 0: fp32 MFMA.  Both give Q accurate to fp32 rounding, so rounding Q to
// bf16 agrees with rounding the exact Q except in rare ties at the boundary.
int build(const float* theta, int64_t nblk, int b, float* q32, uint16_t* qbf, uint16_t* qtbf, void* ws, int mode,
          hipStream_t s) {
  if (nblk <= 0) return POETX_OK;
  Tm tm(s, "cayley_build", 2.0 * b * (double)b * b * nblk, 0.0);
  if (b <= 256) {
    GJArgs g{};
    g.theta = theta;
    g.q32 = q32;
    g.qbf = qbf;
    g.qtbf = qtbf;
    launch_gj(b, mode, (int)nblk, g, s);
    return check_launch("cayley builder");
  }
  // b = 512: 2x2 block inverse with 256-wide Schur complement.
  //   [A B; C D]^-1 = [Ai + Ai B Si C Ai, -Ai B Si; -Si C Ai, Si], Si = (D - C Ai B)^-1
  Arena a(ws);
  float* Af = a.take<float>((size_t)nblk * 512 * 512);
  float* Mf = a.take<float>((size_t)nblk * 512 * 512);
  float* Tm = a.take<float>((size_t)nblk * 256 * 256);
  float* Vm = a.take<float>((size_t)nblk * 256 * 256);
  const int64_t SB = 512 * 512, SH = 256 * 256;
  launch_unpack_eye_minus_s(theta, 512, (int)nblk, Af, s);
  GJArgs g{};
  g.in = Af; g.in_stride = SB; g.in_ld = 512;
  g.out = Mf; g.out_stride = SB; g.out_ld = 512;      // A^-1 into M11
  launch_gj(256, mode, (int)nblk, g, s);
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
  gemm(M11, 512, A12, 512, Tm, 256, 1.f, 0.f, SB, SB, SH);        // T = Ai B
  gemm(A21, 512, Tm, 256, A22, 512, -1.f, 1.f, SB, SH, SB);       // Sc = D - C T
  GJArgs g2{};
  g2.in = A22; g2.in_stride = SB; g2.in_ld = 512;
  g2.out = M22; g2.out_stride = SB; g2.out_ld = 512;               // Si
  launch_gj(256, mode, (int)nblk, g2, s);
  gemm(A21, 512, M11, 512, Vm, 256, 1.f, 0.f, SB, SB, SH);        // V = C Ai
  gemm(Tm, 256, M22, 512, M12, 512, -1.f, 0.f, SH, SB, SB);       // M12 = -T Si
  gemm(M22, 512, Vm, 256, M21, 512, -1.f, 0.f, SB, SH, SB);       // M21 = -Si V
  gemm(M12, 512, Vm, 256, M11, 512, -1.f, 1.f, SB, SH, SB);       // M11 = Ai - M12 V
  launch_finalize_q(Mf, 512, (int)nblk, q32, qbf, qtbf, s);
  return check_launch("cayley builder (b=512)");
}

// dtheta from G = dL/dQ:  G_S = 1/2 (I + Q^T) G (I + Q^T);  dtheta_p = G_S[i][j] - G_S[j][i]
int chain(float* G, const float* q32, float* tmp, int64_t nblk, int b, float* dth, bool accumulate, int mode,
          hipStream_t s) {
  if (nblk <= 0) return POETX_OK;
  Tm tm(s, "chain_rule", 4.0 * b * (double)b * b * nblk, 0.0);
  const int64_t sb = (int64_t)b * b;
  BGemmArgs q{};
  q.M = q.N = q.K = b;
  q.A = G; q.sA = sb; q.lda = b;
  q.B = q32; q.sB = sb; q.ldb = b; q.transB = 1; q.addIB = 1;
  q.C = tmp; q.sC = sb; q.ldc = b;
  q.alpha = 1.f; q.beta = 0.f;
  launch_bgemm(mode, (int)nblk, q, s);
  BGemmArgs r{};
  r.M = r.N = r.K = b;
  r.A = q32; r.sA = sb; r.lda = b; r.transA = 1; r.addIA = 1;
  r.B = tmp; r.sB = sb; r.ldb = b;
  r.C = G; r.sC = sb; r.ldc = b;
  r.alpha = 0.5f; r.beta = 0.f;
  launch_bgemm(mode, (int)nblk, r, s);
  launch_skew_project(G, b, (int)nblk, dth, accumulate ? 1 : 0, s);
  return check_launch("chain rule");
}

// block-product flops of one transform: N tokens x k blocks x 2 b^2
double xf_flops(int64_t N, int k, int b) { return 2.0 * N * k * (double)b * b; }

struct Shape {
  int64_t m, n, N;
  int b, kR, kP;
  bool f32;
  size_t es;  // element size of activations / weight
};

Shape shape_of(const poetx_layer* L, int64_t N) {
  Shape S;
  S.m = L->m; S.n = L->n; S.N = N; S.b = L->b;
  S.kR = (int)(L->m / L->b);
  S.kP = (int)(L->n / L->b);
  S.f32 = L->dtype == POETX_F32;
  S.es = S.f32 ? 4 : 2;
  return S;
}

// ---- workspace plans (same code sizes and carves)
struct FwdWs {
  float *q32R, *q32P;
  uint16_t *qbR, *qbP;
  void* bws;
  void *z1, *z2;
};
FwdWs plan_fwd(const Shape& S, void* base, size_t* bytes) {
  Arena a(base);
  FwdWs w{};
  if (S.f32) {
    w.q32R = a.take<float>((size_t)S.kR * S.b * S.b);
    w.q32P = a.take<float>((size_t)S.kP * S.b * S.b);
  } else {
    w.qbR = a.take<uint16_t>((size_t)S.kR * S.b * S.b);
    w.qbP = a.take<uint16_t>((size_t)S.kP * S.b * S.b);
  }
  w.bws = a.take<char>(build_ws_bytes(std::max(S.kR, S.kP), S.b));
  w.z1 = a.take<char>((size_t)S.N * S.n * S.es);
  w.z2 = a.take<char>((size_t)S.N * S.m * S.es);
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
};
BwdWs plan_bwd(const Shape& S, void* base, size_t* bytes) {
  Arena a(base);
  BwdWs w{};
  const size_t bb = (size_t)S.b * S.b;
  w.q32R = a.take<float>(S.kR * bb);
  w.q32P = a.take<float>(S.kP * bb);
  if (!S.f32) {
    w.qbP = a.take<uint16_t>(S.kP * bb);
    w.qtR = a.take<uint16_t>(S.kR * bb);
    w.qtP = a.take<uint16_t>(S.kP * bb);
  }
  w.bws = a.take<char>(build_ws_bytes(std::max(S.kR, S.kP), S.b));
  w.z1 = a.take<char>((size_t)S.N * S.n * S.es);
  w.xg = a.take<char>((size_t)S.N * S.n * S.es);
  w.z2 = a.take<char>((size_t)S.N * S.m * S.es);
  w.gyg = a.take<char>((size_t)S.N * S.m * S.es);
  w.gz2 = a.take<char>((size_t)S.N * S.m * S.es);
  w.GR = a.take<float>(S.kR * bb);
  w.GP = a.take<float>(S.kP * bb);
  w.tmp = a.take<float>(std::max(S.kR, S.kP) * bb);
  const size_t pb = std::max(gram_partials_bytes(S.N, S.b, S.kR, S.f32), gram_partials_bytes(S.N, S.b, S.kP, S.f32));
  w.part = a.take<char>(pb);
  *bytes = a.off + kAlign;
  return w;
}

struct MrgWs {
  float *q32R, *q32P;
  uint16_t *qbR, *qtP;
  void* bws;
  void* V;
  uint64_t* keys;
  int32_t *snew, *tnew, *sinv, *tinv;
};
MrgWs plan_merge(const Shape& S, void* base, size_t* bytes) {
  Arena a(base);
  MrgWs w{};
  const size_t bb = (size_t)S.b * S.b;
  if (S.f32) {
    w.q32R = a.take<float>(S.kR * bb);
    w.q32P = a.take<float>(S.kP * bb);
  } else {
    w.qbR = a.take<uint16_t>(S.kR * bb);
    w.qtP = a.take<uint16_t>(S.kP * bb);
  }
  w.bws = a.take<char>(build_ws_bytes(std::max(S.kR, S.kP), S.b));
  w.V = a.take<char>((size_t)S.m * S.n * S.es * (S.f32 ? 2 : 1));
  w.keys = a.take<uint64_t>(std::max(S.m, S.n));
  w.snew = a.take<int32_t>(S.m);
  w.tnew = a.take<int32_t>(S.n);
  w.sinv = a.take<int32_t>(S.m);
  w.tinv = a.take<int32_t>(S.n);
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
  if (op != POETX_OP_MERGE && validate_N(N) != POETX_OK) return 0;
  const Shape S = shape_of(layer, op == POETX_OP_MERGE ? 0 : N);
  size_t bytes = 0;
  switch (op) {
    case POETX_OP_FORWARD: plan_fwd(S, nullptr, &bytes); break;
    case POETX_OP_BACKWARD: plan_bwd(S, nullptr, &bytes); break;
    case POETX_OP_MERGE: plan_merge(S, nullptr, &bytes); break;
    default: fail(POETX_EINVAL, "unknown op %d", op); return 0;
  }
  return bytes;
}

int poetx_build_blocks(const float* theta, int64_t nblocks, int32_t b, float* Q32, void* Qbf16, void* QTbf16,
                       void* ws, size_t ws_bytes, void* stream) {
  if (!valid_b(b)) return fail(POETX_EINVAL, "block size b=%d not in {32,64,128,256,512}", b);
  if (nblocks < 0 || nblocks > (int64_t(1) << 20)) return fail(POETX_ESHAPE, "nblocks=%lld", (long long)nblocks);
  if (nblocks == 0) return POETX_OK;
  if (!theta) return fail(POETX_EINVAL, "theta is NULL");
  if (!Q32 && !Qbf16 && !QTbf16) return fail(POETX_EINVAL, "no output requested");
  const int rc = check_ws(ws, ws_bytes, build_ws_bytes(nblocks, b));
  if (rc) return rc;
  return build(theta, nblocks, b, Q32, static_cast<uint16_t*>(Qbf16), static_cast<uint16_t*>(QTbf16), ws, 6,
               static_cast<hipStream_t>(stream));
}

int poetx_forward(const poetx_layer* layer, const void* W0p, const float* thR, const float* thP,
                  const int32_t* sigma, const int32_t* tau, const void* X, int64_t N, void* Y, void* ws,
                  size_t ws_bytes, void* stream) {
  int rc = validate_layer(layer);
  if (rc) return rc;
  if ((rc = validate_N(N))) return rc;
  if (N == 0) return POETX_OK;
  const Shape S = shape_of(layer, N);
  if (!W0p || !sigma || !tau || !X || !Y) return fail(POETX_EINVAL, "NULL tensor argument");
  if ((S.kR > 0 && !thR) || (S.kP > 0 && !thP)) return fail(POETX_EINVAL, "NULL generator");
  size_t need = 0;
  plan_fwd(S, nullptr, &need);
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  FwdWs w = plan_fwd(S, ws, &need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int bmode = S.f32 ? 0 : 6;
  // Cayley blocks (recomputed every call; nothing is cached between calls)
  if (S.f32) {
    if ((rc = build(thR, S.kR, S.b, w.q32R, nullptr, nullptr, w.bws, bmode, s))) return rc;
    if ((rc = build(thP, S.kP, S.b, w.q32P, nullptr, nullptr, w.bws, bmode, s))) return rc;
  } else {
    if ((rc = build(thR, S.kR, S.b, nullptr, w.qbR, nullptr, w.bws, bmode, s))) return rc;
    if ((rc = build(thP, S.kP, S.b, nullptr, w.qbP, nullptr, w.bws, bmode, s))) return rc;
  }
  // z1' = D_P (Pi_tau x): gather by tau, multiply by Q_P^T per block
  XformArgs p{};
  p.in = X; p.out = w.z1; p.emit = nullptr; p.perm = tau; p.N = N; p.W = (int)S.n; p.B = S.b; p.k = S.kP;
  {
    Tm tm(s, "xform_gather_in", xf_flops(N, S.kP, S.b), 2.0 * N * S.n * S.es);
    if (S.f32) { p.bq = w.q32P; p.trans = 0; launch_gather_in_f32(p, s); }
    else { p.bq = w.qbP; if (!launch_gather_in_bf16(p, s)) return fail(POETX_ESHAPE, "no transform config for n=%lld b=%d", (long long)S.n, S.b); }
  }
  if ((rc = check_launch("P-side transform"))) return rc;
  // z2' = z1' W0p^T
  {
    Tm tm(s, "gemm_nt", 2.0 * N * S.m * S.n, (double)(N * S.n + S.m * S.n + N * S.m) * S.es);
    if (S.f32) launch_gemm_f32(false, (const float*)w.z1, (const float*)W0p, (float*)w.z2, N, S.m, S.n, s);
    else launch_gemm_bf16(false, (const uint16_t*)w.z1, (const uint16_t*)W0p, (uint16_t*)w.z2, N, S.m, S.n, s);
  }
  if ((rc = check_launch("forward GEMM"))) return rc;
  // y = Pi_sigma^T (D_R z2'): multiply by Q_R^T per block, scatter by sigma
  XformArgs r{};
  r.in = w.z2; r.out = Y; r.perm = sigma; r.N = N; r.W = (int)S.m; r.B = S.b; r.k = S.kR;
  {
    Tm tm(s, "xform_scatter_out", xf_flops(N, S.kR, S.b), 2.0 * N * S.m * S.es);
    if (S.f32) { r.bq = w.q32R; r.trans = 0; launch_scatter_out_f32(r, s); }
    else { r.bq = w.qbR; if (!launch_scatter_out_bf16(r, s)) return fail(POETX_ESHAPE, "no transform config for m=%lld b=%d", (long long)S.m, S.b); }
  }
  return check_launch("R-side transform");
}

int poetx_backward(const poetx_layer* layer, const void* W0p, const float* thR, const float* thP,
                   const int32_t* sigma, const int32_t* tau, const void* X, const void* dY, int64_t N, void* dX,
                   float* dthR, float* dthP, void* ws, size_t ws_bytes, void* stream) {
  int rc = validate_layer(layer);
  if (rc) return rc;
  if ((rc = validate_N(N))) return rc;
  const Shape S = shape_of(layer, N);
  if (N > 0 && (!W0p || !sigma || !tau || !X || !dY)) return fail(POETX_EINVAL, "NULL tensor argument");
  if ((S.kR > 0 && (!thR || !dthR)) || (S.kP > 0 && (!thP || !dthP)))
    return fail(POETX_EINVAL, "NULL generator or generator gradient");
  const bool accum = (layer->flags & POETX_ACCUMULATE_GRAD) != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t ntR = (int64_t)S.kR * (S.b * (S.b - 1) / 2), ntP = (int64_t)S.kP * (S.b * (S.b - 1) / 2);
  if (N == 0) {
    if (!accum) {
      launch_fill_f32(dthR, 0.f, ntR, s);
      launch_fill_f32(dthP, 0.f, ntP, s);
    }
    return check_launch("zero gradients");
  }
  size_t need = 0;
  plan_bwd(S, nullptr, &need);
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  BwdWs w = plan_bwd(S, ws, &need);
  const int bmode = S.f32 ? 0 : 6;   // Cayley builder
  const int cmode = S.f32 ? 0 : 3;   // chain-rule products
  // recompute the blocks (not stored between forward and backward)
  if (S.f32) {
    if ((rc = build(thR, S.kR, S.b, w.q32R, nullptr, nullptr, w.bws, bmode, s))) return rc;
    if ((rc = build(thP, S.kP, S.b, w.q32P, nullptr, nullptr, w.bws, bmode, s))) return rc;
  } else {
    if ((rc = build(thR, S.kR, S.b, w.q32R, nullptr, w.qtR, w.bws, bmode, s))) return rc;
    if ((rc = build(thP, S.kP, S.b, w.q32P, w.qbP, w.qtP, w.bws, bmode, s))) return rc;
  }
  // recompute z1' (and keep the gathered x' for dL/dQ_P), then z2'
  XformArgs p{};
  p.in = X; p.out = w.z1; p.emit = w.xg; p.perm = tau; p.N = N; p.W = (int)S.n; p.B = S.b; p.k = S.kP;
  {
    // recompute pass: algorithmic bytes are the read of X and the write of z1'
    Tm tm(s, "xform_gather_in", xf_flops(N, S.kP, S.b), 2.0 * N * S.n * S.es);
    if (S.f32) { p.bq = w.q32P; p.trans = 0; launch_gather_in_f32(p, s); }
    else { p.bq = w.qbP; if (!launch_gather_in_bf16(p, s)) return fail(POETX_ESHAPE, "no transform config for n=%lld", (long long)S.n); }
  }
  {
    Tm tm(s, "gemm_nt", 2.0 * N * S.m * S.n, (double)(N * S.n + S.m * S.n + N * S.m) * S.es);
    if (S.f32) launch_gemm_f32(false, (const float*)w.z1, (const float*)W0p, (float*)w.z2, N, S.m, S.n, s);
    else launch_gemm_bf16(false, (const uint16_t*)w.z1, (const uint16_t*)W0p, (uint16_t*)w.z2, N, S.m, S.n, s);
  }
  if ((rc = check_launch("recompute"))) return rc;
  // R side: gY' = Pi_sigma gY (kept), gz2' = D_R^T gY' (blocks Q_R), G_R = gY'^T z2'
  XformArgs r{};
  r.in = dY; r.out = w.gz2; r.emit = w.gyg; r.perm = sigma; r.N = N; r.W = (int)S.m; r.B = S.b; r.k = S.kR;
  {
    // algorithmic bytes: read gY, write gz2' (the gathered copy is implementation traffic)
    Tm tm(s, "xform_gather_in", xf_flops(N, S.kR, S.b), 2.0 * N * S.m * S.es);
    if (S.f32) { r.bq = w.q32R; r.trans = 1; launch_gather_in_f32(r, s); }
    else { r.bq = w.qtR; if (!launch_gather_in_bf16(r, s)) return fail(POETX_ESHAPE, "no transform config for m=%lld", (long long)S.m); }
  }
  {
    // algorithmic bytes: the read of z2' (gY is counted with the transform)
    Tm tm(s, "gram", xf_flops(N, S.kR, S.b), 1.0 * N * S.m * S.es);
    launch_gram(S.f32, w.gyg, w.z2, N, (int)S.m, S.b, S.kR, w.GR, w.part, s);
  }
  if ((rc = check_launch("R-side backward"))) return rc;
  // gz1' = gz2' W0p (into the z1' buffer)
  void* gz1 = w.z1;
  {
    Tm tm(s, "gemm_nn", 2.0 * N * S.m * S.n, (double)(N * S.n + S.m * S.n + N * S.m) * S.es);
    if (S.f32) launch_gemm_f32(true, (const float*)w.gz2, (const float*)W0p, (float*)gz1, N, S.n, S.m, s);
    else launch_gemm_bf16(true, (const uint16_t*)w.gz2, (const uint16_t*)W0p, (uint16_t*)gz1, N, S.n, S.m, s);
  }
  // P side: G_P = gz1'^T x', dX = Pi_tau^T D_P^T gz1'
  {
    // algorithmic bytes: the read of x (gz1' is counted with the dX transform)
    Tm tm(s, "gram", xf_flops(N, S.kP, S.b), 1.0 * N * S.n * S.es);
    launch_gram(S.f32, gz1, w.xg, N, (int)S.n, S.b, S.kP, w.GP, w.part, s);
  }
  if (dX) {
    XformArgs q{};
    q.in = gz1; q.out = dX; q.perm = tau; q.N = N; q.W = (int)S.n; q.B = S.b; q.k = S.kP;
    Tm tm(s, "xform_scatter_out", xf_flops(N, S.kP, S.b), 2.0 * N * S.n * S.es);
    if (S.f32) { q.bq = w.q32P; q.trans = 1; launch_scatter_out_f32(q, s); }
    else { q.bq = w.qtP; if (!launch_scatter_out_bf16(q, s)) return fail(POETX_ESHAPE, "no transform config for n=%lld", (long long)S.n); }
  }
  if ((rc = check_launch("P-side backward"))) return rc;
  // chain rule through the Cayley map onto the stored upper triangle
  if ((rc = chain(w.GR, w.q32R, w.tmp, S.kR, S.b, dthR, accum, cmode, s))) return rc;
  if ((rc = chain(w.GP, w.q32P, w.tmp, S.kP, S.b, dthP, accum, cmode, s))) return rc;
  return POETX_OK;
}

int poetx_merge(const poetx_layer* layer, void* W0p, float* thR, float* thP, int32_t* sigma, int32_t* tau,
                uint64_t perm_seed, uint64_t merge_index, void* ws, size_t ws_bytes, void* stream) {
  int rc = validate_layer(layer);
  if (rc) return rc;
  const Shape S = shape_of(layer, 0);
  if (!W0p || !sigma || !tau) return fail(POETX_EINVAL, "NULL tensor argument");
  if ((S.kR > 0 && !thR) || (S.kP > 0 && !thP)) return fail(POETX_EINVAL, "NULL generator");
  size_t need = 0;
  plan_merge(S, nullptr, &need);
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  MrgWs w = plan_merge(S, ws, &need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int bmode = S.f32 ? 0 : 6;
  if (S.f32) {
    if ((rc = build(thR, S.kR, S.b, w.q32R, nullptr, nullptr, w.bws, bmode, s))) return rc;
    if ((rc = build(thP, S.kP, S.b, w.q32P, nullptr, nullptr, w.bws, bmode, s))) return rc;
    launch_merge_tiles(true, W0p, w.V, w.q32R, w.q32P, S.m, S.n, S.b, S.kR, S.kP, s);
  } else {
    if ((rc = build(thR, S.kR, S.b, nullptr, w.qbR, nullptr, w.bws, bmode, s))) return rc;
    if ((rc = build(thP, S.kP, S.b, nullptr, nullptr, w.qtP, w.bws, bmode, s))) return rc;
    Tm tm(s, "merge_tiles", 4.0 * S.m * S.n * S.b, 2.0 * S.m * S.n * S.es);
    launch_merge_tiles(false, W0p, w.V, w.qbR, w.qtP, S.m, S.n, S.b, S.kR, S.kP, s);
  }
  if ((rc = check_launch("merge tiles"))) return rc;
  // new permutations, old inverses, relayout into the caller's buffer
  launch_perm_keys_rank(perm_seed, merge_index, 0, S.m, w.keys, w.snew, s);
  launch_perm_keys_rank(perm_seed, merge_index, 1, S.n, w.keys, w.tnew, s);
  launch_invert_perm(sigma, S.m, w.sinv, s);
  launch_invert_perm(tau, S.n, w.tinv, s);
  {
    Tm tm(s, "merge_relayout", 0.0, 2.0 * S.m * S.n * S.es);
    launch_relayout(S.f32, w.V, W0p, w.sinv, w.snew, w.tinv, w.tnew, S.m, S.n, s);
  }
  launch_copy_i32(w.snew, sigma, S.m, s);
  launch_copy_i32(w.tnew, tau, S.n, s);
  launch_fill_f32(thR, 0.f, (int64_t)S.kR * (S.b * (S.b - 1) / 2), s);
  launch_fill_f32(thP, 0.f, (int64_t)S.kP * (S.b * (S.b - 1) / 2), s);
  return check_launch("merge relayout");
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
