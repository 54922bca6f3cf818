// Per-block gradient with respect to the orthogonal blocks:
//   G[l][i][j] = sum_t A[t][l*B + i] * C[t][l*B + j]
// e.g. dL/dQ_R,l = gY'_l^T z2'_l and dL/dQ_P,l = gz1'_l^T x'_l, both in the
// working (permuted) layout so every operand row is contiguous.  This is the
// token reduction that automatic differentiation would perform before the
// Cayley chain rule [P1 "POET-X：基于正交变换缩放的内存高效LLM训练方法", 实践 2 step 3].
//
// bf16 path: the reduction index (tokens) is the MFMA K dimension; token-major
// tiles are staged in LDS as loaded and read K-major with the gfx950
// transposing LDS load.  Workgroups own a (TI x TI) tile of one block and a
// chunk of tokens; per-chunk fp32 partials are summed in a fixed order by a
// second kernel, so the result is deterministic.
#include "common.h"
#include "kernels.h"
#include "ranges.h"

namespace poetx {

__device__ __forceinline__ i16x4 ds_read_tr16g(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, const_cast<uint16_t*>(p)));
}

static int gram_tile(int B) { return B < 128 ? B : 128; }

// token chunks per launch: about 512 workgroups in all.  More chunks fill
// the chip faster but every chunk writes a full fp32 partial of the blocks,
// which the reduction reads back (at 32 chunks the partials outweigh the
// bf16 operands); measured on the 2048- and 5632-wide layer-set shapes.
static int gram_chunks(int64_t N, int B, int k) {
  const int ti = gram_tile(B);
  const int64_t tiles = (int64_t)k * (B / ti) * (B / ti);
  int64_t s = (512 + tiles - 1) / (tiles > 0 ? tiles : 1);
  const int64_t maxs = (N + 255) / 256;
  if (s > maxs) s = maxs;
  if (s < 1) s = 1;
  return (int)s;
}

constexpr int GR_S = 7;      // ring stages
constexpr int GR_T = 32;     // tokens per tile
constexpr int GR_TI = 128;   // quadrant side
constexpr int GR_E = GR_T * GR_TI;   // elements of one operand tile

__device__ __forceinline__ void gr_b2l16(__amdgpu_buffer_rsrc_t r, int voff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gr_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr unsigned gr_vm_imm(unsigned vm) { return (vm & 15u) | ((vm >> 4) << 14) | (7u << 4) | (15u << 8); }

// run plan shared by the launcher and the workspace query
static_assert(GR_T == GRAM_T && GR_TI == GRAM_TI && GR_S == GRAM_STAGES, "ranges.h mirrors the tiling");
static bool gram_stream_ok(int64_t N, int W, int B, const void* A, const void* C) {
  if (B != 128 && B != 256) return false;
  if ((W & 7) || (reinterpret_cast<uintptr_t>(A) & 15) || (reinterpret_cast<uintptr_t>(C) & 15)) return false;
  // 32-bit buffer offsets: a run plus the ring's overshoot
  const int64_t ntiles = (N + GR_T - 1) / GR_T;
  return (ntiles + GR_S) * GR_T * (int64_t)W * 2 < 0x7fffffffLL;
}

size_t gram_partials_bytes(int64_t N, int B, int k, bool f32) {
  if (f32 || k <= 0 || N <= 0) return 0;
  int s = gram_chunks(N, B, k);
  if (B == 128 || B == 256) {
    // the streaming kernel's runs (it is used when the operands allow)
    const int r = gram_stream_runs(N, B, k).runs;
    if (r > s) s = r;
  }
  if (s == 1) return 0;
  return (size_t)s * k * B * B * sizeof(float);
}

// TI x TI output tile per workgroup, 4 waves; WTT = MFMA 32x32 tiles per wave side.
template <int TI, int WTT>
__global__ __launch_bounds__(256) void gram_bf16_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ C,
                                                        int64_t N, int W, int B, int k, int chunks, int64_t chunk_len,
                                                        float* __restrict__ out) {
  constexpr int TK = 32;                 // tokens per LDS sub-chunk
  constexpr int RC = TI / 8;             // 16-byte chunks per staged row
  __shared__ __align__(16) uint16_t sa[2][TK * TI];
  __shared__ __align__(16) uint16_t sc[2][TK * TI];
  const int tpb = B / TI;
  int bid = blockIdx.x;
  const int chunk = bid % chunks; bid /= chunks;
  const int tj = bid % tpb; bid /= tpb;
  const int ti = bid % tpb; bid /= tpb;
  const int l = bid;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col_a = l * B + ti * TI, col_c = l * B + tj * TI;
  const int64_t tbeg = (int64_t)chunk * chunk_len;
  int64_t tend = tbeg + chunk_len;
  if (tend > N) tend = N;
  const bool vec = (W & 7) == 0;
  // wave sub-tile
  const int wi = (TI == 32) ? 0 : (wave >> 1), wj = (TI == 32) ? 0 : (wave & 1);
  const bool active = (TI == 32) ? (wave == 0) : true;
  constexpr int WS = 32 * WTT;  // wave tile side

  f32x16 acc[WTT][WTT];
#pragma unroll
  for (int a = 0; a < WTT; ++a)
#pragma unroll
    for (int b = 0; b < WTT; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  uint4 ra[2], rc[2];
  auto gload = [&](int64_t tb) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = tid + 256 * q;
      ra[q] = make_uint4(0, 0, 0, 0);
      rc[q] = make_uint4(0, 0, 0, 0);
      if (e < TK * RC) {
        const int r = e / RC, c = e % RC;
        const int64_t t = tb + r;
        if (t < tend) {
          const uint16_t* pa = A + t * W + col_a + c * 8;
          const uint16_t* pc = C + t * W + col_c + c * 8;
          if (vec) { ra[q] = ldg16(pa); rc[q] = ldg16(pc); }
          else {
            ra[q].x = pack2(pa[0], pa[1]); ra[q].y = pack2(pa[2], pa[3]); ra[q].z = pack2(pa[4], pa[5]); ra[q].w = pack2(pa[6], pa[7]);
            rc[q].x = pack2(pc[0], pc[1]); rc[q].y = pack2(pc[2], pc[3]); rc[q].z = pack2(pc[4], pc[5]); rc[q].w = pack2(pc[6], pc[7]);
          }
        }
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = tid + 256 * q;
      if (e < TK * RC) {
        const int r = e / RC, c = e % RC;
        const int pc = (c ^ (r & 7)) & (RC - 1);
        *reinterpret_cast<uint4*>(&sa[buf][r * TI + pc * 8]) = ra[q];
        *reinterpret_cast<uint4*>(&sc[buf][r * TI + pc * 8]) = rc[q];
      }
    }
  };
  // K-major operand fragment for 32x32x16: lane needs X[t = 8*(lane/32) + e][n = base + lane%32]
  auto frag = [&](const uint16_t* s, int nbase, int ks) -> bf16x8 {
    const int g = lane >> 4, q = lane & 15;
    const int n = nbase + 16 * (g & 1) + 4 * (q & 3);
    const int chn = n >> 3, within = n & 7;
    i16x4 h[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int t = 16 * ks + 8 * (g >> 1) + 4 * hh + (q >> 2);
      h[hh] = ds_read_tr16g(&s[t * TI + (((chn ^ (t & 7)) & (RC - 1)) << 3) + within]);
    }
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
    return __builtin_bit_cast(bf16x8, v);
  };

  const int nsub = (int)((tend - tbeg + TK - 1) / TK);
  if (nsub > 0) {
    gload(tbeg);
    sstore(0);
  }
  __syncthreads();
  for (int sub = 0; sub < nsub; ++sub) {
    const int buf = sub & 1;
    if (sub + 1 < nsub) gload(tbeg + (int64_t)(sub + 1) * TK);
    if (active) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 fa[WTT], fc[WTT];
#pragma unroll
        for (int a = 0; a < WTT; ++a) fa[a] = frag(sa[buf], wi * WS + 32 * a, ks);
#pragma unroll
        for (int b = 0; b < WTT; ++b) fc[b] = frag(sc[buf], wj * WS + 32 * b, ks);
#pragma unroll
        for (int a = 0; a < WTT; ++a)
#pragma unroll
          for (int b = 0; b < WTT; ++b) acc[a][b] = mfma32(fa[a], fc[b], acc[a][b]);
      }
    }
    if (sub + 1 < nsub) sstore(buf ^ 1);
    __syncthreads();
  }
  if (active) {
    float* o = out + ((int64_t)chunk * k + l) * B * B;
#pragma unroll
    for (int a = 0; a < WTT; ++a)
#pragma unroll
      for (int b = 0; b < WTT; ++b) {
        const int j = tj * TI + wj * WS + 32 * b + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = ti * TI + wi * WS + 32 * a + c32_row(lane, r);
          o[(int64_t)i * B + j] = acc[a][b][r];
        }
      }
  }
}

// Streaming variant for B in {128, 256}: one workgroup per (block l,
// 128 x 128 quadrant, token run), 8 waves of 32 x 64; the run's 32-token
// tiles of both operands stream through a ring of GR_S LDS stages with
// buffer-to-LDS loads, GR_S - 1 tiles in flight.  The loop issues exactly two
// loads per lane per tile (past the end of the run they read nothing) and no
// stores, so one constant vmcnt wait is exact.  Items are ordered (block,
// run, quadrant) and laid out so that the four quadrants of a run sit on one
// XCD and share its L2 for the operand halves they have in common.
__global__ __launch_bounds__(512) void gram_stream_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ C,
                                                          int64_t N, int W, int B, int k, int runs, int tpc,
                                                          int nitems, float* __restrict__ out) {
  __shared__ __align__(16) uint16_t L0[2 * GR_E], L1[2 * GR_E], L2[2 * GR_E], L3[2 * GR_E], L4[2 * GR_E],
      L5[2 * GR_E], L6[2 * GR_E];
  static_assert(GR_S == 7, "the ring is spelled out for seven stages");
  const int per = (nitems + 7) / 8;
  const int item = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (item >= nitems) return;
  const int tpb = B / GR_TI, q = tpb * tpb;
  const int quad = item % q, run = (item / q) % runs, l = item / (q * runs);
  const int ti = quad / tpb, tj = quad % tpb;
  const int64_t t0 = (int64_t)run * tpc * GR_T;
  if (t0 >= N) return;
  const int rows = (int)min((int64_t)tpc * GR_T, N - t0);
  const int nt = (rows + GR_T - 1) / GR_T;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = wave >> 1, wj = wave & 1;
  const uint32_t ldb = (uint32_t)W * 2;

  // operand tiles [32 tokens][128 columns], 256-byte rows; chunk c of token
  // row t at c ^ ((t & 3) << 2), so that a 32-lane phase of the transposing
  // fragment read (4 rows x 4 chunks x 2 halves) touches every bank pair once
  const BufRange ga = tile_range(t0, rows, (int64_t)l * B + ti * GR_TI, GR_TI, W, 2);
  const BufRange gc = tile_range(t0, rows, (int64_t)l * B + tj * GR_TI, GR_TI, W, 2);
  const __amdgpu_buffer_rsrc_t ra = gr_rsrc(A + ga.first, (uint32_t)ga.bytes);
  const __amdgpu_buffer_rsrc_t rc = gr_rsrc(C + gc.first, (uint32_t)gc.bytes);
  // wave w fills KiB w of both tiles of a stage: token row 4 w + lane / 16, chunk lane % 16
  int voff;
  {
    const int r = wave * 4 + (lane >> 4), p = lane & 15;
    voff = (int)((uint32_t)r * ldb + (uint32_t)((p ^ ((r & 3) << 2)) << 4));
  }
  const uint32_t tstep = (uint32_t)GR_T * ldb;
  auto load_tile = [&](int i, uint16_t* st) {
    gr_b2l16(ra, voff + (int)((uint32_t)i * tstep), st + wave * 512);
    gr_b2l16(rc, voff + (int)((uint32_t)i * tstep), st + GR_E + wave * 512);
  };

  f32x16 acc[2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;

  // K-major fragment for 32x32x16: lane holds X[t = 16 ks + 8 (lane / 32) + e][n = nbase + lane % 32]
  auto frag = [&](const uint16_t* s, int nbase, int ks) -> bf16x8 {
    const int g = lane >> 4, qq = lane & 15;
    const int n = nbase + 16 * (g & 1) + 4 * (qq & 3);
    const int chn = n >> 3, within = n & 7;
    i16x4 h[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int t = 16 * ks + 8 * (g >> 1) + 4 * hh + (qq >> 2);
      h[hh] = ds_read_tr16g(&s[t * GR_TI + ((chn ^ ((t & 3) << 2)) << 3) + within]);
    }
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
    return __builtin_bit_cast(bf16x8, v);
  };
  auto compute = [&](const uint16_t* st) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 fa = frag(st, 32 * wi, ks);
      const bf16x8 fc0 = frag(st + GR_E, 64 * wj, ks);
      const bf16x8 fc1 = frag(st + GR_E, 64 * wj + 32, ks);
      acc[0] = mfma32(fa, fc0, acc[0]);
      acc[1] = mfma32(fa, fc1, acc[1]);
    }
  };

  // prologue: tiles 0 .. S-2 in issue order
  load_tile(0, L0);
  asm volatile("" ::: "memory");
  load_tile(1, L1);
  asm volatile("" ::: "memory");
  load_tile(2, L2);
  asm volatile("" ::: "memory");
  load_tile(3, L3);
  asm volatile("" ::: "memory");
  load_tile(4, L4);
  asm volatile("" ::: "memory");
  load_tile(5, L5);
  // step i: wait for this lane's loads of tile i (the 2 (S - 2) loads issued
  // after them may stay in flight), barrier, refill the stage tile i - 1
  // used, compute
#define GR_STEP(I, CUR, NEXT)                                  \
  {                                                            \
    asm volatile("" ::: "memory");                             \
    __builtin_amdgcn_s_waitcnt(gr_vm_imm(2 * (GR_S - 2)));     \
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");         \
    __builtin_amdgcn_s_barrier();                              \
    asm volatile("" ::: "memory");                             \
    load_tile((I) + GR_S - 1, NEXT);                           \
    compute(CUR);                                              \
  }
  // whole rounds (no early exit inside: that makes the compiler copy the
  // accumulators), then the remaining steps
  int i = 0;
  for (; i + GR_S <= nt; i += GR_S) {
    GR_STEP(i, L0, L6) GR_STEP(i + 1, L1, L0) GR_STEP(i + 2, L2, L1) GR_STEP(i + 3, L3, L2)
    GR_STEP(i + 4, L4, L3) GR_STEP(i + 5, L5, L4) GR_STEP(i + 6, L6, L5)
  }
  if (i < nt) GR_STEP(i, L0, L6)
  if (i + 1 < nt) GR_STEP(i + 1, L1, L0)
  if (i + 2 < nt) GR_STEP(i + 2, L2, L1)
  if (i + 3 < nt) GR_STEP(i + 3, L3, L2)
  if (i + 4 < nt) GR_STEP(i + 4, L4, L3)
  if (i + 5 < nt) GR_STEP(i + 5, L5, L4)
#undef GR_STEP
  // fills past the end of the run may still be writing this workgroup's LDS
  __builtin_amdgcn_s_waitcnt(gr_vm_imm(0));

  // partial of this run: acc[b] register r of lane l is G[32 wi + c32_row(l, r)][64 wj + 32 b + l % 32]
  float* o = out + ((int64_t)run * k + l) * B * B;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int j = tj * GR_TI + 64 * wj + 32 * b + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ii = ti * GR_TI + 32 * wi + c32_row(lane, r);
      o[(int64_t)ii * B + j] = acc[b][r];
    }
  }
}

__global__ void gram_reduce_kernel(const float* __restrict__ part, int chunks, int64_t count, float* __restrict__ G) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= count) return;
  float s = 0.f;
  for (int c = 0; c < chunks; ++c) s += part[(int64_t)c * count + e];
  G[e] = s;
}

__global__ void gram_f32_kernel(const float* __restrict__ A, const float* __restrict__ C, int64_t N, int W, int B, int k,
                                float* __restrict__ G) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)k * B * B) return;
  const int l = (int)(e / ((int64_t)B * B));
  const int rem = (int)(e - (int64_t)l * B * B);
  const int i = rem / B, j = rem % B;
  float s = 0.f;
  for (int64_t t = 0; t < N; ++t) s = fmaf(A[t * W + l * B + i], C[t * W + l * B + j], s);
  G[e] = s;
}

void launch_gram(bool f32, const void* A, const void* C, int64_t N, int W, int B, int k, float* G, void* partials,
                 hipStream_t s) {
  if (k <= 0) return;
  const int64_t count = (int64_t)k * B * B;
  if (f32) {
    hipLaunchKernelGGL(gram_f32_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s,
                       static_cast<const float*>(A), static_cast<const float*>(C), N, W, B, k, G);
    return;
  }
  if (N <= 0) {
    launch_fill_f32(G, 0.f, count, s);
    return;
  }
  if (gram_stream_ok(N, W, B, A, C)) {
    const GramRuns gr = gram_stream_runs(N, B, k);
    const int q = (B / GR_TI) * (B / GR_TI);
    const int nitems = k * q * gr.runs;
    float* dst = gr.runs == 1 ? G : static_cast<float*>(partials);
    hipLaunchKernelGGL(gram_stream_kernel, dim3((unsigned)(((nitems + 7) / 8) * 8)), dim3(512), 0, s,
                       static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(C), N, W, B, k, gr.runs, gr.tpc,
                       nitems, dst);
    if (gr.runs > 1)
      hipLaunchKernelGGL(gram_reduce_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s,
                         static_cast<const float*>(partials), gr.runs, count, G);
    return;
  }
  const int ti = gram_tile(B);
  const int chunks = gram_chunks(N, B, k);
  int64_t clen = (N + chunks - 1) / chunks;
  clen = ((clen + 31) / 32) * 32;
  float* dst = chunks == 1 ? G : static_cast<float*>(partials);
  const int tpb = B / ti;
  dim3 grid((unsigned)((int64_t)k * tpb * tpb * chunks));
  const uint16_t* a16 = static_cast<const uint16_t*>(A);
  const uint16_t* c16 = static_cast<const uint16_t*>(C);
  if (ti == 128) hipLaunchKernelGGL((gram_bf16_kernel<128, 2>), grid, dim3(256), 0, s, a16, c16, N, W, B, k, chunks, clen, dst);
  else if (ti == 64) hipLaunchKernelGGL((gram_bf16_kernel<64, 1>), grid, dim3(256), 0, s, a16, c16, N, W, B, k, chunks, clen, dst);
  else hipLaunchKernelGGL((gram_bf16_kernel<32, 1>), grid, dim3(256), 0, s, a16, c16, N, W, B, k, chunks, clen, dst);
  if (chunks > 1)
    hipLaunchKernelGGL(gram_reduce_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s,
                       static_cast<const float*>(partials), chunks, count, G);
}

}  // namespace poetx
