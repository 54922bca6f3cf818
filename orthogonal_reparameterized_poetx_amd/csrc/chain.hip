// Chain rule from G = dL/dQ to the stored generator, bf16 layers.
//
// dL/dS = 1/2 (I + Q^T) G (I + Q^T) and dtheta_p = G_S[i][j] - G_S[j][i] for
// the generator's strict upper triangle (automatic differentiation carried to
// the generator [P1 "POET-X：基于正交变换缩放的内存高效LLM训练方法", 实践 2];
// upper-triangle storage [P3 "POET-X: Memory-efficient LLM Training by
// Scaling Orthogonal Transformation", Methodologie item 4]).
//
// The two b x b products per block must be fp32-accurate: G_S is nearly
// symmetric for small generators and the projection keeps only its
// antisymmetric part.  Each product runs on bf16 MFMA over split operands
// (x = hi + lo with hi = bf16(x), lo = bf16(x - hi); x*y ~ hi*hi + hi*lo +
// lo*hi, fp32 accumulation).  The split happens while a tile moves from
// global memory to LDS, so the products read the fp32 operands once and no
// split copies are stored:
//   product 1:  C1 = 1/2 (I + Q) G^T   (= T^T / 2 with T = G (I + Q^T))
//   product 2:  G_S = (I + Q^T) C1^T   (= 1/2 (I + Q^T) T)
// Both are "NT" products C[i][j] = sum_k A[i][k] Bt[j][k]; product 2 reads
// Q by columns and transposes it in registers on the way to LDS.
#include "common.h"
#include "kernels.h"

namespace poetx {

__device__ __forceinline__ int chain_seg_of(const ChainSegs& cs, int z) {
  int sg = 0;
  while (sg + 1 < cs.nseg && z >= cs.start[sg + 1]) ++sg;
  return sg;
}

// Workgroup tile TM x TM of one block's C, K in steps of 32.  Waves form a
// WG x WG grid, each owning WT x WT MFMA tiles of 32 x 32.
template <int TM> struct CpShape {
  static constexpr int WG = TM >= 64 ? 2 : 1;
  static constexpr int WT = TM / (32 * WG);
  static constexpr int NT = 64 * WG * WG;
  static constexpr int ROWB = 64;                 // bytes per LDS row: 32 bf16 of k
  static constexpr int ARR = TM * ROWB;           // one of A_hi, A_lo, B_hi, B_lo
  static constexpr int STAGE = 4 * ARR;
  static constexpr int PN = TM * 8 / NT;          // row-wise float4 loads per thread per operand
  static constexpr int PT = 8 * TM / NT;          // column-wise 4-element groups per thread
};

// LDS byte offset of k-quad q (4 bf16, 0..7) of row r; 16-byte chunks are
// xor-swizzled by row so that the 32 rows an MFMA operand read touches fall
// on distinct banks.
__device__ __forceinline__ int cp_off(int r, int q) {
  return r * 64 + (((q >> 1) ^ ((r >> 1) & 3)) << 4) + ((q & 1) << 3);
}

__device__ __forceinline__ void cp_put(char* lds_hi, char* lds_lo, int off, float4 v) {
  bf16 h0, h1, h2, h3, l0, l1, l2, l3;
  split_bf16(v.x, h0, l0);
  split_bf16(v.y, h1, l1);
  split_bf16(v.z, h2, l2);
  split_bf16(v.w, h3, l3);
  const bf16x4 h = {h0, h1, h2, h3}, l = {l0, l1, l2, l3};
  *reinterpret_cast<bf16x4*>(lds_hi + off) = h;
  *reinterpret_cast<bf16x4*>(lds_lo + off) = l;
}

// AT: A[i][k] = delta_ik + Q[k][i] (else delta_ik + Q[i][k]).
// BSEG: Bt comes from the segments' g arrays (else the contiguous array Bc).
// C[z] = alpha * A Bt^T, contiguous [nblk][b][b].
template <int TM, bool AT, bool BSEG>
__global__ __launch_bounds__(CpShape<TM>::NT) void chain_product_kernel(ChainSegs cs, int b, const float* Bc,
                                                                        float* C, float alpha, int total) {
  using S = CpShape<TM>;
  __shared__ __align__(16) char cp_lds[2 * S::STAGE];
  const int nt = b / TM, tpb = nt * nt;
  // XCD-aware order: workgroup g runs on XCD g % 8; consecutive logical tiles
  // (the tiles of one block, which share operand panels) go to one XCD's L2.
  const int per = (total + 7) / 8;
  const int lg = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (lg >= total) return;
  const int z = lg / tpb, t = lg - z * tpb;
  const int i0 = (t / nt) * TM, j0 = (t % nt) * TM;
  const int64_t bb = (int64_t)b * b;
  const int sg = chain_seg_of(cs, z);
  const int64_t zl = z - cs.start[sg];
  const float* __restrict__ Q = cs.seg[sg].q + zl * bb;
  const float* __restrict__ Bt = BSEG ? cs.seg[sg].g + zl * bb : Bc + (int64_t)z * bb;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / S::WG, wn = w % S::WG;

  float4 ra[AT ? S::PT : S::PN], rb[S::PN];
  auto load = [&](int k0) {
    if (AT) {
#pragma unroll
      for (int p = 0; p < S::PT; ++p) {
        const int i = tid % TM, g = tid / TM + (S::NT / TM) * p;
        const float* src = Q + (int64_t)(k0 + 4 * g) * b + i0 + i;
        ra[p] = make_float4(src[0], src[b], src[2 * b], src[3 * b]);
      }
    } else {
#pragma unroll
      for (int p = 0; p < S::PN; ++p) {
        const int r = tid / 8 + (S::NT / 8) * p, q = tid % 8;
        ra[p] = *reinterpret_cast<const float4*>(Q + (int64_t)(i0 + r) * b + k0 + 4 * q);
      }
    }
#pragma unroll
    for (int p = 0; p < S::PN; ++p) {
      const int r = tid / 8 + (S::NT / 8) * p, q = tid % 8;
      rb[p] = *reinterpret_cast<const float4*>(Bt + (int64_t)(j0 + r) * b + k0 + 4 * q);
    }
  };
  auto stage = [&](int s, int k0) {
    char* base = cp_lds + s * S::STAGE;
    if (AT) {
#pragma unroll
      for (int p = 0; p < S::PT; ++p) {
        const int i = tid % TM, g = tid / TM + (S::NT / TM) * p;
        float4 v = ra[p];
        const int d = i0 + i - (k0 + 4 * g);   // identity entry at k = i
        if (d == 0) v.x += 1.f;
        if (d == 1) v.y += 1.f;
        if (d == 2) v.z += 1.f;
        if (d == 3) v.w += 1.f;
        cp_put(base, base + S::ARR, cp_off(i, g), v);
      }
    } else {
#pragma unroll
      for (int p = 0; p < S::PN; ++p) {
        const int r = tid / 8 + (S::NT / 8) * p, q = tid % 8;
        float4 v = ra[p];
        const int d = i0 + r - (k0 + 4 * q);
        if (d == 0) v.x += 1.f;
        if (d == 1) v.y += 1.f;
        if (d == 2) v.z += 1.f;
        if (d == 3) v.w += 1.f;
        cp_put(base, base + S::ARR, cp_off(r, q), v);
      }
    }
#pragma unroll
    for (int p = 0; p < S::PN; ++p) {
      const int r = tid / 8 + (S::NT / 8) * p, q = tid % 8;
      cp_put(base + 2 * S::ARR, base + 3 * S::ARR, cp_off(r, q), rb[p]);
    }
  };

  f32x16 acc[S::WT][S::WT];
#pragma unroll
  for (int a = 0; a < S::WT; ++a)
#pragma unroll
    for (int c = 0; c < S::WT; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][c][r] = 0.f;

  const int nk = b / 32;
  load(0);
  stage(0, 0);
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    if (it + 1 < nk) load(32 * (it + 1));
    const char* base = cp_lds + (it & 1) * S::STAGE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int q = 4 * ks + 2 * (lane >> 5);   // first k-quad of this lane's 8 k
      bf16x8 ah[S::WT], al[S::WT], bh[S::WT], bl[S::WT];
#pragma unroll
      for (int a = 0; a < S::WT; ++a) {
        const int r = (wm * S::WT + a) * 32 + (lane & 31);
        ah[a] = *reinterpret_cast<const bf16x8*>(base + cp_off(r, q));
        al[a] = *reinterpret_cast<const bf16x8*>(base + S::ARR + cp_off(r, q));
      }
#pragma unroll
      for (int c = 0; c < S::WT; ++c) {
        const int r = (wn * S::WT + c) * 32 + (lane & 31);
        bh[c] = *reinterpret_cast<const bf16x8*>(base + 2 * S::ARR + cp_off(r, q));
        bl[c] = *reinterpret_cast<const bf16x8*>(base + 3 * S::ARR + cp_off(r, q));
      }
#pragma unroll
      for (int a = 0; a < S::WT; ++a)
#pragma unroll
        for (int c = 0; c < S::WT; ++c) {
          acc[a][c] = mfma32(ah[a], bh[c], acc[a][c]);
          acc[a][c] = mfma32(ah[a], bl[c], acc[a][c]);
          acc[a][c] = mfma32(al[a], bh[c], acc[a][c]);
        }
    }
    if (it + 1 < nk) stage((it + 1) & 1, 32 * (it + 1));
    __syncthreads();
  }

  float* Cz = C + (int64_t)z * bb;
#pragma unroll
  for (int a = 0; a < S::WT; ++a)
#pragma unroll
    for (int c = 0; c < S::WT; ++c) {
      const int rb0 = i0 + (wm * S::WT + a) * 32, cb0 = j0 + (wn * S::WT + c) * 32;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        Cz[(int64_t)(rb0 + c32_row(lane, r)) * b + cb0 + (lane & 31)] = alpha * acc[a][c][r];
    }
}

// dtheta[p(i, j)] (+)= GS[i][j] - GS[j][i] for i < j.  One workgroup per pair
// of 32 x 32 tiles (I, J), I <= J, of one block; tile (J, I) is read by rows
// and transposed through LDS, so both reads are coalesced.
__global__ __launch_bounds__(256) void skew_project_kernel(const float* __restrict__ GS, int b, ChainSegs cs,
                                                           int accumulate) {
  __shared__ float tt[32][33];
  const int z = blockIdx.y;
  const int nt = b / 32;
  int I = 0, pr = blockIdx.x;   // pair index -> (I, J), J = I .. nt-1
  while (pr >= nt - I) { pr -= nt - I; ++I; }
  const int J = I + pr;
  const int64_t bb = (int64_t)b * b;
  const float* g = GS + (int64_t)z * bb;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  // tt[c][r] = GS[32J + r][32I + c]
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = ty + 8 * k;
    tt[tx][r] = g[(int64_t)(32 * J + r) * b + 32 * I + tx];
  }
  __syncthreads();
  const int sg = chain_seg_of(cs, z);
  float* dth = cs.seg[sg].dth + (int64_t)(z - cs.start[sg]) * (b * (b - 1) / 2);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = ty + 8 * k;
    const int i = 32 * I + r, j = 32 * J + tx;
    if (j <= i) continue;
    const float v = g[(int64_t)i * b + j] - tt[r][tx];
    float* d = dth + (i * b - i * (i + 1) / 2 + (j - i - 1));
    *d = accumulate ? (*d + v) : v;
  }
}

// ----------------------------------------------------------------------------
template <int TM, bool AT, bool BSEG>
static void launch_cp(const ChainSegs& cs, int nblk, int b, const float* Bc, float* C, float alpha, hipStream_t s) {
  using S = CpShape<TM>;
  const int total = nblk * (b / TM) * (b / TM);
  const int grid = ((total + 7) / 8) * 8;
  hipLaunchKernelGGL((chain_product_kernel<TM, AT, BSEG>), dim3(grid), dim3(S::NT), 0, s, cs, b, Bc, C,
                     alpha, total);
}

template <int TM>
static void chain_products_t(const ChainSegs& cs, int nblk, int b, float* C1, float* GS, hipStream_t s) {
  launch_cp<TM, false, true>(cs, nblk, b, nullptr, C1, 0.5f, s);   // C1 = (I + Q) G^T / 2
  launch_cp<TM, true, false>(cs, nblk, b, C1, GS, 1.f, s);         // G_S = (I + Q^T) C1^T
}

void launch_chain_products(const ChainSegs& cs, int nblk, int b, float* C1, float* GS, hipStream_t s) {
  if (nblk <= 0) return;
  if (b >= 128) chain_products_t<128>(cs, nblk, b, C1, GS, s);
  else if (b == 64) chain_products_t<64>(cs, nblk, b, C1, GS, s);
  else chain_products_t<32>(cs, nblk, b, C1, GS, s);
}

void launch_skew_project(const float* GS, int b, int nblk, const ChainSegs& cs, int accumulate, hipStream_t s) {
  if (nblk <= 0) return;
  const int nt = b / 32;
  dim3 grid((unsigned)(nt * (nt + 1) / 2), (unsigned)nblk);
  hipLaunchKernelGGL(skew_project_kernel, grid, dim3(256), 0, s, GS, b, cs, accumulate);
}

}  // namespace poetx
