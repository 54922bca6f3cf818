// Dense products with the frozen weight: the one weight-sized matmul that the
// input-centric formulation keeps per pass
// [P3 "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
// Transformation", Probleemstelling (dense matmuls made POET slow) and
// Methodologie item 1].
//
//   NT: C[M][N] = A[M][K] * B[N][K]^T   (z2 = z1 W0p^T; both K-contiguous)
//   NN: C[M][N] = A[M][K] * B[K][N]     (gz1 = gz2 W0p; B is N-contiguous)
//
// bf16 operands, fp32 accumulation on 32x32x16 MFMA, bf16 output.  256x256x64
// tiles, 8 waves of 128x64, double-buffered LDS with 16-byte XOR swizzle; the
// NN B operand is read K-major straight from the N-contiguous tile with the
// gfx950 transposing LDS load.  Tiles are assigned so that the workgroups on
// one XCD (blockIdx mod 8) work on neighbouring output tiles and share L2.
#include "common.h"
#include "kernels.h"

namespace poetx {

constexpr int GBM = 256, GBN = 256, GBK = 64;

__device__ __forceinline__ i16x4 ds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, const_cast<uint16_t*>(p)));
}

template <bool NN>
__global__ __launch_bounds__(512) void gemm_bf16_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bm,
                                                        uint16_t* __restrict__ C, int M, int N, int K, int tiles_n,
                                                        int ntiles) {
  __shared__ __align__(16) uint16_t As[2][GBM * GBK];
  __shared__ __align__(16) uint16_t Bs[2][GBN * GBK];
  // XCD-aware tile order: dispatch id d runs on XCD d % 8; give each XCD a
  // contiguous run of tiles (row-major over the tile grid).
  const int d = blockIdx.x;
  const int per = (ntiles + 7) / 8;
  const int tile = (d % 8) * per + d / 8;
  if (tile >= ntiles) return;
  const int bm = tile / tiles_n, bn = tile % tiles_n;
  const int m0 = bm * GBM, n0 = bn * GBN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 512 * q;
      const int row = e >> 3, c = e & 7;
      const int gm = m0 + row, gk = k0 + c * 8;
      ra[q] = (gm < M && gk < K) ? ldg16(A + (int64_t)gm * K + gk) : make_uint4(0, 0, 0, 0);
      if constexpr (!NN) {
        const int gn = n0 + row;
        rb[q] = (gn < N && gk < K) ? ldg16(Bm + (int64_t)gn * K + gk) : make_uint4(0, 0, 0, 0);
      } else {
        const int kr = e >> 5, cn = e & 31;
        const int gkr = k0 + kr, gn = n0 + cn * 8;
        rb[q] = (gkr < K && gn < N) ? ldg16(Bm + (int64_t)gkr * N + gn) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 512 * q;
      const int row = e >> 3, c = e & 7;
      *reinterpret_cast<uint4*>(&As[buf][row * GBK + ((c ^ (row & 7)) << 3)]) = ra[q];
      if constexpr (!NN) {
        *reinterpret_cast<uint4*>(&Bs[buf][row * GBK + ((c ^ (row & 7)) << 3)]) = rb[q];
      } else {
        const int kr = e >> 5, cn = e & 31;
        *reinterpret_cast<uint4*>(&Bs[buf][kr * GBN + ((cn ^ (kr & 7)) << 3)]) = rb[q];
      }
    }
  };

  const int nk = (K + GBK - 1) / GBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * GBK);
    const uint16_t* as = As[buf];
    const uint16_t* bs = Bs[buf];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + (lane & 31);
        const int ch = 2 * s + (lane >> 5);
        af[i] = *reinterpret_cast<const bf16x8*>(&as[row * GBK + ((ch ^ (row & 7)) << 3)]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (!NN) {
          const int row = wn * 64 + j * 32 + (lane & 31);
          const int ch = 2 * s + (lane >> 5);
          bfr[j] = *reinterpret_cast<const bf16x8*>(&bs[row * GBK + ((ch ^ (row & 7)) << 3)]);
        } else {
          const int g = lane >> 4, q = lane & 15;
          const int ncol = wn * 64 + j * 32 + 16 * (g & 1) + 4 * (q & 3);
          const int chn = ncol >> 3, within = ncol & 7;
          i16x4 h[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int kr = 16 * s + 8 * (g >> 1) + 4 * hh + (q >> 2);
            h[hh] = ds_read_tr16(&bs[kr * GBN + ((chn ^ (kr & 7)) << 3) + within]);
          }
          typedef short i16x8 __attribute__((ext_vector_type(8)));
          i16x8 v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
          bfr[j] = __builtin_bit_cast(bf16x8, v);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: bf16 stores
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int gn = n0 + wn * 64 + j * 32 + (lane & 31);
      if (gn < N) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int gm = m0 + wm * 128 + i * 32 + c32_row(lane, r);
          if (gm < M) C[(int64_t)gm * N + gn] = f32_to_bits(acc[i][j][r]);
        }
      }
    }
}

// Generic bf16 GEMM for shapes the tiled kernel cannot take (K or N not a
// multiple of 8): 16x16 outputs per workgroup, LDS tiles, fp32 sums.
template <bool NN>
__global__ __launch_bounds__(256) void gemm_bf16_generic_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bm,
                                                                uint16_t* __restrict__ C, int M, int N, int K) {
  __shared__ float as[16][17], bs[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int gm = blockIdx.y * 16 + ty, gn = blockIdx.x * 16 + tx;
  float s = 0.f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const int ar = blockIdx.y * 16 + ty, ak = k0 + tx;
    as[ty][tx] = (ar < M && ak < K) ? bits_to_f32(A[(int64_t)ar * K + ak]) : 0.f;
    const int bk = k0 + ty, bn = blockIdx.x * 16 + tx;
    float bv = 0.f;
    if (bk < K && bn < N) bv = NN ? bits_to_f32(Bm[(int64_t)bk * N + bn]) : bits_to_f32(Bm[(int64_t)bn * K + bk]);
    bs[ty][tx] = bv;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) s = fmaf(as[ty][kk], bs[kk][tx], s);
    __syncthreads();
  }
  if (gm < M && gn < N) C[(int64_t)gm * N + gn] = f32_to_bits(s);
}

void launch_gemm_bf16(bool nn, const uint16_t* A, const uint16_t* Bm, uint16_t* C, int64_t M, int64_t N, int64_t K,
                      hipStream_t s) {
  if (M <= 0 || N <= 0) return;
  if ((K % 8) == 0 && (N % 8) == 0 && K > 0) {
    const int tn = (int)((N + GBN - 1) / GBN), tm = (int)((M + GBM - 1) / GBM);
    const int nt = tn * tm;
    const int grid = ((nt + 7) / 8) * 8;
    if (nn) hipLaunchKernelGGL(gemm_bf16_kernel<true>, dim3(grid), dim3(512), 0, s, A, Bm, C, (int)M, (int)N, (int)K, tn, nt);
    else hipLaunchKernelGGL(gemm_bf16_kernel<false>, dim3(grid), dim3(512), 0, s, A, Bm, C, (int)M, (int)N, (int)K, tn, nt);
  } else {
    dim3 grid((unsigned)((N + 15) / 16), (unsigned)((M + 15) / 16));
    if (nn) hipLaunchKernelGGL(gemm_bf16_generic_kernel<true>, grid, dim3(256), 0, s, A, Bm, C, (int)M, (int)N, (int)K);
    else hipLaunchKernelGGL(gemm_bf16_generic_kernel<false>, grid, dim3(256), 0, s, A, Bm, C, (int)M, (int)N, (int)K);
  }
}

// fp32 GEMM: 64x64 tile, 256 threads x (4x4), K chunks of 16, fp32 FMA
template <bool NN>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ Bm,
                                                       float* __restrict__ C, int M, int N, int K) {
  __shared__ float as[16][65], bs[16][65];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int e = tid; e < 1024; e += 256) {
      const int kk = e & 15, r = e >> 4;
      const int gm = m0 + r, gk = k0 + kk;
      as[kk][r] = (gm < M && gk < K) ? A[(int64_t)gm * K + gk] : 0.f;
      float bv = 0.f;
      if (NN) {
        const int kr = e >> 6, c = e & 63;
        const int gkr = k0 + kr, gn = n0 + c;
        if (gkr < K && gn < N) bv = Bm[(int64_t)gkr * N + gn];
        bs[kr][c] = bv;
      } else {
        const int gn = n0 + r;
        if (gn < N && gk < K) bv = Bm[(int64_t)gn * K + gk];
        bs[kk][r] = bv;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = as[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gm = m0 + ty * 4 + i, gn = n0 + tx * 4 + j;
      if (gm < M && gn < N) C[(int64_t)gm * N + gn] = acc[i][j];
    }
}

void launch_gemm_f32(bool nn, const float* A, const float* Bm, float* C, int64_t M, int64_t N, int64_t K,
                     hipStream_t s) {
  if (M <= 0 || N <= 0) return;
  dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
  if (nn) hipLaunchKernelGGL(gemm_f32_kernel<true>, grid, dim3(256), 0, s, A, Bm, C, (int)M, (int)N, (int)K);
  else hipLaunchKernelGGL(gemm_f32_kernel<false>, grid, dim3(256), 0, s, A, Bm, C, (int)M, (int)N, (int)K);
}

}  // namespace poetx
