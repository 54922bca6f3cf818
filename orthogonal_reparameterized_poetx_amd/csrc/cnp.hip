// The truncated Neumann (CNP) form of the Cayley map [P3 "POET-X:
// Memory-efficient LLM Training by Scaling Orthogonal Transformation",
// Methodologie item 4]: for ||S|| < 1, (I - S)^-1 = I + S + S^2 + ..., so
// Q = (I - S)^-1 (I + S) = I + 2 (S + S^2 + ...).  With k terms kept the
// dropped tail has spectral norm at most 2 f^{k+1} / (1 - f), f = ||S||_F;
// a block takes the truncated series only where that bound is within the
// tolerance, every other block the exact solve.  The powers come from
// fp32-accurate batched products (Horner: T_1 = S, T_j = S (I + T_{j-1})).
#include "common.h"
#include "kernels.h"

namespace poetx {

// S of each block from its packed strict upper triangle (row-major)
__global__ void cnp_unpack_s_kernel(const float* __restrict__ theta, int b, float* __restrict__ S) {
  const int blk = blockIdx.y;
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)b * b) return;
  const int i = (int)(e / b), j = (int)(e % b);
  const float* th = theta + (int64_t)blk * (b * (b - 1) / 2);
  float v = 0.f;
  if (i < j) v = th[i * b - i * (i + 1) / 2 + (j - i - 1)];
  else if (i > j) v = -th[j * b - j * (j + 1) / 2 + (i - j - 1)];
  S[(int64_t)blk * b * b + e] = v;
}

// use[blk] = 1 where the truncated series meets the tolerance: f < 1 and
// 2 f^{terms+1} / (1 - f) <= tol, f = ||S||_F (summed in double)
__global__ __launch_bounds__(256) void cnp_guard_kernel(const float* __restrict__ S, int b, int terms, float tol,
                                                        int* __restrict__ use) {
  __shared__ double red[4];
  const int blk = blockIdx.x;
  const float* p = S + (int64_t)blk * b * b;
  double acc = 0.0;
  for (int64_t e = threadIdx.x; e < (int64_t)b * b; e += blockDim.x) acc += (double)p[e] * p[e];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double f = sqrt(red[0] + red[1] + red[2] + red[3]);
    int ok = 0;
    if (f < 1.0) ok = 2.0 * pow(f, terms + 1) / (1.0 - f) <= (double)tol;
    use[blk] = ok;
  }
}

// Q = I + 2 T for the blocks that use the series, into Q32 / Qbf16 / QTbf16
// (32x32 tiles, transposed through LDS)
__global__ __launch_bounds__(256) void cnp_finalize_kernel(const float* __restrict__ T, const int* __restrict__ use,
                                                           int b, float* q32, uint16_t* qbf, uint16_t* qtbf) {
  __shared__ uint16_t t[32][33];
  const int blk = blockIdx.z;
  if (!use[blk]) return;
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t base = (int64_t)blk * b * b;
  for (int r = ty; r < 32; r += 8) {
    const int i = i0 + r, j = j0 + tx;
    const float q = 2.f * T[base + (int64_t)i * b + j] + (i == j ? 1.f : 0.f);
    if (q32) q32[base + (int64_t)i * b + j] = q;
    const uint16_t h = f32_to_bits(q);
    if (qbf) qbf[base + (int64_t)i * b + j] = h;
    t[r][tx] = h;
  }
  __syncthreads();
  if (qtbf)
    for (int r = ty; r < 32; r += 8) qtbf[base + (int64_t)(j0 + r) * b + i0 + tx] = t[tx][r];
}

void launch_cnp_unpack_s(const float* theta, int b, int nblk, float* S, hipStream_t s) {
  if (nblk <= 0) return;
  dim3 grid((unsigned)(((int64_t)b * b + 255) / 256), nblk);
  hipLaunchKernelGGL(cnp_unpack_s_kernel, grid, dim3(256), 0, s, theta, b, S);
}

void launch_cnp_guard(const float* S, int b, int nblk, int terms, float tol, int* use, hipStream_t s) {
  if (nblk <= 0) return;
  hipLaunchKernelGGL(cnp_guard_kernel, dim3(nblk), dim3(256), 0, s, S, b, terms, tol, use);
}

void launch_cnp_finalize(const float* T, const int* use, int b, int nblk, float* q32, uint16_t* qbf, uint16_t* qtbf,
                         hipStream_t s) {
  if (nblk <= 0) return;
  dim3 grid(b / 32, b / 32, nblk);
  hipLaunchKernelGGL(cnp_finalize_kernel, grid, dim3(256), 0, s, T, use, b, q32, qbf, qtbf);
}

}  // namespace poetx
