// Weight storage formats.  The transposed copy: bf16 W0p [m][n] written as
// [n][m] beside it, so that the forward products can read the weight with
// its output features along the rows' contiguous direction.
//
// POET-XQ weight storage: the frozen base weight kept as INT8 codes with one
// fp32 scale per row and dequantized to bf16 for each pass that reads it
// [P3 "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
// Transformation", Methodologie item 5 (POET-XQ)].  The pages fix no
// granularity; the codes here are symmetric per row (one scale per output
// feature), decided in fp32:
//   s_i = max_j |w_ij| / 127,  q_ij = clamp(rne(w_ij / s_i), -127, 127)
// (s_i = 0 and q_i = 0 for a row of zeros), and the dequantized weight is
// bf16(fp32(s_i * q_ij)), round-to-nearest-even at both steps.
#include "common.h"
#include "kernels.h"

namespace poetx {

// bf16 w[i][j] = bf16(s_i * q[i][j]); 8 codes per thread where rows are
// 8-element aligned, one otherwise
__global__ __launch_bounds__(256) void dequant_rows_kernel(const int8_t* __restrict__ q, const float* __restrict__ sc,
                                                           uint16_t* __restrict__ w, int64_t m, int64_t n, int vec) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if (vec) {
    const int64_t total = m * n / 8;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
      const int64_t e = t * 8;
      const float s = sc[e / n];
      const uint2 c = *reinterpret_cast<const uint2*>(q + e);
      uint32_t o[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t word = h < 2 ? c.x : c.y;
        const int sh = 16 * (h & 1);
        const float lo = (float)(int8_t)(word >> sh) * s;
        const float hi = (float)(int8_t)(word >> (sh + 8)) * s;
        o[h] = pack2(f32_to_bits(lo), f32_to_bits(hi));
      }
      *reinterpret_cast<uint4*>(w + e) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  } else {
    const int64_t total = m * n;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride)
      w[e] = f32_to_bits((float)q[e] * sc[e / n]);
  }
}

// one workgroup per row: the row's absolute maximum, its scale, then the codes
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint16_t* __restrict__ w, int8_t* __restrict__ q,
                                                            float* __restrict__ sc, int64_t n) {
  __shared__ float red[4];
  const int64_t i = blockIdx.x;
  const uint16_t* row = w + i * n;
  int8_t* qrow = q + i * n;
  float a = 0.f;
  for (int64_t j = threadIdx.x; j < n; j += blockDim.x) a = fmaxf(a, fabsf(bits_to_f32(row[j])));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = a / 127.0f;   // IEEE division, round to nearest even
  if (threadIdx.x == 0) sc[i] = s;
  for (int64_t j = threadIdx.x; j < n; j += blockDim.x) {
    int c = 0;
    if (s > 0.f) c = (int)fminf(fmaxf(rintf(bits_to_f32(row[j]) / s), -127.f), 127.f);
    qrow[j] = (int8_t)c;
  }
}

void launch_dequant_rows(const int8_t* q, const float* sc, uint16_t* w, int64_t m, int64_t n, hipStream_t s) {
  if (m <= 0 || n <= 0) return;
  const bool vec = n % 8 == 0 && (reinterpret_cast<uintptr_t>(q) & 7) == 0 && (reinterpret_cast<uintptr_t>(w) & 15) == 0;
  const int64_t work = vec ? m * n / 8 : m * n;
  const int64_t blocks = std::min<int64_t>((work + 255) / 256, 4096);
  hipLaunchKernelGGL(dequant_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, q, sc, w, m, n, vec ? 1 : 0);
}

void launch_quantize_rows(const uint16_t* w, int8_t* q, float* sc, int64_t m, int64_t n, hipStream_t s) {
  if (m <= 0 || n <= 0) return;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)m), dim3(256), 0, s, w, q, sc, n);
}

// writes the 64 x 64 tile t (rows r0.., columns c0.. of an [m][n] matrix)
// transposed into out [n][m]: 16-byte stores of output rows where they are
// 8-element aligned and inside (vout), element by element at ragged edges
__device__ __forceinline__ void store_tile_transposed(const uint16_t (*t)[66], uint16_t* __restrict__ out, int64_t r0,
                                                      int64_t c0, int64_t m, int64_t n, int vout) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int id = tid + 256 * h, col = id >> 3, ch = id & 7;
    const int64_t oc = c0 + col, orr = r0 + ch * 8;   // output row oc, columns orr ..
    if (oc >= n) continue;
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = t[ch * 8 + e][col];
    uint16_t* dst = out + oc * m + orr;
    if (vout && orr + 8 <= m) {
      uint4 x;
      x.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
      x.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
      x.z = (uint32_t)v[4] | ((uint32_t)v[5] << 16);
      x.w = (uint32_t)v[6] | ((uint32_t)v[7] << 16);
      *reinterpret_cast<uint4*>(dst) = x;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (orr + e < m) dst[e] = v[e];
    }
  }
}

// out[c][r] = in[r][c] for a 64 x 64 tile through LDS (pitch 66 elements):
// 16-byte loads of input rows where they are 8-element aligned and the chunk
// lies inside (vin), element by element at ragged edges
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ in, uint16_t* __restrict__ out,
                                                             int64_t m, int64_t n, int vin, int vout) {
  __shared__ uint16_t t[64][66];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int id = tid + 256 * h, row = id >> 3, ch = id & 7;
    const int64_t gr = r0 + row, gc = c0 + ch * 8;
    uint16_t v[8];
    if (vin && gr < m && gc + 8 <= n) {
      const uint4 x = *reinterpret_cast<const uint4*>(in + gr * n + gc);
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (gr < m && gc + e < n) ? in[gr * n + gc + e] : (uint16_t)0;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) t[row][ch * 8 + e] = v[e];
  }
  __syncthreads();
  store_tile_transposed(t, out, r0, c0, m, n, vout);
}

// out [n][m] = bf16(s_i q[i][j]) transposed: the dequantized weight of an INT8
// layer in the layout of the transposed copy (same rounding as
// dequant_rows_kernel); 16 codes per thread where rows are 16-byte aligned
// (vin), one per thread otherwise
__global__ __launch_bounds__(256) void dequant_transpose_kernel(const int8_t* __restrict__ q,
                                                                const float* __restrict__ sc,
                                                                uint16_t* __restrict__ out, int64_t m, int64_t n,
                                                                int vin, int vout) {
  __shared__ uint16_t t[64][66];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int tid = threadIdx.x;
  if (vin) {
    const int row = tid >> 2, cc = (tid & 3) * 16;
    const int64_t gr = r0 + row, gc = c0 + cc;
    uint16_t v[16];
    if (gr < m && gc + 16 <= n) {
      const float s = sc[gr];
      const uint4 x = *reinterpret_cast<const uint4*>(q + gr * n + gc);
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = f32_to_bits((float)(int8_t)(w[e >> 2] >> (8 * (e & 3))) * s);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        v[e] = (gr < m && gc + e < n) ? f32_to_bits((float)q[gr * n + gc + e] * sc[gr]) : (uint16_t)0;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) t[row][cc + e] = v[e];
  } else {
    const int col = tid & 63;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int row = (tid >> 6) + 4 * k;
      const int64_t gr = r0 + row, gc = c0 + col;
      t[row][col] = (gr < m && gc < n) ? f32_to_bits((float)q[gr * n + gc] * sc[gr]) : (uint16_t)0;
    }
  }
  __syncthreads();
  store_tile_transposed(t, out, r0, c0, m, n, vout);
}

void launch_dequant_transpose(const int8_t* q, const float* sc, uint16_t* out, int64_t m, int64_t n, hipStream_t s) {
  if (m <= 0 || n <= 0) return;
  const int vin = n % 16 == 0 && (reinterpret_cast<uintptr_t>(q) & 15) == 0;
  const int vout = m % 8 == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  const dim3 grid((unsigned)((n + 63) / 64), (unsigned)((m + 63) / 64));
  hipLaunchKernelGGL(dequant_transpose_kernel, grid, dim3(256), 0, s, q, sc, out, m, n, vin, vout);
}

void launch_transpose_bf16(const uint16_t* in, uint16_t* out, int64_t m, int64_t n, hipStream_t s) {
  if (m <= 0 || n <= 0) return;
  const int vin = n % 8 == 0 && (reinterpret_cast<uintptr_t>(in) & 15) == 0;
  const int vout = m % 8 == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  const dim3 grid((unsigned)((n + 63) / 64), (unsigned)((m + 63) / 64));
  hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, s, in, out, m, n, vin, vout);
}

}  // namespace poetx
