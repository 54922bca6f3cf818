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

}  // namespace poetx
