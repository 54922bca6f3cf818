// Permuted block-diagonal transforms of token rows (the P and R sides).
//
// The orthogonal factors are permutation x block-diagonal x permutation; the
// permutations are applied as index maps, never as matrices, and the blocks
// are treated as a batch of independent b x b products
// [P3 "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
// Transformation", Methodologie items 2 and 3].
//
// bf16 path: a transform is a row permutation (this file) plus one batched
// block product over contiguous columns (the strided GEMM of gemm.hip):
//   gather-in  (P forward, R backward): x' = Pi x (permute), then z = D x'
//   scatter-out (R forward, P backward): r = D z, then y = Pi^T r (permute)
// The permutation kernels stream whole rows through LDS at copy speed; the
// block product then reads its operands as contiguous tiles.  (A fused
// kernel that gathers MFMA operand fragments straight from the staged rows
// has to re-read every b x b block once per token tile in fragment order,
// which L2 serves several times slower than contiguous tile loads.)
//
// fp32 path: one thread per output element, sequential fp32 sums.
#include "common.h"
#include "kernels.h"

namespace poetx {

__device__ __forceinline__ void vm_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 16-byte global -> LDS copy without VGPRs: lane i of the wave writes lds_base + 16 i
__device__ __forceinline__ void g2l16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

constexpr int PERM_THREADS = 256;

// rows per workgroup: as many as fit in 64 KiB of LDS, at most 16
static int perm_rows(int W) {
  int r = 32768 / (W > 0 ? W : 1);
  return r < 1 ? 1 : (r > 16 ? 16 : r);
}

// gather: out[t][j] = in[t][perm[j]]; tail_out[t][j] = the same for j >= tail0
template <bool VEC>
__global__ __launch_bounds__(PERM_THREADS) void permute_gather_kernel(PermArgs a, int R) {
  extern __shared__ __align__(16) uint16_t rows[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = a.W;
  const int64_t t0 = (int64_t)blockIdx.x * R;
  const int nr = (int)min((int64_t)R, a.N - t0);
  const uint16_t* __restrict__ in = a.in + t0 * W;
  if (VEC) {
    const int cpr = (W + 511) >> 9;   // 1 KiB chunks per row
    for (int c = wave; c < nr * cpr; c += PERM_THREADS / 64) {
      const int r = c / cpr, j = c - r * cpr;
      const int e0 = (j << 9) + lane * 8;
      if (e0 < W) g2l16(in + (int64_t)r * W + e0, rows + r * W + (j << 9));
    }
    vm_wait_all();
  } else {
    for (int e = tid; e < nr * W; e += PERM_THREADS) rows[e] = in[e];
  }
  __syncthreads();
  uint16_t* __restrict__ out = a.out + t0 * W;
  uint16_t* __restrict__ tout = a.tail_out ? a.tail_out + t0 * W : nullptr;
  if (VEC) {
    // each thread owns 8-column chunks and reads their indices once for all
    // rows of the workgroup
    const int nch = W >> 3;
    for (int c = tid; c < nch; c += PERM_THREADS) {
      const int4 pa = *reinterpret_cast<const int4*>(a.perm + c * 8);
      const int4 pb = *reinterpret_cast<const int4*>(a.perm + c * 8 + 4);
      const bool tl = tout && c * 8 >= a.tail0;
      for (int r = 0; r < nr; ++r) {
        const uint16_t* row = rows + r * W;
        uint4 v;
        v.x = pack2(row[pa.x], row[pa.y]);
        v.y = pack2(row[pa.z], row[pa.w]);
        v.z = pack2(row[pb.x], row[pb.y]);
        v.w = pack2(row[pb.z], row[pb.w]);
        stg16(out + (int64_t)r * W + c * 8, v);
        if (tl) stg16(tout + (int64_t)r * W + c * 8, v);
      }
    }
  } else {
    for (int e = tid; e < nr * W; e += PERM_THREADS) {
      const int r = e / W, j = e - r * W;
      const uint16_t v = rows[r * W + a.perm[j]];
      out[e] = v;
      if (tout && j >= a.tail0) tout[e] = v;
    }
  }
}

// scatter: out[t][perm[j]] = src[t][j], src = in for j < tail0, tail_in beyond
template <bool VEC>
__global__ __launch_bounds__(PERM_THREADS) void permute_scatter_kernel(PermArgs a, int R) {
  extern __shared__ __align__(16) uint16_t rows[];
  const int tid = threadIdx.x;
  const int W = a.W;
  const int64_t t0 = (int64_t)blockIdx.x * R;
  const int nr = (int)min((int64_t)R, a.N - t0);
  const uint16_t* __restrict__ in = a.in + t0 * W;
  const uint16_t* __restrict__ tin = (a.tail_in ? a.tail_in : a.in) + t0 * W;
  if (VEC) {
    const int nch = W >> 3;
    for (int c = tid; c < nch; c += PERM_THREADS) {
      const int4 pa = *reinterpret_cast<const int4*>(a.perm + c * 8);
      const int4 pb = *reinterpret_cast<const int4*>(a.perm + c * 8 + 4);
      const uint16_t* src = (c * 8 < a.tail0 ? in : tin) + c * 8;
      for (int r = 0; r < nr; ++r) {
        const uint4 v = ldg16(src + (int64_t)r * W);
        uint16_t* row = rows + r * W;
        row[pa.x] = (uint16_t)(v.x & 0xffff); row[pa.y] = (uint16_t)(v.x >> 16);
        row[pa.z] = (uint16_t)(v.y & 0xffff); row[pa.w] = (uint16_t)(v.y >> 16);
        row[pb.x] = (uint16_t)(v.z & 0xffff); row[pb.y] = (uint16_t)(v.z >> 16);
        row[pb.z] = (uint16_t)(v.w & 0xffff); row[pb.w] = (uint16_t)(v.w >> 16);
      }
    }
  } else {
    for (int e = tid; e < nr * W; e += PERM_THREADS) {
      const int r = e / W, j = e - r * W;
      rows[r * W + a.perm[j]] = (j < a.tail0 ? in : tin)[e];
    }
  }
  __syncthreads();
  uint16_t* __restrict__ out = a.out + t0 * W;
  if (VEC) {
    const int nch = W >> 3;
    for (int e = tid; e < nr * nch; e += PERM_THREADS) {
      const int r = e / nch, c = e - r * nch;
      stg16(out + (int64_t)r * W + c * 8, *reinterpret_cast<const uint4*>(rows + r * W + c * 8));
    }
  } else {
    for (int e = tid; e < nr * W; e += PERM_THREADS) out[e] = rows[e];
  }
}

static bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

void launch_permute_bf16(bool gather, const PermArgs& a, hipStream_t s) {
  if (a.N <= 0 || a.W <= 0) return;
  const int R = perm_rows(a.W);
  const dim3 grid((unsigned)((a.N + R - 1) / R));
  const size_t lds = (size_t)R * a.W * sizeof(uint16_t);
  const bool vec = (a.W % 8) == 0 && a16(a.in) && a16(a.out) && (!a.tail_in || a16(a.tail_in)) &&
                   (!a.tail_out || a16(a.tail_out));
  if (gather) {
    if (vec) hipLaunchKernelGGL(permute_gather_kernel<true>, grid, dim3(PERM_THREADS), lds, s, a, R);
    else hipLaunchKernelGGL(permute_gather_kernel<false>, grid, dim3(PERM_THREADS), lds, s, a, R);
  } else {
    if (vec) hipLaunchKernelGGL(permute_scatter_kernel<true>, grid, dim3(PERM_THREADS), lds, s, a, R);
    else hipLaunchKernelGGL(permute_scatter_kernel<false>, grid, dim3(PERM_THREADS), lds, s, a, R);
  }
}

// ---------------------------------------------------------------------------
// fp32 path: one thread per output element, sequential fp32 sums
// ---------------------------------------------------------------------------
__global__ void gather_in_f32_kernel(XformArgs a) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int W = a.W, B = a.B;
  if (e >= a.N * W) return;
  const int64_t t = e / W;
  const int j = (int)(e - t * W);
  const float* in = static_cast<const float*>(a.in) + t * W;
  const float* q = static_cast<const float*>(a.bq);
  float v;
  if (j >= a.k * B) v = in[a.perm[j]];
  else {
    const int l = j / B, i = j - l * B;
    const float* ql = q + (int64_t)l * B * B;
    float s = 0.f;
    for (int kk = 0; kk < B; ++kk) {
      const float m = a.trans ? ql[(int64_t)kk * B + i] : ql[(int64_t)i * B + kk];
      s = fmaf(in[a.perm[l * B + kk]], m, s);
    }
    v = s;
  }
  static_cast<float*>(a.out)[e] = v;
  if (a.emit) static_cast<float*>(a.emit)[e] = in[a.perm[j]];
}

__global__ void scatter_out_f32_kernel(XformArgs a) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int W = a.W, B = a.B;
  if (e >= a.N * W) return;
  const int64_t t = e / W;
  const int j = (int)(e - t * W);  // working-layout column
  const float* in = static_cast<const float*>(a.in) + t * W;
  const float* q = static_cast<const float*>(a.bq);
  float v;
  if (j >= a.k * B) v = in[j];
  else {
    const int l = j / B, i = j - l * B;
    const float* ql = q + (int64_t)l * B * B;
    float s = 0.f;
    for (int kk = 0; kk < B; ++kk) {
      const float m = a.trans ? ql[(int64_t)kk * B + i] : ql[(int64_t)i * B + kk];
      s = fmaf(in[l * B + kk], m, s);
    }
    v = s;
  }
  static_cast<float*>(a.out)[t * W + a.perm[j]] = v;
}

void launch_gather_in_f32(const XformArgs& a, hipStream_t s) {
  const int64_t tot = a.N * a.W;
  if (tot <= 0) return;
  hipLaunchKernelGGL(gather_in_f32_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, a);
}
void launch_scatter_out_f32(const XformArgs& a, hipStream_t s) {
  const int64_t tot = a.N * a.W;
  if (tot <= 0) return;
  hipLaunchKernelGGL(scatter_out_f32_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, a);
}

}  // namespace poetx
