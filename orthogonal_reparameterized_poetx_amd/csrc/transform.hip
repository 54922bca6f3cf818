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

// rows per workgroup: as many as fit in 32 KiB of LDS, at most 16
static int perm_rows(int W) {
  int r = 16384 / (W > 0 ? W : 1);
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

// ---------------------------------------------------------------------------
// Streaming permutation.  One workgroup owns a run of token rows; groups of
// PS_R = 8192 / W rows stream through a ring of PS_S LDS stages with
// buffer-to-LDS loads (PS_S - 1 groups in flight), and every output chunk of 8
// columns is gathered from the staged rows through a uint16 index table in
// LDS (the permutation for a gather, its inverse for a scatter) and leaves as
// one 16-byte buffer store.  Reads of one group overlap the writes of the
// previous ones, which the load-everything-then-store kernel above cannot
// do.  Per lane every iteration issues exactly two loads and NS stores (idle
// slots use offsets past the buffer range: the loads read nothing and the
// stores write nothing), in an order that compiler barriers fix, so the wait
// for a group is one constant from the PS_S-th iteration on and a smaller one
// before.
// ---------------------------------------------------------------------------
constexpr int PS_S = 6;          // ring stages
constexpr int PS_E = 8192;       // elements per stage (16 KiB)
constexpr int PS_THREADS = 512;
constexpr int PS_OOB = 0x7ffffff0;   // a buffer offset past every range

typedef unsigned ps_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ps_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void ps_b2l16(__amdgpu_buffer_rsrc_t r, int voff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, voff, 0, 0, 0);
}
constexpr unsigned ps_vm_imm(unsigned vm) { return (vm & 15u) | ((vm >> 4) << 14) | (7u << 4) | (15u << 8); }
__device__ __forceinline__ uint32_t ps_lds_addr(const void* p) { return (uint32_t)reinterpret_cast<uintptr_t>(p); }

// LDS reads of the loop as inline asm: the compiler's wait insertion cannot
// tell which ring stage an asynchronous fill targets and would wait for
// nearly all of them before every read; the explicit vmcnt wait and the
// barriers order these instead.  Each block waits for its own results, and
// its outputs are early-clobber (no in-flight read can land in a register a
// later address of the block still needs).
__device__ __forceinline__ void ps_read_idx(uint4& v, uint32_t a) {
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(a) : "memory");
}
__device__ __forceinline__ void ps_read8(uint32_t (&x)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_u16 %0, %8\n\tds_read_u16 %1, %9\n\tds_read_u16 %2, %10\n\tds_read_u16 %3, %11\n\t"
      "ds_read_u16 %4, %12\n\tds_read_u16 %5, %13\n\tds_read_u16 %6, %14\n\tds_read_u16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

// SCATTER: out[t][perm[j]] = in[t][j] (no separate tail source);
// else out[t][j] = in[t][perm[j]], and TAILOUT also writes tail_out[t][j] for j >= tail0
template <bool SCATTER, bool TAILOUT>
__global__ __launch_bounds__(PS_THREADS) void permute_stream_kernel(PermArgs a, int spr) {
  __shared__ __align__(16) uint16_t P0[PS_E], P1[PS_E], P2[PS_E], P3[PS_E], P4[PS_E], P5[PS_E];
  __shared__ __align__(16) uint16_t IDX[PS_E];
  static_assert(PS_S == 6, "the ring is spelled out for six stages");
  constexpr int NS = TAILOUT ? 4 : 2;                       // stores per lane and iteration
  const int W = a.W, R = PS_E / W, cpr = W >> 3;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t t0 = (int64_t)blockIdx.x * spr * R;
  if (t0 >= a.N) return;
  const int rows = (int)min((int64_t)spr * R, a.N - t0);
  const int nt = (rows + R - 1) / R;                         // row groups of this run
  const uint32_t gbytes = (uint32_t)R * W * 2;               // bytes of one group

  // loads: slot h * 512 + tid of a stage = element 8 (h * 512 + tid), row / column of the
  // group; instruction h of wave w fills the KiB at element h * 4096 + w * 512
  const __amdgpu_buffer_rsrc_t rin = ps_rsrc(a.in + t0 * W, (uint32_t)rows * W * 2);
  int lo[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = (h * PS_THREADS + tid) * 8;
    lo[h] = e < R * W ? e * 2 : -1;
  }
  auto load_group = [&](int i, uint16_t* st) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      ps_b2l16(rin, lo[h] >= 0 ? lo[h] + (int)((uint32_t)i * gbytes) : PS_OOB, st + h * PS_THREADS * 8 + wave * 512);
  };
  // the first S - 1 groups, in issue order, while the index table is built
  load_group(0, P0);
  asm volatile("" ::: "memory");
  load_group(1, P1);
  asm volatile("" ::: "memory");
  load_group(2, P2);
  asm volatile("" ::: "memory");
  load_group(3, P3);
  asm volatile("" ::: "memory");
  load_group(4, P4);
  asm volatile("" ::: "memory");
  for (int j = tid; j < W; j += PS_THREADS) {
    const int p = a.perm[j];
    if (SCATTER) IDX[p] = (uint16_t)j;
    else IDX[j] = (uint16_t)p;
  }

  // stores: items m * 512 + tid of a group = (row, 8-column chunk)
  const __amdgpu_buffer_rsrc_t rout = ps_rsrc(a.out + t0 * W, (uint32_t)rows * W * 2);
  const __amdgpu_buffer_rsrc_t rtail = ps_rsrc(TAILOUT ? a.tail_out + t0 * W : a.out, TAILOUT ? (uint32_t)rows * W * 2 : 0u);
  int so[2], ro[2], io[2];
  bool tl[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int item = m * PS_THREADS + tid;
    const int r = item / cpr, c = item - r * cpr;
    const bool ok = r < R;
    so[m] = ok ? (r * W + c * 8) * 2 : -1;
    ro[m] = r * W * 2;                        // byte offset of the item's row in a stage
    io[m] = c * 16;                           // byte offset of its 8 indices
    tl[m] = ok && c * 8 >= a.tail0;
  }
  const uint32_t ibase = ps_lds_addr(IDX);

  auto step = [&](int i, const uint16_t* st, uint16_t* next) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();   // all parts of group i landed; the stage of group i - 1 is free
    asm volatile("" ::: "memory");
    load_group(i + PS_S - 1, next);
    const uint32_t sb = ps_lds_addr(st);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      ps_u32x4 v = {0u, 0u, 0u, 0u};
      if (so[m] >= 0) {
        uint4 ix;
        ps_read_idx(ix, ibase + (uint32_t)io[m]);
        const uint32_t rb = sb + (uint32_t)ro[m];
        const uint32_t ad[8] = {rb + 2 * (ix.x & 0xffff), rb + 2 * (ix.x >> 16), rb + 2 * (ix.y & 0xffff), rb + 2 * (ix.y >> 16),
                                rb + 2 * (ix.z & 0xffff), rb + 2 * (ix.z >> 16), rb + 2 * (ix.w & 0xffff), rb + 2 * (ix.w >> 16)};
        uint32_t x[8];
        ps_read8(x, ad);
        v = ps_u32x4{x[0] | (x[1] << 16), x[2] | (x[3] << 16), x[4] | (x[5] << 16), x[6] | (x[7] << 16)};
      }
      const int off = so[m] >= 0 ? so[m] + (int)((uint32_t)i * gbytes) : PS_OOB;
      __builtin_amdgcn_raw_buffer_store_b128(v, rout, off, 0, 0);
      if constexpr (TAILOUT) __builtin_amdgcn_raw_buffer_store_b128(v, rtail, tl[m] ? off : PS_OOB, 0, 0);
    }
  };
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // index table written

#define PS_WAIT(s)                                                                           \
  asm volatile("" ::: "memory");                                                             \
  if (i == 0) __builtin_amdgcn_s_waitcnt(ps_vm_imm(2 * (PS_S - 2) + (s) * NS));              \
  else __builtin_amdgcn_s_waitcnt(ps_vm_imm(2 * (PS_S - 2) + (PS_S - 1) * NS));
  for (int i = 0; i < nt; i += PS_S) {
    PS_WAIT(0) step(i, P0, P5);
    if (i + 1 >= nt) break;
    PS_WAIT(1) step(i + 1, P1, P0);
    if (i + 2 >= nt) break;
    PS_WAIT(2) step(i + 2, P2, P1);
    if (i + 3 >= nt) break;
    PS_WAIT(3) step(i + 3, P3, P2);
    if (i + 4 >= nt) break;
    PS_WAIT(4) step(i + 4, P4, P3);
    if (i + 5 >= nt) break;
    PS_WAIT(5) step(i + 5, P5, P4);
  }
#undef PS_WAIT
  // fills past the end of the run may still be writing this workgroup's LDS
  __builtin_amdgcn_s_waitcnt(ps_vm_imm(0));
}

// true if the streaming kernel took the permutation.  It takes rows of 4096
// to 8192 columns: measured on 8192 x 2048 and 8192 x 5632 bf16 matrices, it
// beats the staging kernel at 5632 (5.7 vs 5.3 TB/s) and loses at 2048
// (4.9 vs 5.4-5.8 TB/s), where a run of 32 rows is only 8 ring iterations.
static bool launch_permute_stream(bool gather, const PermArgs& a, hipStream_t s) {
  const int W = a.W;
  if (W < 4096 || W > PS_E || (W & 7)) return false;
  if (!a16(a.in) || !a16(a.out) || (a.tail_out && !a16(a.tail_out))) return false;
  const bool tail = a.tail0 < W;
  if (!gather && tail && a.tail_in && a.tail_in != a.in) return false;   // separate tail source: not streamed
  const int R = PS_E / W;
  const int64_t groups = (a.N + R - 1) / R;
  int64_t runs = groups < 256 ? groups : 256;
  int64_t spr = (groups + runs - 1) / runs;
  if ((spr + PS_S) * (int64_t)R * W * 2 >= 0x7fffffffLL) return false;
  runs = (groups + spr - 1) / spr;
  const dim3 grid((unsigned)runs);
  if (!gather) hipLaunchKernelGGL((permute_stream_kernel<true, false>), grid, dim3(PS_THREADS), 0, s, a, (int)spr);
  else if (tail && a.tail_out) hipLaunchKernelGGL((permute_stream_kernel<false, true>), grid, dim3(PS_THREADS), 0, s, a, (int)spr);
  else hipLaunchKernelGGL((permute_stream_kernel<false, false>), grid, dim3(PS_THREADS), 0, s, a, (int)spr);
  return true;
}

void launch_permute_bf16(bool gather, const PermArgs& a, hipStream_t s) {
  if (a.N <= 0 || a.W <= 0) return;
  if (launch_permute_stream(gather, a, s)) return;
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
