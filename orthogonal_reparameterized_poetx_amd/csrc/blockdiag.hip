// Block-diagonal products of token rows: the b x b Cayley blocks of the P and
// R sides applied to activations whose columns are already permuted, so that
// each block acts on b contiguous columns
// [P3 "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
// Transformation", Methodologie items 2 and 3].
//
//   out[t][l*B + i] = sum_kk in[t][l*B + kk] * q[l][i][kk]      (l < k, t < N)
//
// bf16 operands, fp32 accumulation on 32x32x16 MFMA, bf16 output.  The
// product reads and writes 2 bytes per element and does B/2 flops per byte,
// well under the chip's MFMA-to-HBM ratio, so the kernel is built to stream:
//  - one workgroup owns one block l and a contiguous run of 32-token tiles;
//    wave w keeps rows 32w..32w+31 of q[l] in VGPRs as MFMA operand fragments
//    for the whole run (q[l] is read once per workgroup);
//  - token tiles stream into a ring of BD_S LDS stages with buffer-to-LDS
//    loads (no VGPRs, one contiguous KiB per instruction), BD_S - 1 tiles in
//    flight;
//  - results go through an LDS staging tile and leave as whole-row 16-byte
//    buffer stores; rows past N fall outside the buffer range, so ragged tails
//    need no branches.
// Each iteration issues exactly two tile loads (past the end of the run they
// read nothing) and two stores per lane, in an order that compiler barriers
// fix; vector-memory operations complete in issue order, so a tile has landed
// once at most the operations issued after it are outstanding: a constant
// count from the eighth iteration on, and a smaller one in the first seven.
#include "common.h"
#include "kernels.h"
#include "ranges.h"

namespace poetx {

namespace {

constexpr int BD_T = 32;   // tokens per tile: the N dimension of the swapped MFMA
constexpr int BD_S = 7;    // LDS ring stages; the staging tile is an eighth buffer

template <int B>
struct Bd {
  static constexpr int NW = B / 32;        // waves: one per 32 output columns
  static constexpr int NT = NW * 64;       // threads (= 2 B)
  static constexpr int CPR = B / 8;        // 16-byte chunks per row
  static constexpr int CPRS = CPR < 16 ? CPR : 16;
  static constexpr int SH = CPRS == 16 ? 0 : (CPRS == 8 ? 1 : 2);
  static constexpr int TILE = BD_T * B;    // elements per tile, and per wave's rows of q
  static constexpr int KS = B / 16;        // MFMA k steps
  // vector-memory ops issued after the loads of tile i, at the wait of
  // iteration i: the loads of tiles i+1 .. i+S-2 and the stores of iterations
  // i-S+1 .. i-1 that exist (2 of each per lane)
  static constexpr int vm_after(int i) { return i < BD_S - 1 ? 2 * (BD_S - 2) + 2 * i : 4 * BD_S - 6; }
  static_assert(NW == 1 || NW == 2 || NW == 4 || NW == 8, "q is staged in NW of the LDS buffers");
};

// 16-byte chunk c of row r sits at chunk c ^ swz(r).  A 16-lane phase of a
// fragment read (16 consecutive rows, one logical chunk) and of a staging
// read (consecutive chunks of one or a few rows) then touches each of the 64
// banks once; with 2 B-byte rows, rows r and r + 16 share a bank pattern and
// are separated by the half swap of the staging writes.
template <int B>
__device__ __forceinline__ int swz(int r) {
  return (r >> Bd<B>::SH) & (Bd<B>::CPRS - 1);
}

__device__ __forceinline__ void b2l16(__amdgpu_buffer_rsrc_t r, int voff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void g2l16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// two floats -> packed bf16 pair (round to nearest even), a in the low half
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, bf16x2{(bf16)a, (bf16)b});
}
__device__ __forceinline__ void bst16(u32x4 v, __amdgpu_buffer_rsrc_t r, int voff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, 0);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// LDS accesses of the streaming loop, written as inline asm.  The compiler's
// wait insertion cannot tell which ring stage an asynchronous fill targets
// once several fills are in flight, and then waits for nearly all of them
// before every LDS read; these accesses are ordered by the explicit vmcnt
// wait and the barriers instead.  Each read block waits for its own results
// before it ends, and its outputs are early-clobber, so no in-flight read can
// land in a register that a later address of the block still needs.
__device__ __forceinline__ void lds_read8(i32x4 (&x)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\tds_read_b128 %3, %11\n\t"
      "ds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\tds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}
__device__ __forceinline__ void lds_read2(i32x4& x0, i32x4& x1, uint32_t a0, uint32_t a1) {
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(x0), "=&v"(x1)
               : "v"(a0), "v"(a1)
               : "memory");
}
__device__ __forceinline__ void lds_write8b(uint32_t a, uint2 v) {
  asm volatile("ds_write_b64 %0, %1" ::"v"(a), "v"(v) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8; the maximum of a field means "do not wait").  The
// builtin, unlike inline asm, is seen by the compiler's wait insertion, which
// then knows which asynchronous LDS fills have completed.
constexpr unsigned wait_imm(unsigned vm, unsigned lgkm) {
  return (vm & 15u) | ((vm >> 4) << 14) | (7u << 4) | (lgkm << 8);
}

// workgroup barrier for LDS traffic only: waits for this wave's LDS reads and
// writes, not for its outstanding global loads and stores (a release fence
// would also wait for every asynchronous global-to-LDS fill in flight)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace

template <int B>
// in and out may be the same matrix (the merge's in-place block product): a
// workgroup reads every element of its tiles before it writes them, and no
// two workgroups touch the same elements
__global__ __launch_bounds__(Bd<B>::NT) void blockdiag_kernel(const uint16_t* in, const uint16_t* __restrict__ q,
                                                             uint16_t* out, int64_t N, int64_t lda, int64_t ldc, int k,
                                                             int tpc) {
  using C = Bd<B>;
  // the ring and the staging tile as separate LDS objects, each named at
  // compile time, so that the compiler tells reads of one stage from the
  // asynchronous fill of another
  __shared__ __align__(16) uint16_t L0[C::TILE], L1[C::TILE], L2[C::TILE], L3[C::TILE], L4[C::TILE],
      L5[C::TILE], L6[C::TILE], ST[C::TILE];
  static_assert(BD_S == 7, "the ring is spelled out for seven stages");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = blockIdx.x % k;
  const int64_t t0 = (int64_t)(blockIdx.x / k) * tpc * BD_T;
  if (t0 >= N) return;
  const int rows = (int)min((int64_t)tpc * BD_T, N - t0);
  const int nt = (rows + BD_T - 1) / BD_T;
  const uint32_t ldab = (uint32_t)lda * 2, ldcb = (uint32_t)ldc * 2;

  // ---- q[l] -> VGPR fragments: rows 32 a .. 32 a + 31 go to LDS buffer a
  // (all waves fill every buffer, each buffer named statically), then wave w
  // reads its rows from buffer w
  bf16x8 qf[C::KS];
  {
    const __amdgpu_buffer_rsrc_t rq = rsrc(q + (int64_t)l * B * B, 2u * B * B);
    auto qload = [&](uint16_t* dst, int a) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = (h * C::NW + wave) * 64 + lane, r = c / C::CPR, p = c % C::CPR;
        b2l16(rq, ((32 * a + r) * B + ((p ^ swz<B>(r)) << 3)) * 2, dst + (h * C::NW + wave) * 512);
      }
    };
    qload(L0, 0);
    if constexpr (C::NW > 1) qload(L1, 1);
    if constexpr (C::NW > 2) { qload(L2, 2); qload(L3, 3); }
    if constexpr (C::NW > 4) { qload(L4, 4); qload(L5, 5); qload(L6, 6); qload(ST, 7); }
    __builtin_amdgcn_s_waitcnt(wait_imm(0, 15));
    lds_barrier();
    const uint16_t* qb = wave == 0 ? L0 : wave == 1 ? L1 : wave == 2 ? L2 : wave == 3 ? L3
                       : wave == 4 ? L4 : wave == 5 ? L5 : wave == 6 ? L6 : ST;
    const int r = lane & 31;
#pragma unroll
    for (int j = 0; j < C::KS; ++j)
      qf[j] = *reinterpret_cast<const bf16x8*>(qb + r * B + (((2 * j + (lane >> 5)) ^ swz<B>(r)) << 3));
  }
  lds_barrier();   // every wave holds its fragments; the buffers are free

  // ---- per-lane tile addressing
  // loads: instruction h of wave w fills KiB (h NW + w) of a stage; lane i
  // writes slot c = 64 (h NW + w) + i = row c / CPR, chunk c % CPR
  const BufRange gin = tile_range(t0, rows, (int64_t)l * B, B, lda, 2);
  const __amdgpu_buffer_rsrc_t rin = rsrc(in + gin.first, (uint32_t)gin.bytes);
  int voff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = (h * C::NW + wave) * 64 + lane, r = c / C::CPR, p = c % C::CPR;
    voff[h] = (int)((uint32_t)r * ldab + (uint32_t)((p ^ swz<B>(r)) << 4));
  }
  const uint32_t tin = (uint32_t)BD_T * ldab, tout = (uint32_t)BD_T * ldcb;
  // stores: thread tid writes chunks idx = h NT + tid = row idx / CPR, chunk idx % CPR
  const BufRange gout = tile_range(t0, rows, (int64_t)l * B, B, ldc, 2);
  const __amdgpu_buffer_rsrc_t rout = rsrc(out + gout.first, (uint32_t)gout.bytes);
  int soff[2], sl[2];
  bool sw[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int idx = h * C::NT + tid, r = idx / C::CPR, p = idx % C::CPR;
    soff[h] = (int)((uint32_t)r * ldcb + (uint32_t)(p << 4));
    sl[h] = r * B + ((p ^ swz<B>(r)) << 3);
    sw[h] = (r >> 4) & 1;
  }

  auto load_tile = [&](int i, uint16_t* stage) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      b2l16(rin, voff[h] + (int)((uint32_t)i * tin), stage + (h * C::NW + wave) * 512);
  };

  // fragment-read byte offsets within a stage, shared by all stages (the
  // stage base folds into the instruction's immediate offset)
  const int r32 = lane & 31, hl = lane >> 5;
  int xoff[C::KS];
#pragma unroll
  for (int j = 0; j < C::KS; ++j) xoff[j] = r32 * (2 * B) + (((2 * j + hl) ^ swz<B>(r32)) << 4);
  // staging-tile byte offsets: the four 8-byte writes of this lane and the
  // two 16-byte reads of this thread
  uint32_t wst[4];
#pragma unroll
  for (int g = 0; g < 4; ++g)
    wst[g] = lds_addr(ST) + 2u * (r32 * B + (((4 * wave + g) ^ swz<B>(r32)) << 3) + ((hl ^ ((r32 >> 4) & 1)) << 2));
  const uint32_t rst0 = lds_addr(ST) + 2u * sl[0], rst1 = lds_addr(ST) + 2u * sl[1];

  // the wait for tile i comes first: this lane's part of tile i has landed
  auto step = [&](int i, const uint16_t* stage, uint16_t* next) {
    lds_barrier();   // all parts landed; stage of tile i - 1 and the staging tile are free
    load_tile(i + BD_S - 1, next);
    i32x4 xf[C::KS];
    const uint32_t sb = lds_addr(stage);
#pragma unroll
    for (int j0 = 0; j0 < C::KS; j0 += 8) {
      if constexpr (C::KS >= 8) {
        uint32_t a[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] = sb + (uint32_t)xoff[j0 + j];
        lds_read8(*reinterpret_cast<i32x4(*)[8]>(&xf[j0]), a);
      }
    }
    if constexpr (C::KS == 4) {
      lds_read2(xf[0], xf[1], sb + (uint32_t)xoff[0], sb + (uint32_t)xoff[1]);
      lds_read2(xf[2], xf[3], sb + (uint32_t)xoff[2], sb + (uint32_t)xoff[3]);
    } else if constexpr (C::KS == 2) {
      lds_read2(xf[0], xf[1], sb + (uint32_t)xoff[0], sb + (uint32_t)xoff[1]);
    }
    f32x16 acc = {};
#pragma unroll
    for (int j = 0; j < C::KS; ++j) acc = mfma32(qf[j], __builtin_bit_cast(bf16x8, xf[j]), acc);
    // acc register 4 g + e of lane l is out[token l % 32][col 32 w + 8 g + 4 (l / 32) + e]
#pragma unroll
    for (int g = 0; g < 4; ++g)
      lds_write8b(wst[g], uint2{pk_bf16(acc[4 * g], acc[4 * g + 1]), pk_bf16(acc[4 * g + 2], acc[4 * g + 3])});
    lds_barrier();
    i32x4 v0, v1;
    lds_read2(v0, v1, rst0, rst1);
    bst16(__builtin_bit_cast(u32x4, sw[0] ? v0.zwxy : v0), rout, soff[0] + (int)((uint32_t)i * tout));
    bst16(__builtin_bit_cast(u32x4, sw[1] ? v1.zwxy : v1), rout, soff[1] + (int)((uint32_t)i * tout));
  };

  // the first S - 1 tiles, in issue order
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
  // vm(s): wait for the tile of ring position s, in the first pass over the
  // ring (the prologue's loads have no stores between them) or a later one
#define BD_WAIT(s)                                                          \
  asm volatile("" ::: "memory");                                           \
  if (i == 0) __builtin_amdgcn_s_waitcnt(wait_imm(C::vm_after(s), 15));    \
  else __builtin_amdgcn_s_waitcnt(wait_imm(C::vm_after(BD_S), 15));
  for (int i = 0; i < nt; i += BD_S) {
    BD_WAIT(0) step(i, L0, L6);
    if (i + 1 >= nt) break;
    BD_WAIT(1) step(i + 1, L1, L0);
    if (i + 2 >= nt) break;
    BD_WAIT(2) step(i + 2, L2, L1);
    if (i + 3 >= nt) break;
    BD_WAIT(3) step(i + 3, L3, L2);
    if (i + 4 >= nt) break;
    BD_WAIT(4) step(i + 4, L4, L3);
    if (i + 5 >= nt) break;
    BD_WAIT(5) step(i + 5, L5, L4);
    if (i + 6 >= nt) break;
    BD_WAIT(6) step(i + 6, L6, L5);
  }
#undef BD_WAIT
  // fills past the end of the run may still be writing this workgroup's LDS
  __builtin_amdgcn_s_waitcnt(wait_imm(0, 15));
}

// Launch plan: grid = k blocks x C token runs, C sized so that the grid is
// about one wave of workgroups over the 256 CUs at the occupancy the LDS
// footprint allows.  Returns false (nothing launched) where the kernel does
// not apply: b outside {32, 64, 128, 256}, rows not 16-byte aligned, or
// operands too large for 32-bit buffer offsets.
bool launch_blockdiag_bf16(const uint16_t* in, const uint16_t* q, uint16_t* out, int64_t N, int64_t lda,
                           int64_t ldc, int b, int k, hipStream_t s) {
  if (b != 32 && b != 64 && b != 128 && b != 256) return false;
  if (N <= 0 || k <= 0) return true;
  if ((lda & 7) || (ldc & 7) || (reinterpret_cast<uintptr_t>(in) & 15) || (reinterpret_cast<uintptr_t>(out) & 15) ||
      (reinterpret_cast<uintptr_t>(q) & 15))
    return false;
  static_assert(BD_T == BDIAG_T && BD_S == BDIAG_STAGES, "ranges.h mirrors the tiling");
  const BdiagRuns br = blockdiag_runs(N, lda, ldc, b, k);
  if (br.runs < 1) return false;
  const int64_t runs = br.runs, tpc = br.tpc;
  const int64_t grid = runs * k;
  if (grid > 0x7fffffffLL) return false;
  switch (b) {
    case 32: hipLaunchKernelGGL(blockdiag_kernel<32>, dim3((unsigned)grid), dim3(64), 0, s, in, q, out, N, lda, ldc, k, (int)tpc); break;
    case 64: hipLaunchKernelGGL(blockdiag_kernel<64>, dim3((unsigned)grid), dim3(128), 0, s, in, q, out, N, lda, ldc, k, (int)tpc); break;
    case 128: hipLaunchKernelGGL(blockdiag_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, in, q, out, N, lda, ldc, k, (int)tpc); break;
    default: hipLaunchKernelGGL(blockdiag_kernel<256>, dim3((unsigned)grid), dim3(512), 0, s, in, q, out, N, lda, ldc, k, (int)tpc); break;
  }
  return true;
}


}  // namespace poetx
