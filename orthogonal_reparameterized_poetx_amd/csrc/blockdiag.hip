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

// b = 256 with the two halves of the workgroup out of phase.  Waves 0-3 own
// output columns 0-127 of the block, waves 4-7 columns 128-255; every wave
// alternates a memory phase (refill a ring stage, store its half of the
// previous tile from its staging half, read the tile's fragments) and a
// compute phase (16 MFMAs, results to its staging half), with a workgroup
// barrier between phases, and waves 4-7 run one phase behind waves 0-3, so
// one half issues MFMAs while the other works on LDS (in blockdiag_kernel
// every wave does both in the same phase, so the two costs add).  Tile i must
// have landed before waves 0-3 read it: waves 0-3 wait for their part of it
// before their memory phase, waves 4-7 before their compute phase of tile
// i - 1, both at the barrier that opens that read.
namespace {
constexpr int PP_S = BDIAG_PP_STAGES;   // ring stages (the staging tile is one more buffer)
// vector-memory operations a wave has issued after its loads of tile j when
// it waits for them: the prologue loads tiles 0 .. S-2; memory phase m loads
// tile m + S - 1 and (m >= 1) stores tile m - 1, two operations each
constexpr int pp_vm(int j) {
  return j == 0 ? 2 * (PP_S - 2) : j < PP_S - 1 ? 2 * PP_S - 6 + 2 * j : j == PP_S - 1 ? 4 * (PP_S - 2) : 4 * PP_S - 6;
}
static_assert(pp_vm(PP_S) < 64, "vmcnt field");
}  // namespace

__global__ __launch_bounds__(512) void blockdiag_pp_kernel(const uint16_t* in, const uint16_t* __restrict__ q,
                                                           uint16_t* out, int64_t N, int64_t lda, int64_t ldc, int k,
                                                           int tpc) {
  constexpr int B = 256;
  using C = Bd<B>;
  // the seven ring stages, then the staging tile (every access in the loop is
  // an explicit LDS instruction, so the stages need no names of their own)
  __shared__ __align__(16) uint16_t RING[(PP_S + 1) * C::TILE];
  uint16_t* const ST = RING + PP_S * C::TILE;
  static_assert(C::NW == 8 && (PP_S + 1) * C::TILE * 2 <= 160 * 1024, "eight waves; the LDS holds the ring");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wg = wave & 3;
  const int l = blockIdx.x % k;
  const int64_t t0 = (int64_t)(blockIdx.x / k) * tpc * BD_T;
  if (t0 >= N) return;
  const int rows = (int)min((int64_t)tpc * BD_T, N - t0);
  const int nt = (rows + BD_T - 1) / BD_T;
  const uint32_t ldab = (uint32_t)lda * 2, ldcb = (uint32_t)ldc * 2;

  // ---- q[l] -> VGPR fragments (as in blockdiag_kernel)
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
#pragma unroll
    for (int a = 0; a < 8; ++a) qload(RING + a * C::TILE, a);
    __builtin_amdgcn_s_waitcnt(wait_imm(0, 15));
    lds_barrier();
    const uint16_t* qb = RING + wave * C::TILE;
    const int r = lane & 31;
#pragma unroll
    for (int j = 0; j < C::KS; ++j)
      qf[j] = *reinterpret_cast<const bf16x8*>(qb + r * B + (((2 * j + (lane >> 5)) ^ swz<B>(r)) << 3));
  }
  lds_barrier();

  // ---- tile loads (as in blockdiag_kernel)
  const BufRange gin = tile_range(t0, rows, (int64_t)l * B, B, lda, 2);
  const __amdgpu_buffer_rsrc_t rin = rsrc(in + gin.first, (uint32_t)gin.bytes);
  int voff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = (h * C::NW + wave) * 64 + lane, r = c / C::CPR, p = c % C::CPR;
    voff[h] = (int)((uint32_t)r * ldab + (uint32_t)((p ^ swz<B>(r)) << 4));
  }
  const uint32_t tin = (uint32_t)BD_T * ldab, tout = (uint32_t)BD_T * ldcb;
  auto load_tile = [&](int i, uint16_t* stage) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      b2l16(rin, voff[h] + (int)((uint32_t)i * tin), stage + (h * C::NW + wave) * 512);
  };
  const int r32 = lane & 31, hl = lane >> 5;
  // fragment j of this lane: row r32, 16-byte chunk 2 j + hl (swizzled)
  const uint32_t xrow = (uint32_t)(r32 * (2 * B)), xsw = (uint32_t)swz<B>(r32);

  // ---- staging: half grp of ST holds this half's 32 x 128 results, rows of
  // 256 bytes, 16-byte chunk c of row r at c ^ (r & 15)
  const uint32_t stb = lds_addr(ST) + (uint32_t)grp * 8192u;
  uint32_t wst[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) wst[g] = stb + (uint32_t)(r32 * 256 + (((4 * wg + g) ^ (r32 & 15)) << 4) + (hl << 3));
  // stores: thread t of the half writes row t / 8, chunks t % 8 and 8 + t % 8
  const BufRange gout = tile_range(t0, rows, (int64_t)l * B, B, ldc, 2);
  const __amdgpu_buffer_rsrc_t rout = rsrc(out + gout.first, (uint32_t)gout.bytes);
  const int tg = tid & 255, sr = tg >> 3;
  uint32_t rst[2];
  int sof[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int cc = 8 * h + (tg & 7);
    rst[h] = stb + (uint32_t)(sr * 256 + ((cc ^ (sr & 15)) << 4));
    sof[h] = (int)((uint32_t)sr * ldcb + (uint32_t)((128 * grp + 8 * cc) * 2));
  }
  auto store_prev = [&](int i) {   // this half of tile i from staging
    i32x4 v0, v1;
    lds_read2(v0, v1, rst[0], rst[1]);
    bst16(__builtin_bit_cast(u32x4, v0), rout, sof[0] + (int)((uint32_t)i * tout));
    bst16(__builtin_bit_cast(u32x4, v1), rout, sof[1] + (int)((uint32_t)i * tout));
  };

  f32x16 acc;
  i32x4 xf[C::KS];
  // memory phase of tile i (ring stage `stage`; `next` held tile i - 1)
  auto mem = [&](int i, const uint16_t* stage, uint16_t* next) {
    load_tile(i + PP_S - 1, next);
    if (i > 0) store_prev(i - 1);
    const uint32_t sb = lds_addr(stage) + xrow;
    uint32_t a[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = sb + ((((uint32_t)(2 * j + hl)) ^ xsw) << 4);
    lds_read8(*reinterpret_cast<i32x4(*)[8]>(&xf[0]), a);
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = sb + ((((uint32_t)(2 * (8 + j) + hl)) ^ xsw) << 4);
    lds_read8(*reinterpret_cast<i32x4(*)[8]>(&xf[8]), a);
  };
  auto mma = [&]() {
    acc = f32x16{};
#pragma unroll
    for (int j = 0; j < C::KS; ++j) acc = mfma32(qf[j], __builtin_bit_cast(bf16x8, xf[j]), acc);
    // acc register 4 g + e of lane l is out[token l % 32][col 32 w + 8 g + 4 (l / 32) + e]
#pragma unroll
    for (int g = 0; g < 4; ++g)
      lds_write8b(wst[g], uint2{pk_bf16(acc[4 * g], acc[4 * g + 1]), pk_bf16(acc[4 * g + 2], acc[4 * g + 3])});
  };

#pragma unroll
  for (int t = 0; t < PP_S - 1; ++t) {
    load_tile(t, RING + t * C::TILE);
    asm volatile("" ::: "memory");
  }
  if (grp == 1) {
    // tile 0 must be complete at the barrier that opens waves 0-3's first read
    __builtin_amdgcn_s_waitcnt(wait_imm(pp_vm(0), 15));
    lds_barrier();
  }
  // wait (immediate count) for this wave's loads of tile j
  auto wait_tile = [](int j) {
    switch (j) {
      case 0: __builtin_amdgcn_s_waitcnt(wait_imm(pp_vm(0), 15)); break;
      case 1: __builtin_amdgcn_s_waitcnt(wait_imm(pp_vm(1), 15)); break;
      case 2: __builtin_amdgcn_s_waitcnt(wait_imm(pp_vm(2), 15)); break;
      case 3: __builtin_amdgcn_s_waitcnt(wait_imm(pp_vm(3), 15)); break;
      case 4: __builtin_amdgcn_s_waitcnt(wait_imm(pp_vm(4), 15)); break;
      case 5: __builtin_amdgcn_s_waitcnt(wait_imm(pp_vm(5), 15)); break;
      case 6: __builtin_amdgcn_s_waitcnt(wait_imm(pp_vm(6), 15)); break;
      case 7: __builtin_amdgcn_s_waitcnt(wait_imm(pp_vm(7), 15)); break;
      case 8: __builtin_amdgcn_s_waitcnt(wait_imm(pp_vm(8), 15)); break;
      default: __builtin_amdgcn_s_waitcnt(wait_imm(pp_vm(PP_S), 15)); break;
    }
  };
  static_assert(PP_S <= 9, "wait_tile spells out the first pass for up to nine stages");
  // tile i: the memory phase, then the compute phase, each opened by a barrier
  int cs = 0, ns = PP_S - 1;   // ring stages of tile i and of tile i - 1
  for (int i = 0; i < nt; ++i) {
    asm volatile("" ::: "memory");
    if (grp == 0) wait_tile(i);
    lds_barrier();
    mem(i, RING + cs * C::TILE, RING + ns * C::TILE);
    asm volatile("" ::: "memory");
    if (grp == 1) wait_tile(i + 1);
    lds_barrier();
    mma();
    ns = cs;
    cs = cs == PP_S - 1 ? 0 : cs + 1;
  }
  // the last tile: each half stores its staging after a barrier; waves 0-3
  // take one more barrier so that both halves pass the same number
  lds_barrier();
  store_prev(nt - 1);
  if (grp == 0) lds_barrier();
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
    default: hipLaunchKernelGGL(blockdiag_pp_kernel, dim3((unsigned)grid), dim3(512), 0, s, in, q, out, N, lda, ldc, k, (int)tpc); break;
  }
  return true;
}


// ---------------------------------------------------------------------------
// Row gather and block product in one pass (the gather-in side: P forward,
// its recompute, R backward), b = 256 and rows of at most 2048 columns:
//   out[t][l*256 + i] = sum_kk q[l][i][kk] * in[t][perm[l*256 + kk]]   (l < k)
//   emit[t][l*256 + kk] = in[t][perm[l*256 + kk]]                      (optional)
// One workgroup per (block l, token run), the block in VGPRs as in
// blockdiag_kernel.  The gather needs b columns spread over the whole row, so
// the run's tiles of 16 whole token rows are loaded (contiguous 16-byte loads
// into registers, three tiles ahead) and written to one of two LDS stages,
// and the block's columns are picked from there through the permutation into
// a contiguous 16 x 256 tile that the MFMAs (16x16x32) read.  Every block of a
// run reads the same rows: the k workgroups of a run sit on one XCD
// (blockIdx mod 8), so the rows come from HBM once and from L2 for the
// others, and each workgroup touches the rows of the tile GB_PF beyond its
// loads with one 4-byte load per 128-byte line, so that they are in L2 when
// loaded.  Against a permutation pass and a block-product pass, the permuted
// rows are neither written nor read back (with emit they are written once,
// for a later Gram product).  Each tile costs about 2 us whatever the width,
// so with 8 blocks per row the two streaming passes are faster; the kernel is
// used up to 6 blocks per row.
// ---------------------------------------------------------------------------
namespace {
constexpr int GB_T = 16;                 // tokens per tile
constexpr int GB_B = 256;                // block size
constexpr int GB_MAXW = 2048;            // widest row the kernel takes (16 rows fill a 64 KiB stage)
constexpr int GB_MAXK = 6;               // widest row it is used for: 6 blocks (see gather_blockdiag_applies)
constexpr int GB_PF = 3;                 // tiles of L2 prefetch ahead of staging

__device__ __forceinline__ void b2l4(__amdgpu_buffer_rsrc_t r, int voff, int soff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 4, voff, soff, 0, 0);
}
__device__ __forceinline__ void b2l16s(__amdgpu_buffer_rsrc_t r, int voff, int soff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, voff, soff, 0, 0);
}
// eight 2-byte LDS reads at independent addresses, packed in pairs (the first
// of a pair in the low half)
__device__ __forceinline__ u32x4 lds_gather8(const uint32_t (&a)[8]) {
  uint32_t v[8];
  asm volatile(
      "ds_read_u16 %0, %8\n\tds_read_u16 %1, %9\n\tds_read_u16 %2, %10\n\tds_read_u16 %3, %11\n\t"
      "ds_read_u16 %4, %12\n\tds_read_u16 %5, %13\n\tds_read_u16 %6, %14\n\tds_read_u16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
  return u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
}
__device__ __forceinline__ void lds_write16(uint32_t a, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(v) : "memory");
}
__device__ __forceinline__ u32x4 lds_read16(uint32_t a) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(a) : "memory");
  return v;
}
}  // namespace

// NOPS = W / 256: 16-byte row loads per thread per tile
template <bool EMIT, int NOPS>
__global__ __launch_bounds__(512) void gather_blockdiag_kernel(GatherBdArgs a) {
  // the two row stages, each named at compile time (see blockdiag_kernel)
  __shared__ __align__(16) uint16_t R0[GB_T * GB_MAXW], R1[GB_T * GB_MAXW];
  __shared__ __align__(16) uint16_t XT[GB_T * GB_B], OT[GB_T * GB_B];
  __shared__ __align__(16) uint32_t PD[512];   // sink of the prefetch loads (never read)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k = a.k, W = a.W;
  // workgroup g runs on XCD g % 8; the k blocks of a run share an XCD
  const int g = blockIdx.x, j = g >> 3;
  const int l = j % k, run = (g & 7) + 8 * (j / k);
  if (run >= a.runs) return;
  const int64_t t0 = (int64_t)run * a.tpr * GB_T;
  if (t0 >= a.N) return;
  const int rows = (int)min((int64_t)a.tpr * GB_T, a.N - t0);
  const int nt = (rows + GB_T - 1) / GB_T;

  // ---- q[l] -> LDS (rows 0..127 in R0, 128..255 in R1; 16-byte chunk c of
  // row r at c ^ (r & 15)), then wave w takes rows 32 w .. 32 w + 31 as
  // 16x16x32 A fragments: qf[mt][ks] = rows 32 w + 16 mt + lane % 16,
  // k = 32 ks + 8 (lane / 16) .. + 7
  bf16x8 qf[2][8];
  {
    const __amdgpu_buffer_rsrc_t rq = rsrc(a.q + (int64_t)l * GB_B * GB_B, 2u * GB_B * GB_B);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const int slot = c * 512 + tid, r = slot >> 5, p = slot & 31;
      uint16_t* dst = (c < 8 ? R0 : R1) + ((c & 7) * 512 + wave * 64) * 8;
      b2l16s(rq, (r * GB_B + ((p ^ (r & 15)) << 3)) * 2, 0, dst);
    }
    __builtin_amdgcn_s_waitcnt(wait_imm(0, 15));
    lds_barrier();
    const int r0 = 32 * wave + (lane & 15);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int r = r0 + 16 * mt;
      const uint16_t* base = (r < 128 ? R0 : R1) + (r & 127) * GB_B;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        qf[mt][ks] = *reinterpret_cast<const bf16x8*>(base + (((4 * ks + (lane >> 4)) ^ (lane & 15)) << 3));
    }
    lds_barrier();   // the stages are free
  }

  // ---- this thread's gather: token row t = tid / 32 of a tile, block columns
  // kk = 8 kg .. 8 kg + 7 (kg = tid % 32), from row columns perm[l*256 + kk]
  const int gt = tid >> 5, kg = tid & 31;
  uint32_t gof[8];
  {
    const int4* pp = reinterpret_cast<const int4*>(a.perm + (int64_t)l * GB_B + 8 * kg);
    const int4 p0 = pp[0], p1 = pp[1];
    const int pc[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) gof[e] = (uint32_t)(gt * W + pc[e]) * 2u;
  }
  const uint32_t xw = lds_addr(XT) + (uint32_t)(gt * 512 + ((kg ^ (gt & 15)) << 4));
  // fragment reads of the x' tile: token lane % 16, chunk 4 ks + lane / 16
  uint32_t xra[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    xra[ks] = lds_addr(XT) + (uint32_t)((lane & 15) * 512 + (((4 * ks + (lane >> 4)) ^ (lane & 15)) << 4));
  // output staging: lane writes out[token lane % 16][32 w + 16 mt + 4 (lane / 16) .. + 3]
  uint32_t ow[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int c = 4 * wave + 2 * mt + (lane >> 5), h = (lane >> 4) & 1;
    ow[mt] = lds_addr(OT) + (uint32_t)((lane & 15) * 512 + ((c ^ (lane & 15)) << 4) + (h << 3));
  }
  const uint32_t orr = lds_addr(OT) + (uint32_t)(gt * 512 + ((kg ^ (gt & 15)) << 4));

  // ---- global ranges and per-lane offsets
  const BufRange gin = tile_range(t0, rows, 0, W, a.lda, 2);
  const __amdgpu_buffer_rsrc_t rin = rsrc(a.in + gin.first, (uint32_t)gin.bytes);
  const BufRange gout = tile_range(t0, rows, (int64_t)l * GB_B, GB_B, a.ldc, 2);
  const __amdgpu_buffer_rsrc_t rout = rsrc(a.out + gout.first, (uint32_t)gout.bytes);
  __amdgpu_buffer_rsrc_t remit = rout;
  if constexpr (EMIT) {
    const BufRange ge = tile_range(t0, rows, (int64_t)l * GB_B, GB_B, a.lde, 2);
    remit = rsrc(a.emit + ge.first, (uint32_t)ge.bytes);
  }
  const int cpr = W >> 3;                  // 16-byte chunks per row
  int voff[NOPS];
#pragma unroll
  for (int op = 0; op < NOPS; ++op) {
    const int c = op * 512 + tid, r = c / cpr, p = c - r * cpr;
    voff[op] = (int)((uint32_t)r * (uint32_t)a.lda * 2u + (uint32_t)(p << 4));
  }
  // prefetch: lane tid touches 128-byte line tid of the tile's rows (lines past
  // the tile repeat its last one)
  int pvoff;
  {
    const int lpr = W >> 6, lines = GB_T * lpr;
    const int L = tid < lines ? tid : lines - 1, r = L / lpr;
    pvoff = (int)((uint32_t)r * (uint32_t)a.lda * 2u + (uint32_t)((L - r * lpr) << 7));
  }
  const uint32_t tin = (uint32_t)GB_T * (uint32_t)a.lda * 2u;
  const int soutv = gt * (int)a.ldc * 2 + kg * 16;
  const int semit = EMIT ? gt * (int)a.lde * 2 + kg * 16 : 0;
  const uint32_t tout = (uint32_t)GB_T * (uint32_t)a.ldc * 2u, temit = EMIT ? (uint32_t)GB_T * (uint32_t)a.lde * 2u : 0u;

  // tile rows travel through registers: tile j is loaded into register set
  // j % 2 three steps ahead, written to LDS stage j % 2 one step ahead, and
  // gathered in step j, so two tiles are in flight from memory while one is
  // gathered (the LDS alone holds only two tiles of 2048-column rows)
  typedef u32x4 RowSet[NOPS];
  RowSet V0, V1;
  auto vload = [&](int i, RowSet& v) {
#pragma unroll
    for (int op = 0; op < NOPS; ++op)
      v[op] = __builtin_amdgcn_raw_buffer_load_b128(rin, voff[op], (int)((uint32_t)i * tin), 0);
  };
  const uint32_t vsl = (uint32_t)tid * 16u;
  auto vstore = [&](const RowSet& v, uint16_t* st) {
    const uint32_t sb = lds_addr(st) + vsl;
#pragma unroll
    for (int op = 0; op < NOPS; ++op) lds_write16(sb + (uint32_t)op * 8192u, v[op]);
  };
  auto prefetch = [&](int i) { b2l4(rin, pvoff, (int)((uint32_t)i * tin), PD + wave * 64); };

  // prologue: tiles 0..2 into registers (tile 0 on to stage 0), L2 prefetch
  // of tiles 3 .. 2 + GB_PF
  vload(0, V0);
  vload(1, V1);
#pragma unroll
  for (int i = 3; i < 3 + GB_PF; ++i) prefetch(i);
  vstore(V0, R0);
  vload(2, V0);

  // step i: tile i in stage cur; register set vn holds tile i + 1
  auto step = [&](int i, const uint16_t* cur, uint16_t* nxt, RowSet& vn) {
    lds_barrier();                      // tile i staged; x' and output tiles free
    prefetch(i + 3 + GB_PF);            // past the run: reads nothing
    uint32_t ad[8];
    const uint32_t cb = lds_addr(cur);
#pragma unroll
    for (int e = 0; e < 8; ++e) ad[e] = cb + gof[e];
    const u32x4 xv = lds_gather8(ad);
    lds_write16(xw, xv);
    if constexpr (EMIT)
      __builtin_amdgcn_raw_buffer_store_b128(xv, remit, semit + (int)((uint32_t)i * temit), 0, 0);
    vstore(vn, nxt);                    // tile i + 1; stage nxt held tile i - 1, gathered before the barrier
    vload(i + 3, vn);
    lds_barrier();                      // x' tile complete
    // the eight k steps' fragments in one block of reads (one LDS round trip)
    i32x4 xf[8];
    lds_read8(xf, xra);
    f32x4 acc[2] = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      acc[0] = mfma16(qf[0][ks], __builtin_bit_cast(bf16x8, xf[ks]), acc[0]);
      acc[1] = mfma16(qf[1][ks], __builtin_bit_cast(bf16x8, xf[ks]), acc[1]);
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      lds_write8b(ow[mt], uint2{pk_bf16(acc[mt][0], acc[mt][1]), pk_bf16(acc[mt][2], acc[mt][3])});
    lds_barrier();                      // output tile complete
    const u32x4 ov = lds_read16(orr);
    bst16(ov, rout, soutv + (int)((uint32_t)i * tout));
  };
  int i = 0;
  for (; i + 2 <= nt; i += 2) {
    step(i, R0, R1, V1);
    step(i + 1, R1, R0, V0);
  }
  if (i < nt) step(i, R0, R1, V1);
  // prefetches past the run may still be writing LDS
  __builtin_amdgcn_s_waitcnt(wait_imm(0, 15));
}

// Launch plan: runs of whole 16-token tiles, about 256 workgroups, at least 4
// tiles per run.  The launch returns false (nothing launched) where the
// kernel does not apply: b != 256, W = k b above 2048, unaligned rows or
// operands, offsets past 32 bits.
namespace {
struct GbPlan { int64_t runs, tpr; };
GbPlan gather_blockdiag_plan(int64_t N, int k) {
  const int64_t ntiles = (N + GB_T - 1) / GB_T;
  int64_t runs = 256 / k;
  if (runs > ntiles / 4) runs = ntiles / 4;
  runs = runs / 8 * 8;
  if (runs < 8) runs = 8;
  if (runs > ntiles) runs = ntiles;
  const int64_t tpr = (ntiles + runs - 1) / runs;
  return GbPlan{(ntiles + tpr - 1) / tpr, tpr};
}
}  // namespace

bool gather_blockdiag_applies(const void* in, const int32_t* perm, const void* q, const void* out, const void* emit,
                              int64_t N, int W, int b, int k, int64_t lda, int64_t ldc, int64_t lde) {
  // measured against the permutation + block-product passes (8192 tokens):
  // 7.1 vs 11.2 us at 256 columns, 15.0 vs 24.8 at 1024, 23.4 vs 26.7 at
  // 1536, 32.3 vs 30.5 at 2048; so up to 6 blocks per row
  if (b != GB_B || k <= 0 || k > GB_MAXK || W != k * GB_B || N <= 0) return false;
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  if ((lda & 7) || (ldc & 7) || (emit && (lde & 7)) || !al16(in) || !al16(out) || !al16(q) || (emit && !al16(emit)) ||
      !al16(perm))
    return false;
  // every per-lane offset, with the row loads and prefetches up to GB_PF + 3
  // tiles past a run, below 2^31
  const GbPlan p = gather_blockdiag_plan(N, k);
  const int64_t ld = std::max(lda, std::max(ldc, emit ? lde : (int64_t)0));
  return (p.tpr + GB_PF + 4) * GB_T * ld * 2 < 0x7fffffffLL;
}

bool launch_gather_blockdiag_bf16(const uint16_t* in, const int32_t* perm, const uint16_t* q, uint16_t* out,
                                  uint16_t* emit, int64_t N, int W, int b, int k, int64_t lda, int64_t ldc,
                                  int64_t lde, hipStream_t s) {
  if (!gather_blockdiag_applies(in, perm, q, out, emit, N, W, b, k, lda, ldc, lde)) return false;
  const GbPlan p = gather_blockdiag_plan(N, k);
  const int64_t runs = p.runs, tpr = p.tpr;
  GatherBdArgs a{};
  a.in = in; a.perm = perm; a.q = q; a.out = out; a.emit = emit;
  a.N = N; a.W = W; a.k = k; a.runs = (int)runs; a.tpr = (int)tpr;
  a.lda = lda; a.ldc = ldc; a.lde = lde;
  const int64_t grid = 8 * (int64_t)k * ((runs + 7) / 8);
  auto go = [&](auto em, auto nops) {
    hipLaunchKernelGGL((gather_blockdiag_kernel<decltype(em)::value, decltype(nops)::value>), dim3((unsigned)grid),
                       dim3(512), 0, s, a);
  };
  auto by_k = [&](auto em) {
    switch (k) {
      case 1: go(em, std::integral_constant<int, 1>{}); break;
      case 2: go(em, std::integral_constant<int, 2>{}); break;
      case 3: go(em, std::integral_constant<int, 3>{}); break;
      case 4: go(em, std::integral_constant<int, 4>{}); break;
      case 5: go(em, std::integral_constant<int, 5>{}); break;
      case 6: go(em, std::integral_constant<int, 6>{}); break;
      case 7: go(em, std::integral_constant<int, 7>{}); break;
      default: go(em, std::integral_constant<int, 8>{}); break;
    }
  };
  if (emit) by_k(std::true_type{});
  else by_k(std::false_type{});
  return true;
}

}  // namespace poetx
