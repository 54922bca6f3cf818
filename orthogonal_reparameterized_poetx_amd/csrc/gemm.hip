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

// 16-byte global -> LDS copy that bypasses the VGPRs: lane i of the wave
// writes lds_base + 16 i (lds_base must be wave-uniform).  Streaming tiles this
// way, one contiguous KiB per instruction, reaches several times the L2
// bandwidth of register loads in MFMA-fragment order.
__device__ __forceinline__ void g2l16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Buffer resource over [base, base + bytes): loads past the end read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int nrec = (int)(bytes < 0x7fffffff ? (bytes > 0 ? bytes : 0) : 0x7fffffff);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nrec, 0x00020000);
}
// 16-byte buffer load straight into LDS: lane i writes lds_base + 16 i
__device__ __forceinline__ void b2l16(__amdgpu_buffer_rsrc_t r, int voff, int soff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, voff, soff, 0, 0);
}

// LDS tile layouts (bf16, 16-byte chunks XOR-swizzled by row):
//   A (and NT B): [256 rows][64 k], chunk c of row r stored at chunk c ^ ((r >> 1) & 7):
//     a 16-lane phase of a fragment read (16 consecutive rows, one chunk)
//     then touches every bank once (rows r, r+1 differ in the bank half,
//     the key spreads the 8 row pairs over the 8 chunk positions)
//   NN B:         [64 k rows][256 n], chunk c of row r stored at chunk c ^ (r & 7)
// The direct loads pick each lane's source chunk so that the fixed lane ->
// LDS slot placement produces exactly this layout.
// BATCHED only names the instantiation used for batched block products, so
// that profiles tell it apart from the weight products.  OUTF32 writes the
// fp32 accumulators to g.Cf instead of bf16 to g.C.
template <bool NN, bool BATCHED, bool OUTF32 = false>
__global__ __launch_bounds__(512) void gemm_bf16_kernel(GemmArgs g, int tiles_m, int tiles_n, int ntiles) {
  // two buffers as separate LDS objects, each named at compile time below, so
  // the compiler can tell reads of one from the asynchronous fill of the other
  __shared__ __align__(16) uint16_t As0[GBM * GBK], As1[GBM * GBK];
  __shared__ __align__(16) uint16_t Bs0[GBN * GBK], Bs1[GBN * GBK];
  // XCD-aware tile order: dispatch id d runs on XCD d % 8; give each XCD a
  // contiguous run of tiles (batch-major, then row-major over the tile grid).
  const int d = blockIdx.x;
  const int per = (ntiles + 7) / 8;
  const int tile = (d % 8) * per + d / 8;
  if (tile >= ntiles) return;
  const int tpb = tiles_m * tiles_n;
  const int bz = tile / tpb, rem = tile - bz * tpb;
  const int bm = rem / tiles_n, bn = rem - bm * tiles_n;
  const int m0 = bm * GBM, n0 = bn * GBN;
  const int M = g.M, N = g.N, K = g.K;
  const uint16_t* __restrict__ A = g.A + bz * g.sA;
  const uint16_t* __restrict__ Bm = g.B + bz * g.sB;
  uint16_t* __restrict__ C = OUTF32 ? nullptr : g.C + bz * g.sC;
  float* __restrict__ Cf = OUTF32 ? g.Cf + bz * g.sC : nullptr;
  const int64_t lda = g.lda, ldb = g.ldb, ldc = g.ldc;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS bases stay scalar
  const int wm = wave >> 2, wn = wave & 3;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // full K step: asynchronous buffer loads into LDS.  Per lane, one 32-bit
  // byte offset per instruction is loop-invariant; the K position is a
  // scalar offset.  Rows past M (or N) lie outside the tile's buffer range
  // and read zero.
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (int64_t)m0 * lda, (int64_t)min(M - m0, GBM) * lda * 2);
  const __amdgpu_buffer_rsrc_t rb = NN ? make_rsrc(Bm + n0, ((int64_t)K * ldb - n0) * 2)
                                       : make_rsrc(Bm + (int64_t)n0 * ldb, (int64_t)min(N - n0, GBN) * ldb * 2);
  int voa[4], vob[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = wave * 32 + q * 8 + (lane >> 3);
    const int cs = (lane & 7) ^ ((r >> 1) & 7);
    voa[q] = (int)(((int64_t)r * lda + cs * 8) * 2);
    if constexpr (!NN) {
      vob[q] = (int)(((int64_t)r * ldb + cs * 8) * 2);
    } else {
      const int kr = wave * 8 + q * 2 + (lane >> 5);
      const int cn = (lane & 31) ^ (kr & 7);
      vob[q] = (int)(((int64_t)kr * ldb + cn * 8) * 2);
    }
  }
  // On a partial last K step the A (and NT B) lanes whose chunk lies at or
  // past K load nothing: with a strided operand those columns can run past
  // the end of the allocation on its last row (the buffer range covers whole
  // rows).  zero_tail fills their slots.
  auto dload = [&](int k0, uint16_t* as_, uint16_t* bs_) {
    const int kv = K - k0;
    if (kv >= GBK) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        b2l16(ra, voa[q], k0 * 2, as_ + (wave * 32 + q * 8) * GBK);
        if constexpr (!NN) b2l16(rb, vob[q], k0 * 2, bs_ + (wave * 32 + q * 8) * GBK);
        else b2l16(rb, vob[q], (int)((int64_t)k0 * ldb * 2), bs_ + (wave * 8 + q * 2) * GBN);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = wave * 32 + q * 8 + (lane >> 3);
        if (((lane & 7) ^ ((r >> 1) & 7)) * 8 < kv) {
          b2l16(ra, voa[q], k0 * 2, as_ + (wave * 32 + q * 8) * GBK);
          if constexpr (!NN) b2l16(rb, vob[q], k0 * 2, bs_ + (wave * 32 + q * 8) * GBK);
        }
        if constexpr (NN) b2l16(rb, vob[q], (int)((int64_t)k0 * ldb * 2), bs_ + (wave * 8 + q * 2) * GBN);
      }
    }
  };
  // partial last K step: the loads above also fetch columns (A, NT B) or
  // rows (NN B) past K.  Each lane zeroes the LDS slots its own loads filled,
  // after its wave's loads have landed (slots of other waves' loads may
  // still be in flight).
  auto zero_tail = [&](int k0, uint16_t* as_, uint16_t* bs_) {
    const int kv = K - k0;                  // valid k in this step (multiple of 8)
    if (kv >= GBK) return;
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = wave * 32 + q * 8 + (lane >> 3);
      const int cs = (lane & 7) ^ ((r >> 1) & 7);     // the source chunk this lane loaded
      if (cs * 8 >= kv) {
        *reinterpret_cast<uint4*>(as_ + (wave * 32 + q * 8) * GBK + lane * 8) = z;
        if constexpr (!NN) *reinterpret_cast<uint4*>(bs_ + (wave * 32 + q * 8) * GBK + lane * 8) = z;
      }
      if constexpr (NN) {
        const int kr = wave * 8 + q * 2 + (lane >> 5);
        if (kr >= kv) *reinterpret_cast<uint4*>(bs_ + (wave * 8 + q * 2) * GBN + lane * 8) = z;
      }
    }
  };
  auto compute = [&](const uint16_t* as, const uint16_t* bs) {
    // recompute the fragment addresses here rather than keep two hoisted sets
    // (one per buffer) alive across the loop
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    // fragments of k sub-step s (16 wide) for this wave's 128 x 64 output
    auto frag = [&](int s, bf16x8* af, bf16x8* bfr) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + (lane & 31);
        const int ch = 2 * s + (lane >> 5);
        af[i] = *reinterpret_cast<const bf16x8*>(&as[row * GBK + ((ch ^ ((row >> 1) & 7)) << 3)]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (!NN) {
          const int row = wn * 64 + j * 32 + (lane & 31);
          const int ch = 2 * s + (lane >> 5);
          bfr[j] = *reinterpret_cast<const bf16x8*>(&bs[row * GBK + ((ch ^ ((row >> 1) & 7)) << 3)]);
        } else {
          const int gq = lane >> 4, q = lane & 15;
          const int ncol = wn * 64 + j * 32 + 16 * (gq & 1) + 4 * (q & 3);
          const int chn = ncol >> 3, within = ncol & 7;
          i16x4 h[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int kr = 16 * s + 8 * (gq >> 1) + 4 * hh + (q >> 2);
            h[hh] = ds_read_tr16(&bs[kr * GBN + ((chn ^ (kr & 7)) << 3) + within]);
          }
          typedef short i16x8 __attribute__((ext_vector_type(8)));
          i16x8 v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
          bfr[j] = __builtin_bit_cast(bf16x8, v);
        }
      }
    };
    // fragments of sub-step s + 1 load while the products of sub-step s run
    bf16x8 af[2][4], bfr[2][2];
    frag(0, af[0], bfr[0]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s + 1 < 4) frag(s + 1, af[(s + 1) & 1], bfr[(s + 1) & 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(bfr[s & 1][j], af[s & 1][i], acc[i][j]);
    }
  };

  // double buffer, unrolled by two so each step names its buffers
  // statically; pairs of steps in the loop (one back edge, no early exit),
  // an odd last step after it
  const int nk = (K + GBK - 1) / GBK;
  dload(0, As0, Bs0);
  vm_wait();
  zero_tail(0, As0, Bs0);
  __syncthreads();
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {
    dload((kt + 1) * GBK, As1, Bs1);
    compute(As0, Bs0);
    vm_wait();
    zero_tail((kt + 1) * GBK, As1, Bs1);
    __syncthreads();
    if (kt + 2 < nk) dload((kt + 2) * GBK, As0, Bs0);
    compute(As1, Bs1);
    vm_wait();
    if (kt + 2 < nk) zero_tail((kt + 2) * GBK, As0, Bs0);
    __syncthreads();
  }
  if (kt < nk) compute(As0, Bs0);

  // epilogue.  The products run with the operands swapped, so acc[i][j]
  // holds the transposed 32 x 32 sub-tile: register r of lane l is
  // C[row l % 32][col 8 (r / 4) + 4 (l / 32) + r % 4], i.e. four
  // consecutive columns of one row per register quad.
  if constexpr (OUTF32) {
    // fp32: the same staging in two rounds of 64 rows (16 KiB per wave and
    // round): 16-byte writes into 256-byte rows, chunk c at c ^ (row & 15),
    // then 16-byte row-order stores (4 rows of 256 bytes per instruction)
    uint32_t* st = reinterpret_cast<uint32_t*>((wave < 2 ? As0 : wave < 4 ? As1 : wave < 6 ? Bs0 : Bs1) +
                                               (wave & 1) * (128 * 64));
    const bool vec = (ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(Cf) & 15) == 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      __syncthreads();
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * h + ii;
        const int row = ii * 32 + (lane & 31);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x16& a = acc[i][j];
            const int chunk = j * 8 + 2 * q + (lane >> 5);
            *reinterpret_cast<float4*>(st + row * 64 + ((chunk ^ (row & 15)) << 2)) =
                make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
          }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int e = it * 64 + lane;
        const int row = e >> 4, chunk = e & 15;
        const float4 v = *reinterpret_cast<const float4*>(st + row * 64 + ((chunk ^ (row & 15)) << 2));
        const int gm = m0 + wm * 128 + h * 64 + row, gn = n0 + wn * 64 + chunk * 4;
        if (gm < M && gn < N) {
          float* cp = Cf + (int64_t)gm * ldc + gn;
          if (vec && gn + 3 < N) *reinterpret_cast<float4*>(cp) = v;
          else {
            const float w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2)
              if (gn + e2 < N) cp[e2] = w[e2];
          }
        }
      }
    }
  } else {
    // bf16: each wave stages its 128 x 64 tile (16 KiB) in the now idle LDS
    // buffers, 8-byte writes into 128-byte rows, chunk c at c ^ ((row >> 1) & 7)
    // and the two halves of a chunk swapped on rows with bit 4 set (32 rows of
    // one write touch each bank pair once); then whole rows leave as 16-byte
    // stores, 8 rows of 128 bytes per wave instruction.
    __syncthreads();
    uint16_t* st = (wave < 2 ? As0 : wave < 4 ? As1 : wave < 6 ? Bs0 : Bs1) + (wave & 1) * (128 * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = i * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16& a = acc[i][j];
          const int chunk = j * 4 + q, half = lane >> 5;
          const int off = row * 64 + ((chunk ^ ((row >> 1) & 7)) << 3) + ((half ^ ((row >> 4) & 1)) << 2);
          uint2 v;
          v.x = pack2(f32_to_bits(a[4 * q]), f32_to_bits(a[4 * q + 1]));
          v.y = pack2(f32_to_bits(a[4 * q + 2]), f32_to_bits(a[4 * q + 3]));
          *reinterpret_cast<uint2*>(st + off) = v;
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's staging writes are done
    const bool vec = (ldc & 7) == 0 && (reinterpret_cast<uintptr_t>(C) & 15) == 0;
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int e = it * 64 + lane;
      const int row = e >> 3, chunk = e & 7;
      uint4 v = *reinterpret_cast<const uint4*>(st + row * 64 + ((chunk ^ ((row >> 1) & 7)) << 3));
      if ((row >> 4) & 1) v = make_uint4(v.z, v.w, v.x, v.y);
      const int gm = m0 + wm * 128 + row, gn = n0 + wn * 64 + chunk * 8;
      if (gm < M && gn < N) {
        uint16_t* cp = C + (int64_t)gm * ldc + gn;
        if (vec) *reinterpret_cast<uint4*>(cp) = v;
        else {
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e2 = 0; e2 < 8; ++e2)
            if (gn + e2 < N) cp[e2] = (uint16_t)(w[e2 >> 1] >> (16 * (e2 & 1)));
        }
      }
    }
  }
}

// Generic bf16 GEMM for shapes the tiled kernel cannot take (a dimension,
// stride or offset not a multiple of 8): 16x16 outputs per workgroup, LDS
// tiles, fp32 sums.
template <bool NN>
__global__ __launch_bounds__(256) void gemm_bf16_generic_kernel(GemmArgs g) {
  __shared__ float as[16][17], bs[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int M = g.M, N = g.N, K = g.K;
  const uint16_t* __restrict__ A = g.A + blockIdx.z * g.sA;
  const uint16_t* __restrict__ Bm = g.B + blockIdx.z * g.sB;
  uint16_t* __restrict__ C = g.C + blockIdx.z * g.sC;
  const int gm = blockIdx.y * 16 + ty, gn = blockIdx.x * 16 + tx;
  float s = 0.f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const int ar = blockIdx.y * 16 + ty, ak = k0 + tx;
    as[ty][tx] = (ar < M && ak < K) ? bits_to_f32(A[(int64_t)ar * g.lda + ak]) : 0.f;
    const int bk = k0 + ty, bn = blockIdx.x * 16 + tx;
    float bv = 0.f;
    if (bk < K && bn < N) bv = NN ? bits_to_f32(Bm[(int64_t)bk * g.ldb + bn]) : bits_to_f32(Bm[(int64_t)bn * g.ldb + bk]);
    bs[ty][tx] = bv;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) s = fmaf(as[ty][kk], bs[kk][tx], s);
    __syncthreads();
  }
  if (gm < M && gn < N) C[(int64_t)gm * g.ldc + gn] = f32_to_bits(s);
}

static bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

void launch_gemm_bf16(bool nn, const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return;
  const bool tiled = g.K > 0 && g.K % 8 == 0 && g.N % 8 == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 &&
                     g.sA % 8 == 0 && g.sB % 8 == 0 && aligned8(g.A) && aligned8(g.B);
  if (tiled) {
    const int tn = (g.N + GBN - 1) / GBN, tm = (g.M + GBM - 1) / GBM;
    const int nt = tn * tm * g.batch;
    const int grid = ((nt + 7) / 8) * 8;
    if (nn) hipLaunchKernelGGL((gemm_bf16_kernel<true, false>), dim3(grid), dim3(512), 0, s, g, tm, tn, nt);
    else if (g.batch > 1) hipLaunchKernelGGL((gemm_bf16_kernel<false, true>), dim3(grid), dim3(512), 0, s, g, tm, tn, nt);
    else hipLaunchKernelGGL((gemm_bf16_kernel<false, false>), dim3(grid), dim3(512), 0, s, g, tm, tn, nt);
  } else {
    dim3 grid((unsigned)((g.N + 15) / 16), (unsigned)((g.M + 15) / 16), (unsigned)g.batch);
    if (nn) hipLaunchKernelGGL(gemm_bf16_generic_kernel<true>, grid, dim3(256), 0, s, g);
    else hipLaunchKernelGGL(gemm_bf16_generic_kernel<false>, grid, dim3(256), 0, s, g);
  }
}

void launch_gemm_bf16_f32out(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return;
  const int tn = (g.N + GBN - 1) / GBN, tm = (g.M + GBM - 1) / GBM;
  const int nt = tn * tm * g.batch;
  const int grid = ((nt + 7) / 8) * 8;
  hipLaunchKernelGGL((gemm_bf16_kernel<true, true, true>), dim3(grid), dim3(512), 0, s, g, tm, tn, nt);
}

void launch_gemm_bf16(bool nn, const uint16_t* A, const uint16_t* Bm, uint16_t* C, int64_t M, int64_t N, int64_t K,
                      hipStream_t s) {
  GemmArgs g{};
  g.A = A; g.B = Bm; g.C = C;
  g.M = (int)M; g.N = (int)N; g.K = (int)K;
  g.lda = K; g.ldb = nn ? N : K; g.ldc = N;
  g.batch = 1;
  launch_gemm_bf16(nn, g, s);
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
