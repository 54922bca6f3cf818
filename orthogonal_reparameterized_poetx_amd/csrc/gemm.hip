// Dense products with the frozen weight: the one weight-sized matmul that the
// input-centric formulation keeps per pass
// [P3 "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
// Transformation", Probleemstelling (dense matmuls made POET slow) and
// Methodologie item 1].
//
//   NT: C[M][N] = A[M][K] * B[N][K]^T   (z2 = z1 W0p^T; both K-contiguous)
//   NN: C[M][N] = A[M][K] * B[K][N]     (gz1 = gz2 W0p; B is N-contiguous)
//
// bf16 operands, fp32 accumulation on 32x32x16 MFMA, bf16 output.  256x256
// output tiles, 8 waves of 128x64, k in steps of 32 through a 4-stage LDS
// ring with 16-byte XOR swizzles; the NN B operand is read K-major straight
// from the N-contiguous tile with the gfx950 transposing LDS load.  The two
// waves of each SIMD alternate ("ping-pong"): while one issues its step's
// MFMAs from registers, the other refills the ring and reads its next
// fragments.  Tiles are assigned so that the workgroups on one XCD
// (blockIdx mod 8) work on neighbouring output tiles and share L2.
#include "common.h"
#include "kernels.h"
#include "ranges.h"

namespace poetx {

constexpr int GBM = 256, GBN = 256;

__device__ __forceinline__ i16x4 ds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, const_cast<uint16_t*>(p)));
}

// Buffer resource over the exact extent of a tile (ranges.h): loads past it
// read zero.  The record count is a 32-bit unsigned field; the launcher keeps
// every operand below 4 GiB.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint16_t* base, BufRange r) {
  const uint32_t nrec = (uint32_t)(r.bytes > 0 ? (r.bytes < 0xffffffffLL ? r.bytes : 0xffffffffLL) : 0);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base + r.first), (short)0, (int)nrec, 0x00020000);
}
// 16-byte buffer load straight into LDS, bypassing the VGPRs: lane i of the
// wave writes lds_base + 16 i (lds_base must be wave-uniform).  Streaming tiles
// this way, one contiguous KiB per instruction, reaches several times the L2
// bandwidth of register loads in MFMA-fragment order.
__device__ __forceinline__ void b2l16(__amdgpu_buffer_rsrc_t r, int voff, int soff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, voff, soff, 0, 0);
}

// Ring of GST LDS stages, each a 32-deep k step of both operands (A tile
// [256 rows][32 k], then B), filled by buffer-to-LDS loads GST - 1 steps
// ahead of the step being computed.  16-byte chunks are XOR-swizzled by row
// (the loads pick each lane's source chunk so that the fixed lane -> LDS slot
// placement produces the swizzle):
//   A, NT B: [256 rows][32 k], 64-byte rows, chunk c of row r at c ^ ((r >> 2) & 3):
//     a 16-lane phase of a fragment read (16 consecutive rows, one chunk)
//     touches every bank once
//   NN B:    [32 k rows][256 n], 512-byte rows, chunk c of row r at
//     c ^ ((r & 3) << 2): a 32-lane phase of the transposing read (4 rows,
//     4 chunks, two halves each) touches every bank pair once
// BATCHED only names the instantiation used for batched block products, so
// that profiles tell it apart from the weight products.  SMALL takes K below
// 32 (GST - 2) + 1, where the ring is never full.
constexpr int GST = 4;                 // ring stages
constexpr int GSE = 2 * 256 * 32;      // elements per stage (A and B)
// s_waitcnt immediate waiting for vmcnt <= vm only (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).  The builtin, unlike inline
// asm, is seen by the compiler's wait insertion, which then knows which
// asynchronous LDS fills have completed.
constexpr unsigned vm_imm(unsigned vm) { return (vm & 15u) | ((vm >> 4) << 14) | (7u << 4) | (15u << 8); }

template <bool NN, bool BATCHED, bool SMALL, bool Q8 = false>
__global__ __launch_bounds__(512) void gemm_bf16_kernel(GemmArgs g, int tiles_m, int tiles_n, int ntiles) {
  // the four ring stages as separate LDS objects, each named at compile time
  // below, so that the compiler can tell reads of one from the asynchronous
  // fills of the others; a stage holds the A tile, then the B tile
  constexpr int S = GST;
  __shared__ __align__(16) uint16_t S0[GSE], S1[GSE], S2[GSE], S3[GSE];
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
  uint16_t* __restrict__ C = g.C + bz * g.sC;
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

  // asynchronous buffer loads into LDS.  Per lane, one 32-bit byte offset per
  // instruction is loop-invariant; the K position is a scalar offset for A
  // and NT B.  Rows past M (or N) lie outside the tile's buffer range and
  // read zero.  The NN B operand adds its K position to the per-lane offset
  // instead: the range check covers only that offset, and the last row of a
  // partial N tile would otherwise read past the end of B.
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, gemm_range_a(m0, M, K, lda));
  const __amdgpu_buffer_rsrc_t rb = NN ? make_rsrc(Bm, gemm_range_b_nn(n0, N, K, ldb))
                                       : make_rsrc(Bm, gemm_range_b_nt(n0, N, K, ldb));
  // per-lane source offsets: instruction q (0, 1) of wave w fills KiB
  // (2 w + q) of a 16 KiB operand tile
  //   A, NT B: [256 rows][32 k], 64-byte rows, chunk c of row r at c ^ ((r >> 2) & 3)
  //   NN B:    [32 k rows][256 n], 512-byte rows, chunk c of row r at c ^ ((r & 3) << 2)
  int voa[2], vob[2], csa[2], krb[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = (wave * 2 + q) * 16 + (lane >> 2);
    const int cs = (lane & 3) ^ ((r >> 2) & 3);
    csa[q] = cs;
    voa[q] = (int)(((int64_t)r * lda + cs * 8) * 2);
    if constexpr (!NN) {
      vob[q] = (int)(((int64_t)r * ldb + cs * 8) * 2);
    } else {
      const int kr = (wave * 2 + q) * 2 + (lane >> 5);
      const int cn = (lane & 31) ^ ((kr & 3) << 2);
      krb[q] = kr;
      vob[q] = (int)(((int64_t)kr * ldb + cn * 8) * 2);
    }
  }
  // k ranges of the stages: stage 0 takes the first r0 = K - 32 (nk - 1)
  // values of k (1..32), stage i >= 1 the 32 from r0 + 32 (i - 1); so only
  // stage 0 can be partial, and it is loaded before the loop.  Its lanes whose
  // source lies at or past r0 load nothing (a strided operand could run past
  // the end of its allocation there) and zero their slot instead.
  const int nk = (K + 31) / 32;
  const int r0 = K - 32 * (nk - 1);

  // Q8: the weight operand B as INT8 codes with one fp32 scale per weight row
  // (g.Bq, g.Bs; ldb counts codes).  Each thread loads 16 codes of one row of
  // a stage's B tile into registers (a step ahead of their use), forms
  // bf16(s * q) exactly as the dequantization kernel does, and writes them
  // into the bf16 tile layout above, so the fragment reads and MFMAs are
  // those of the bf16 kernel and the products are bit-identical.
  //   NT: B tile [256 weight rows][32 k]: row qr = tid / 2, codes 16 qh .. 16 qh + 15
  //   NN: B tile [32 k = weight rows][256 n]: row qk = tid / 16, codes 16 qc .. 16 qc + 15
  typedef int q8v4 __attribute__((ext_vector_type(4)));
  const BufRange rqr = !Q8 ? BufRange{0, 0} : NN ? gemm_range_bq_nn(n0, N, K, ldb) : gemm_range_bq_nt(n0, N, K, ldb);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(Q8 ? g.Bq + rqr.first : g.Bq), (short)0,
      (int)(uint32_t)(rqr.bytes < 0xffffffffLL ? rqr.bytes : 0xffffffffLL), 0x00020000);
  int qoff = 0, qrow = 0, qk0 = 0;
  uint32_t qlds0 = 0, qlds1 = 0;
  float qscale = 0.f;
  if constexpr (Q8) {
    if constexpr (!NN) {
      const int qr = tid >> 1, qh = tid & 1, sw = (qr >> 2) & 3;
      qrow = qr;
      qk0 = 16 * qh;
      qoff = (int)((int64_t)qr * ldb + qh * 16);
      qlds0 = 16384u + (uint32_t)(qr * 64 + (((2 * qh) ^ sw) << 4));
      qlds1 = 16384u + (uint32_t)(qr * 64 + (((2 * qh + 1) ^ sw) << 4));
      qscale = n0 + qr < N ? g.Bs[n0 + qr] : 0.f;
    } else {
      const int qk = tid >> 4, qc = tid & 15, sw = (qk & 3) << 2;
      qrow = qk;
      qoff = (int)((int64_t)qk * ldb + qc * 16);
      qlds0 = 16384u + (uint32_t)(qk * 512 + (((2 * qc) ^ sw) << 4));
      qlds1 = 16384u + (uint32_t)(qk * 512 + (((2 * qc + 1) ^ sw) << 4));
    }
  }
  // codes of the step starting at k0 into registers (NN: with the scale of
  // this thread's weight row)
  auto qload = [&](int k0, q8v4& c, float& sc) {
    if constexpr (Q8) {
      if constexpr (!NN) {
        c = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff, k0, 0);
        sc = qscale;
      } else {
        c = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff + (int)((int64_t)k0 * ldb), 0, 0);
        // one load on every lane (row clamped), so each step issues the same
        // number of vector-memory operations; rows past K occur only in the
        // first step, whose conversion zeroes them (kvalid).  The loaded
        // value is used as is, so nothing waits for it before the conversion
        sc = g.Bs[min(k0 + qrow, K - 1)];
      }
    }
  };
  // bf16(s * q) of the 16 codes into the B half of stage st; kvalid (the
  // first stage only) zeroes the k positions at or past it
  auto qconv = [&](const q8v4& c, float sc, const uint16_t* st, int kvalid) {
    if constexpr (Q8) {
      uint32_t o[8];
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        const uint32_t word = (uint32_t)c[h >> 1];
        const int sh = 16 * (h & 1);
        float lo = (float)(int8_t)(word >> sh) * sc;
        float hi = (float)(int8_t)(word >> (sh + 8)) * sc;
        if (kvalid < 32) {
          // NT: code 2h (+1) of this thread sits at k = qk0 + 2h (+1); NN: all at k = qrow
          const int e0 = qk0 + 2 * h;
          const bool keep_lo = NN ? qrow < kvalid : e0 < kvalid;
          const bool keep_hi = NN ? qrow < kvalid : e0 + 1 < kvalid;
          lo = keep_lo ? lo : 0.f;
          hi = keep_hi ? hi : 0.f;
        }
        o[h] = pack2(f32_to_bits(lo), f32_to_bits(hi));
      }
      const uint32_t sb = (uint32_t)reinterpret_cast<uintptr_t>(st);
      const q8v4 v0 = {(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
      const q8v4 v1 = {(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
      asm volatile("ds_write_b128 %0, %2\n\tds_write_b128 %1, %3" ::"v"(sb + qlds0), "v"(sb + qlds1), "v"(v0),
                   "v"(v1)
                   : "memory");
    }
  };
  auto dload = [&](int k0, uint16_t* st) {
    uint16_t* as_ = st;
    uint16_t* bs_ = st + 256 * 32;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      b2l16(ra, voa[q], k0 * 2, as_ + (wave * 2 + q) * 512);
      if constexpr (Q8) continue;
      if constexpr (!NN) b2l16(rb, vob[q], k0 * 2, bs_ + (wave * 2 + q) * 512);
      else b2l16(rb, vob[q] + (int)((int64_t)k0 * ldb * 2), 0, bs_ + (wave * 2 + q) * 512);
    }
  };
  auto dload_first = [&](uint16_t* st) {
    uint16_t* as_ = st;
    uint16_t* bs_ = st + 256 * 32;
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (csa[q] * 8 < r0) b2l16(ra, voa[q], 0, as_ + (wave * 2 + q) * 512);
      else *reinterpret_cast<uint4*>(as_ + (wave * 2 + q) * 512 + lane * 8) = z;
      if constexpr (Q8) continue;
      if constexpr (!NN) {
        if (csa[q] * 8 < r0) b2l16(rb, vob[q], 0, bs_ + (wave * 2 + q) * 512);
        else *reinterpret_cast<uint4*>(bs_ + (wave * 2 + q) * 512 + lane * 8) = z;
      } else {
        if (krb[q] < r0) b2l16(rb, vob[q], 0, bs_ + (wave * 2 + q) * 512);
        else *reinterpret_cast<uint4*>(bs_ + (wave * 2 + q) * 512 + lane * 8) = z;
      }
    }
  };
  bf16x8 AF[2][4], BF[2][2];
  // loop-invariant byte offsets of this lane's fragment reads within a stage
  // (A tile at 0, B tile at 16 KiB; the swizzles as described above).  The
  // reads are inline asm that waits for its own results: the compiler cannot
  // tell which ring stage an asynchronous fill targets and would otherwise
  // wait for every fill in flight before them.
  uint32_t fa[2], fb[2];
  {
    const int l32 = lane & 31, h = lane >> 5, sw = (l32 >> 2) & 3;
#pragma unroll
    for (int s = 0; s < 2; ++s) fa[s] = (uint32_t)((wm * 128 + l32) * 64 + (((2 * s + h) ^ sw) << 4));
    if constexpr (!NN) {
#pragma unroll
      for (int s = 0; s < 2; ++s) fb[s] = (uint32_t)(16384 + (wn * 64 + l32) * 64 + (((2 * s + h) ^ sw) << 4));
    } else {
      const int gq = lane >> 4, q = lane & 15;
      const int kr0 = 8 * (gq >> 1) + (q >> 2);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int ncol = wn * 64 + j * 32 + 16 * (gq & 1) + 4 * (q & 3);
        const int chn = ncol >> 3, within = ncol & 7;
        fb[j] = (uint32_t)(16384 + 2 * (kr0 * 256 + ((chn ^ ((kr0 & 3) << 2)) << 3) + within));
      }
    }
  }
  auto frags = [&](const uint16_t* st) {
    typedef int pi32x4 __attribute__((ext_vector_type(4)));
    typedef int pi32x2 __attribute__((ext_vector_type(2)));
    const uint32_t sb = (uint32_t)reinterpret_cast<uintptr_t>(st);
    const uint32_t a0 = sb + fa[0], a1 = sb + fa[1], b0 = sb + fb[0], b1 = sb + fb[1];
    pi32x4 x[8];
    if constexpr (!NN) {
      pi32x4 y[4];
      asm volatile(
          "ds_read_b128 %0, %12\n\tds_read_b128 %1, %12 offset:2048\n\t"
          "ds_read_b128 %2, %12 offset:4096\n\tds_read_b128 %3, %12 offset:6144\n\t"
          "ds_read_b128 %4, %13\n\tds_read_b128 %5, %13 offset:2048\n\t"
          "ds_read_b128 %6, %13 offset:4096\n\tds_read_b128 %7, %13 offset:6144\n\t"
          "ds_read_b128 %8, %14\n\tds_read_b128 %9, %14 offset:2048\n\t"
          "ds_read_b128 %10, %15\n\tds_read_b128 %11, %15 offset:2048\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7]),
            "=&v"(y[0]), "=&v"(y[1]), "=&v"(y[2]), "=&v"(y[3])
          : "v"(a0), "v"(a1), "v"(b0), "v"(b1)
          : "memory");
      BF[0][0] = __builtin_bit_cast(bf16x8, y[0]);
      BF[0][1] = __builtin_bit_cast(bf16x8, y[1]);
      BF[1][0] = __builtin_bit_cast(bf16x8, y[2]);
      BF[1][1] = __builtin_bit_cast(bf16x8, y[3]);
    } else {
      // B: j = 0 from b0, j = 1 from b1; k sub-step s at +8192, half hh at +2048
      pi32x2 y[8];
      asm volatile(
          "ds_read_b128 %0, %16\n\tds_read_b128 %1, %16 offset:2048\n\t"
          "ds_read_b128 %2, %16 offset:4096\n\tds_read_b128 %3, %16 offset:6144\n\t"
          "ds_read_b128 %4, %17\n\tds_read_b128 %5, %17 offset:2048\n\t"
          "ds_read_b128 %6, %17 offset:4096\n\tds_read_b128 %7, %17 offset:6144\n\t"
          "ds_read_b64_tr_b16 %8, %18\n\tds_read_b64_tr_b16 %9, %18 offset:2048\n\t"
          "ds_read_b64_tr_b16 %10, %18 offset:8192\n\tds_read_b64_tr_b16 %11, %18 offset:10240\n\t"
          "ds_read_b64_tr_b16 %12, %19\n\tds_read_b64_tr_b16 %13, %19 offset:2048\n\t"
          "ds_read_b64_tr_b16 %14, %19 offset:8192\n\tds_read_b64_tr_b16 %15, %19 offset:10240\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7]),
            "=&v"(y[0]), "=&v"(y[1]), "=&v"(y[2]), "=&v"(y[3]), "=&v"(y[4]), "=&v"(y[5]), "=&v"(y[6]), "=&v"(y[7])
          : "v"(a0), "v"(a1), "v"(b0), "v"(b1)
          : "memory");
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const pi32x2 lo = y[4 * j + 2 * s], hi = y[4 * j + 2 * s + 1];
          const pi32x4 v = {lo[0], lo[1], hi[0], hi[1]};
          BF[s][j] = __builtin_bit_cast(bf16x8, v);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      AF[0][i] = __builtin_bit_cast(bf16x8, x[i]);
      AF[1][i] = __builtin_bit_cast(bf16x8, x[4 + i]);
    }
  };
  auto mma = [&]() {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(BF[s][j], AF[s][i], acc[i][j]);
    }
  };

  // Ping-pong ring.  Each wave alternates a memory phase (refill one stage
  // with buffer-to-LDS loads, read this step's fragments) and a compute phase
  // (the step's 16 MFMAs from registers), with a workgroup barrier between
  // phases.  Waves 4..7 run one phase behind waves 0..3; wave w and wave
  // w + 4 of a workgroup land on the same SIMD (the dispatcher's placement;
  // correctness does not depend on it), so each SIMD always has one wave
  // issuing MFMAs while its partner does memory work.  Stage data for step k is complete before the barrier
  // that opens the first memory phase reading it (every wave waits for its
  // own loads of step k before that barrier); a stage is refilled only in a
  // phase after both halves have read it.
  // Q8 code registers: step j's codes live in set j % 2.  Step 0 is
  // converted here; step j >= 1 in the memory phase of step j - 1, two steps
  // after its codes were loaded, and the set is then refilled with the codes
  // of step j + 2
  q8v4 qcs0{}, qcs1{};
  float qsc0 = 0.f, qsc1 = 0.f;
  dload_first(S0);
  if constexpr (Q8) {
    qload(0, qcs0, qsc0);
    qconv(qcs0, qsc0, S0, r0);
  }
  asm volatile("" ::: "memory");
  if (!SMALL || 1 < nk) {
    dload(r0, S1);
    if constexpr (Q8) qload(r0, qcs1, qsc1);
  }
  asm volatile("" ::: "memory");
  if (!SMALL || 2 < nk) {
    dload(r0 + 32, S2);
    if constexpr (Q8) qload(r0 + 32, qcs0, qsc0);
  }
  asm volatile("" ::: "memory");
  // vector-memory operations one step issues: A and B (bf16), or A, the
  // codes and (NN) the scales (Q8); two steps' worth may stay in flight
  constexpr int QOPS = Q8 ? (NN ? 4 : 3) : 4;
  constexpr int QW = QOPS * (S - 2);
  const bool lag = wave >= 4;
#define PPBAR(VM)                                                                    \
  {                                                                                  \
    __builtin_amdgcn_sched_barrier(0);                                               \
    asm volatile("" ::: "memory");                                                   \
    __builtin_amdgcn_s_waitcnt(vm_imm(VM));                                          \
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");                               \
    __builtin_amdgcn_s_barrier();                                                    \
    asm volatile("" ::: "memory");                                                   \
    __builtin_amdgcn_sched_barrier(0);                                               \
  }
  if (SMALL) PPBAR(0) else PPBAR(QW)
  if (lag) __builtin_amdgcn_s_barrier();
  // memory phase of step I: loads of step I + 3 into stage NEXT; Q8: the
  // codes of step I + 1 (set QS_) converted into stage CONV, then the same set
  // refilled with the codes of step I + 3; the fragments of stage CUR; then
  // the compute phase
#define PPSTEADY(I, CUR, NEXT, CONV, QS_, QC_)                                       \
  {                                                                                  \
    dload(r0 + ((I) + S - 2) * 32, NEXT);                                            \
    asm volatile("" ::: "memory");                                                   \
    if constexpr (Q8) {                                                              \
      qconv(QS_, QC_, CONV, 32);                                                     \
      __builtin_amdgcn_sched_barrier(0);                                             \
      qload(r0 + ((I) + S - 2) * 32, QS_, QC_);                                      \
    }                                                                                \
    frags(CUR);                                                                      \
    PPBAR(QW)                                                                        \
    mma();                                                                           \
    PPBAR(QW)                                                                        \
  }
#define PPSTEP(I, CUR, NEXT, CONV, QS_, QC_)                                         \
  {                                                                                  \
    const int i_ = (I);                                                              \
    const bool more = i_ + S - 1 < nk;                                               \
    if (more) dload(r0 + (i_ + S - 2) * 32, NEXT);                                   \
    asm volatile("" ::: "memory");                                                   \
    if constexpr (Q8) {                                                              \
      if (i_ + 1 < nk) qconv(QS_, QC_, CONV, 32);                                    \
      __builtin_amdgcn_sched_barrier(0);                                             \
      if (more) qload(r0 + (i_ + S - 2) * 32, QS_, QC_);                             \
    }                                                                                \
    frags(CUR);                                                                      \
    if (more) PPBAR(QW) else PPBAR(0)                                                \
    mma();                                                                           \
    if (more) PPBAR(QW) else PPBAR(0)                                                \
  }
  int kt = 0;
  if constexpr (!SMALL) {
    for (; kt + 2 * S - 2 < nk; kt += S) {
      PPSTEADY(kt, S0, S3, S1, qcs1, qsc1)
      PPSTEADY(kt + 1, S1, S0, S2, qcs0, qsc0)
      PPSTEADY(kt + 2, S2, S1, S3, qcs1, qsc1)
      PPSTEADY(kt + 3, S3, S2, S0, qcs0, qsc0)
    }
  }
  if (kt < nk) PPSTEP(kt, S0, S3, S1, qcs1, qsc1)
  if (kt + 1 < nk) PPSTEP(kt + 1, S1, S0, S2, qcs0, qsc0)
  if (kt + 2 < nk) PPSTEP(kt + 2, S2, S1, S3, qcs1, qsc1)
  if (kt + 3 < nk) PPSTEP(kt + 3, S3, S2, S0, qcs0, qsc0)
  if (kt + 4 < nk) PPSTEP(kt + 4, S0, S3, S1, qcs1, qsc1)
  if (kt + 5 < nk) PPSTEP(kt + 5, S1, S0, S2, qcs0, qsc0)
  if (!lag) __builtin_amdgcn_s_barrier();
#undef PPSTEADY
#undef PPSTEP
#undef PPBAR

  // epilogue.  The products run with the operands swapped, so acc[i][j]
  // holds the transposed 32 x 32 sub-tile: register r of lane l is
  // C[row l % 32][col 8 (r / 4) + 4 (l / 32) + r % 4], i.e. four
  // consecutive columns of one row per register quad.
  {
    // bf16: each wave stages its 128 x 64 tile (16 KiB) in the now idle LDS
    // buffers, 8-byte writes into 128-byte rows, chunk c at c ^ ((row >> 1) & 7)
    // and the two halves of a chunk swapped on rows with bit 4 set (32 rows of
    // one write touch each bank pair once); then whole rows leave as 16-byte
    // stores, 8 rows of 128 bytes per wave instruction.
    __syncthreads();
    uint16_t* st = (wave < 2 ? S0 : wave < 4 ? S1 : wave < 6 ? S2 : S3) + (wave & 1) * (128 * 64);
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

// K >= 2048 (a multiple of 64): the same ping-pong schedule with the operand
// whose tile rows are 64-byte segments in the 32-deep ring (A of NT) moved
// to a 3-stage ring of 64-deep stages ([256 rows][64 k], 128-byte rows, chunk
// c of row r at c ^ ((r >> 1) & 7)), so that each of its load instructions
// covers 8 whole 128-byte row segments instead of 16 half ones (half the L2
// requests for that operand).  NT: B takes the 64-deep ring, A keeps a 4-stage
// ring of 32-deep steps; NN: A takes the 64-deep ring, B (512-byte rows
// already) keeps the 32-deep ring.  The rings fill 160 KiB of LDS.  Step t
// reads stage t % 4 of the 32-deep ring and half t % 2 of stage (t / 2) % 3 of
// the 64-deep ring; every step refills one 32-deep stage (chunk t + 3), every
// even step one 64-deep stage (stage t / 2 + 2).  k is summed in the same
// order as in the kernel above, so the results are identical.
//
// RS: the forward's R-side block product in the epilogue, for b in
// {64, 128, 256}; NT reads W0p [m][n], NN its transposed copy [n][m].  A 256-column output tile holds 256 / b whole blocks,
// and each wave's 64 columns lie inside one of them.  The tile, rounded to
// bf16 as z2' is, goes into the LDS as the A operand of an NT product with
// the tile's blocks (B operand: rows = output features; the blocks, one
// after another, form a [256][b] matrix), k in b / 32 chunks of 32 through
// two stages, each wave reading the z2' chunks of its own block; that
// product is what the epilogue writes.  Summed over k in ascending 16-deep
// steps on the same MFMA with the same operand roles as the block product
// kernels, so the result is bit-identical to the two passes; it saves their
// z2' write and read [P3 "POET-X: Memory-efficient LLM Training by Scaling
// Orthogonal Transformation", Methodologie item 3: the block-parallel
// transform].
template <bool NN, bool RS = false>
__global__ __launch_bounds__(512) void gemm_wide_kernel(GemmArgs g, int tiles_m, int tiles_n, int ntiles) {
  // R0..R3: the 32-deep ring (16 KiB stages); W0..W2: the 64-deep ring
  __shared__ __align__(16) uint16_t R0[8192], R1[8192], R2[8192], R3[8192];
  __shared__ __align__(16) uint16_t W0[16384], W1[16384], W2[16384];
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
  uint16_t* __restrict__ C = g.C + bz * g.sC;
  const int64_t lda = g.lda, ldb = g.ldb, ldc = g.ldc;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, gemm_range_a(m0, M, K, lda));
  const __amdgpu_buffer_rsrc_t rb = NN ? make_rsrc(Bm, gemm_range_b_nn(n0, N, K, ldb))
                                       : make_rsrc(Bm, gemm_range_b_nt(n0, N, K, ldb));
  // per-lane source offsets.  32-deep ring, instruction q (0, 1) of wave w
  // fills KiB 2 w + q of a stage: NT A [256 rows][32 k] (chunk c of row r at
  // c ^ ((r >> 2) & 3)), NN B [32 k rows][256 n] (chunk c of row r at
  // c ^ ((r & 3) << 2)).  64-deep ring, instruction q (0..3) fills KiB 4 w + q.
  int von[2], vow[4];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if constexpr (!NN) {
      const int r = (wave * 2 + q) * 16 + (lane >> 2);
      const int cs = (lane & 3) ^ ((r >> 2) & 3);
      von[q] = (int)(((int64_t)r * lda + cs * 8) * 2);
    } else {
      const int kr = (wave * 2 + q) * 2 + (lane >> 5);
      const int cn = (lane & 31) ^ ((kr & 3) << 2);
      von[q] = (int)(((int64_t)kr * ldb + cn * 8) * 2);
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = (wave * 4 + q) * 8 + (lane >> 3);
    const int cs = (lane & 7) ^ ((r >> 1) & 7);
    vow[q] = (int)(((int64_t)r * (NN ? lda : ldb) + cs * 8) * 2);
  }
  const int nk = K / 32, np = K / 64;
  // chunk c (k in [32 c, 32 c + 32)) into a 32-deep stage; the NN B operand
  // adds its k position to the range-checked per-lane offset
  auto dloadN = [&](int c, uint16_t* st) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if constexpr (!NN) b2l16(ra, von[q], c * 64, st + (wave * 2 + q) * 512);
      else b2l16(rb, von[q] + (int)((int64_t)c * 32 * ldb * 2), 0, st + (wave * 2 + q) * 512);
    }
  };
  // stage p (k in [64 p, 64 p + 64)) into a 64-deep stage
  auto dloadW = [&](int p, uint16_t* st) {
#pragma unroll
    for (int q = 0; q < 4; ++q) b2l16(NN ? ra : rb, vow[q], p * 128, st + (wave * 4 + q) * 512);
  };
  bf16x8 AF[2][4], BF[2][2];
  // loop-invariant byte offsets of this lane's fragment reads: fn[s] in a
  // 32-deep stage (NT A, or NN B for tile j = s), fw[hf][s] in half hf of a
  // 64-deep stage
  uint32_t fn[2], fw[2][2];
  {
    const int l32 = lane & 31, h = lane >> 5, swb = (l32 >> 1) & 7;
    const int wrow = NN ? wm * 128 : wn * 64;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        fw[hf][s] = (uint32_t)((wrow + l32) * 128 + ((((hf << 2) | (s << 1) | h) ^ swb) << 4));
    if constexpr (!NN) {
      const int sw = (l32 >> 2) & 3;
#pragma unroll
      for (int s = 0; s < 2; ++s) fn[s] = (uint32_t)((wm * 128 + l32) * 64 + (((2 * s + h) ^ sw) << 4));
    } else {
      const int gq = lane >> 4, q = lane & 15;
      const int kr0 = 8 * (gq >> 1) + (q >> 2);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int ncol = wn * 64 + j * 32 + 16 * (gq & 1) + 4 * (q & 3);
        const int chn = ncol >> 3, within = ncol & 7;
        fn[j] = (uint32_t)(2 * (kr0 * 256 + ((chn ^ ((kr0 & 3) << 2)) << 3) + within));
      }
    }
  }
  // fragments of step t from 32-deep stage stn and half hf of 64-deep stage
  // stw, one asm block that waits for its own reads
  auto frags = [&](const uint16_t* stn, const uint16_t* stw, int hf) {
    typedef int pi32x4 __attribute__((ext_vector_type(4)));
    typedef int pi32x2 __attribute__((ext_vector_type(2)));
    const uint32_t sn = (uint32_t)reinterpret_cast<uintptr_t>(stn);
    const uint32_t sw = (uint32_t)reinterpret_cast<uintptr_t>(stw);
    pi32x4 x[8];
    if constexpr (!NN) {
      const uint32_t a0 = sn + fn[0], a1 = sn + fn[1], b0 = sw + fw[hf][0], b1 = sw + fw[hf][1];
      pi32x4 y[4];
      asm volatile(
          "ds_read_b128 %0, %12\n\tds_read_b128 %1, %12 offset:2048\n\t"
          "ds_read_b128 %2, %12 offset:4096\n\tds_read_b128 %3, %12 offset:6144\n\t"
          "ds_read_b128 %4, %13\n\tds_read_b128 %5, %13 offset:2048\n\t"
          "ds_read_b128 %6, %13 offset:4096\n\tds_read_b128 %7, %13 offset:6144\n\t"
          "ds_read_b128 %8, %14\n\tds_read_b128 %9, %14 offset:4096\n\t"
          "ds_read_b128 %10, %15\n\tds_read_b128 %11, %15 offset:4096\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7]),
            "=&v"(y[0]), "=&v"(y[1]), "=&v"(y[2]), "=&v"(y[3])
          : "v"(a0), "v"(a1), "v"(b0), "v"(b1)
          : "memory");
      BF[0][0] = __builtin_bit_cast(bf16x8, y[0]);
      BF[0][1] = __builtin_bit_cast(bf16x8, y[1]);
      BF[1][0] = __builtin_bit_cast(bf16x8, y[2]);
      BF[1][1] = __builtin_bit_cast(bf16x8, y[3]);
    } else {
      // A: 32-row tiles 4096 bytes apart; B: j = 0 from b0, j = 1 from b1, k
      // sub-step s at +8192, half hh at +2048
      const uint32_t a0 = sw + fw[hf][0], a1 = sw + fw[hf][1], b0 = sn + fn[0], b1 = sn + fn[1];
      pi32x2 y[8];
      asm volatile(
          "ds_read_b128 %0, %16\n\tds_read_b128 %1, %16 offset:4096\n\t"
          "ds_read_b128 %2, %16 offset:8192\n\tds_read_b128 %3, %16 offset:12288\n\t"
          "ds_read_b128 %4, %17\n\tds_read_b128 %5, %17 offset:4096\n\t"
          "ds_read_b128 %6, %17 offset:8192\n\tds_read_b128 %7, %17 offset:12288\n\t"
          "ds_read_b64_tr_b16 %8, %18\n\tds_read_b64_tr_b16 %9, %18 offset:2048\n\t"
          "ds_read_b64_tr_b16 %10, %18 offset:8192\n\tds_read_b64_tr_b16 %11, %18 offset:10240\n\t"
          "ds_read_b64_tr_b16 %12, %19\n\tds_read_b64_tr_b16 %13, %19 offset:2048\n\t"
          "ds_read_b64_tr_b16 %14, %19 offset:8192\n\tds_read_b64_tr_b16 %15, %19 offset:10240\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7]),
            "=&v"(y[0]), "=&v"(y[1]), "=&v"(y[2]), "=&v"(y[3]), "=&v"(y[4]), "=&v"(y[5]), "=&v"(y[6]), "=&v"(y[7])
          : "v"(a0), "v"(a1), "v"(b0), "v"(b1)
          : "memory");
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const pi32x2 lo = y[4 * j + 2 * s], hi = y[4 * j + 2 * s + 1];
          const pi32x4 v = {lo[0], lo[1], hi[0], hi[1]};
          BF[s][j] = __builtin_bit_cast(bf16x8, v);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      AF[0][i] = __builtin_bit_cast(bf16x8, x[i]);
      AF[1][i] = __builtin_bit_cast(bf16x8, x[4 + i]);
    }
  };
  auto mma = [&]() {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(BF[s][j], AF[s][i], acc[i][j]);
    }
  };
  // loads issued by this wave after chunk t + 1 of the 32-deep ring, at the
  // barriers of step t (64-deep stage (t + 1) / 2 is issued before that
  // chunk): the refills of steps t - 1 and t, and for t = 0 the prologue's
  // 64-deep stage 1 and chunk 2
  auto issued_after = [&](int t) {
    if (t + 1 >= nk) return 0;
    int n = t == 0 ? 6 : 0;
#pragma unroll
    for (int s = t - 1; s <= t; ++s)
      if (s >= 0) n += 2 * (s + 3 < nk) + 4 * ((s & 1) == 0 && s / 2 + 2 < np);
    return n;
  };
  // prologue: chunk 0, 64-deep stage 0, chunk 1, 64-deep stage 1, chunk 2
  dloadN(0, R0);
  asm volatile("" ::: "memory");
  dloadW(0, W0);
  asm volatile("" ::: "memory");
  dloadN(1, R1);
  asm volatile("" ::: "memory");
  dloadW(1, W1);
  asm volatile("" ::: "memory");
  dloadN(2, R2);
  asm volatile("" ::: "memory");
  const bool lag = wave >= 4;
#define PPBAR(VM)                                                                    \
  {                                                                                  \
    __builtin_amdgcn_sched_barrier(0);                                               \
    asm volatile("" ::: "memory");                                                   \
    __builtin_amdgcn_s_waitcnt(vm_imm(VM));                                          \
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");                               \
    __builtin_amdgcn_s_barrier();                                                    \
    asm volatile("" ::: "memory");                                                   \
    __builtin_amdgcn_sched_barrier(0);                                               \
  }
#define PPBARN(N_)                                                                   \
  {                                                                                  \
    const int n_ = (N_);                                                             \
    if (n_ >= 12) PPBAR(12) else if (n_ >= 10) PPBAR(10) else if (n_ >= 8) PPBAR(8)  \
    else if (n_ >= 6) PPBAR(6) else if (n_ >= 4) PPBAR(4) else if (n_ >= 2) PPBAR(2) \
    else PPBAR(0)                                                                    \
  }
  // chunk 0 and 64-deep stage 0; issued after them: chunk 1, stage 1, chunk 2
  PPBAR(8)
  if (lag) __builtin_amdgcn_s_barrier();
  // step T (static stage names): 32-deep stage NC, refill NR with chunk
  // T + 3; half HF of 64-deep stage WC; on even steps refill WR with 64-deep
  // stage T / 2 + 2
#define PPSTEADY(T, NC, NR, WC, HF, WR)                                              \
  {                                                                                  \
    if ((HF) == 0) dloadW((T) / 2 + 2, WR);                                          \
    asm volatile("" ::: "memory");                                                   \
    dloadN((T) + 3, NR);                                                             \
    asm volatile("" ::: "memory");                                                   \
    frags(NC, WC, HF);                                                               \
    PPBAR(8)                                                                         \
    mma();                                                                           \
    PPBAR(8)                                                                         \
  }
#define PPSTEP(T, NC, NR, WC, HF, WR)                                                \
  {                                                                                  \
    const int t_ = (T);                                                              \
    if ((HF) == 0 && t_ / 2 + 2 < np) dloadW(t_ / 2 + 2, WR);                        \
    asm volatile("" ::: "memory");                                                   \
    if (t_ + 3 < nk) dloadN(t_ + 3, NR);                                             \
    asm volatile("" ::: "memory");                                                   \
    frags(NC, WC, HF);                                                               \
    const int w_ = issued_after(t_);                                                 \
    PPBARN(w_)                                                                       \
    mma();                                                                           \
    PPBARN(w_)                                                                       \
  }
#define PPGROUP(M, O)                                                                \
  M((O) + 0, R0, R3, W0, 0, W2) M((O) + 1, R1, R0, W0, 1, W2)                        \
  M((O) + 2, R2, R1, W1, 0, W0) M((O) + 3, R3, R2, W1, 1, W0)                        \
  M((O) + 4, R0, R3, W2, 0, W1) M((O) + 5, R1, R0, W2, 1, W1)                        \
  M((O) + 6, R2, R1, W0, 0, W2) M((O) + 7, R3, R2, W0, 1, W2)                        \
  M((O) + 8, R0, R3, W1, 0, W0) M((O) + 9, R1, R0, W1, 1, W0)                        \
  M((O) + 10, R2, R1, W2, 0, W1) M((O) + 11, R3, R2, W2, 1, W1)
#define GSTEP(T, NC, NR, WC, HF, WR) if ((T) < nk) PPSTEP(T, NC, NR, WC, HF, WR)
  // steps 0..11 (guarded), whole groups of 12 whose every refill happens,
  // then the last 12..14 steps (guarded)
  PPGROUP(GSTEP, 0)
  int t0 = 12;
  for (; t0 + 14 < nk; t0 += 12) { PPGROUP(PPSTEADY, t0) }
  PPGROUP(GSTEP, t0)
  GSTEP(t0 + 12, R0, R3, W0, 0, W2)
  GSTEP(t0 + 13, R1, R0, W0, 1, W2)
  if (!lag) __builtin_amdgcn_s_barrier();
  if constexpr (RS) {
    // r = bf16(z2') Q^T for this tile (the ring is drained: every step's
    // loads were waited for).  Q chunks c (k in [32 c, 32 c + 32) of each
    // block) go to the two halves of W2 in the 32-deep layout; the z2' tile
    // fills the other eight 16 KiB stages, stage c holding columns
    // [32 c, 32 c + 32).  This wave's block starts at stage zb.
    const int qb = g.qb, nst = qb >> 5;
    const int zb = ((wn * 64) / qb) * nst;
    __syncthreads();
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(g.Qr, gemm_range_q(bn, qb));
    int vq[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = (wave * 2 + q) * 16 + (lane >> 2);
      const int cs = (lane & 3) ^ ((r >> 2) & 3);
      vq[q] = (r * qb + cs * 8) * 2;
    }
    auto qload = [&](int c, uint16_t* st) {
#pragma unroll
      for (int q = 0; q < 2; ++q) b2l16(rq, vq[q], c * 64, st + (wave * 2 + q) * 512);
    };
    uint16_t* const Q0 = W2;
    uint16_t* const Q1 = W2 + 8192;
    qload(0, Q0);
    asm volatile("" ::: "memory");
    qload(1, Q1);
    asm volatile("" ::: "memory");
    // this wave's 128 x 64 part: column group j is stage 2 wn + j, rows
    // 128 wm ..; lane holds columns 8 q + 4 (lane / 32) + e of row
    // lane % 32 of row group i, i.e. half lane / 32 of 16-byte chunk q,
    // stored at chunk q ^ ((row >> 2) & 3) (the layout of the ring's A
    // stages).  Each stage is named statically, so that the compiler sees
    // that these writes do not touch the stages the Q chunks are filling.
    auto zwrite = [&](uint16_t* zs, int j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + (lane & 31);
        const f32x16& a = acc[i][j];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int off = row * 32 + ((q ^ ((row >> 2) & 3)) << 3) + (lane >> 5) * 4;
          uint2 v;
          v.x = pack2(f32_to_bits(a[4 * q]), f32_to_bits(a[4 * q + 1]));
          v.y = pack2(f32_to_bits(a[4 * q + 2]), f32_to_bits(a[4 * q + 3]));
          *reinterpret_cast<uint2*>(zs + off) = v;
        }
      }
    };
    if (wn == 0) { zwrite(R0, 0); zwrite(R1, 1); }
    else if (wn == 1) { zwrite(R2, 0); zwrite(R3, 1); }
    else if (wn == 2) { zwrite(W0, 0); zwrite(W0 + 8192, 1); }
    else { zwrite(W1, 0); zwrite(W1 + 8192, 1); }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    // fragment offsets in the 32-deep layout: z2' rows 128 wm + l32 (fz),
    // block rows 64 wn + l32 (fq)
    uint32_t fz[2], fq[2];
    {
      const int l32 = lane & 31, h = lane >> 5, sw = (l32 >> 2) & 3;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        fz[s2] = (uint32_t)((wm * 128 + l32) * 64 + (((2 * s2 + h) ^ sw) << 4));
        fq[s2] = (uint32_t)((wn * 64 + l32) * 64 + (((2 * s2 + h) ^ sw) << 4));
      }
    }
    auto zstage = [&](int sg) -> const uint16_t* {
      return sg == 0 ? R0 : sg == 1 ? R1 : sg == 2 ? R2 : sg == 3 ? R3 : (sg < 6 ? W0 : W1) + (sg & 1) * 8192;
    };
    auto rfrags = [&](const uint16_t* zs, const uint16_t* qs) {
      typedef int pi32x4 __attribute__((ext_vector_type(4)));
      const uint32_t zb_ = (uint32_t)reinterpret_cast<uintptr_t>(zs);
      const uint32_t qb_ = (uint32_t)reinterpret_cast<uintptr_t>(qs);
      const uint32_t a0 = zb_ + fz[0], a1 = zb_ + fz[1], b0 = qb_ + fq[0], b1 = qb_ + fq[1];
      pi32x4 x[8], y[4];
      asm volatile(
          "ds_read_b128 %0, %12\n\tds_read_b128 %1, %12 offset:2048\n\t"
          "ds_read_b128 %2, %12 offset:4096\n\tds_read_b128 %3, %12 offset:6144\n\t"
          "ds_read_b128 %4, %13\n\tds_read_b128 %5, %13 offset:2048\n\t"
          "ds_read_b128 %6, %13 offset:4096\n\tds_read_b128 %7, %13 offset:6144\n\t"
          "ds_read_b128 %8, %14\n\tds_read_b128 %9, %14 offset:2048\n\t"
          "ds_read_b128 %10, %15\n\tds_read_b128 %11, %15 offset:2048\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7]),
            "=&v"(y[0]), "=&v"(y[1]), "=&v"(y[2]), "=&v"(y[3])
          : "v"(a0), "v"(a1), "v"(b0), "v"(b1)
          : "memory");
      BF[0][0] = __builtin_bit_cast(bf16x8, y[0]);
      BF[0][1] = __builtin_bit_cast(bf16x8, y[1]);
      BF[1][0] = __builtin_bit_cast(bf16x8, y[2]);
      BF[1][1] = __builtin_bit_cast(bf16x8, y[3]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        AF[0][i] = __builtin_bit_cast(bf16x8, x[i]);
        AF[1][i] = __builtin_bit_cast(bf16x8, x[4 + i]);
      }
    };
    // chunk 0 in, chunk 1 in flight; the z2' tile written
    PPBAR(2)
    // step C (C < nst, the same for every wave): z2' stage zb + C with Q
    // stage QS; once every wave has read QS, refill it with chunk C + 2;
    // then wait for chunk C + 1
#define RSSTEP(C_, QS)                                                               \
  if ((C_) < nst) {                                                                  \
    rfrags(zstage(zb + (C_)), QS);                                                   \
    if ((C_) + 2 < nst) {                                                            \
      PPBAR(2)                                                                       \
      qload((C_) + 2, QS);                                                           \
      asm volatile("" ::: "memory");                                                 \
    }                                                                                \
    mma();                                                                           \
    if ((C_) + 2 < nst) PPBAR(2) else PPBAR(0)                                       \
  }
    RSSTEP(0, Q0) RSSTEP(1, Q1) RSSTEP(2, Q0) RSSTEP(3, Q1)
    RSSTEP(4, Q0) RSSTEP(5, Q1) RSSTEP(6, Q0) RSSTEP(7, Q1)
#undef RSSTEP
  }
#undef PPSTEADY
#undef PPSTEP
#undef PPBAR
#undef PPBARN
#undef PPGROUP
#undef GSTEP
  // epilogue as in the kernel above; each wave stages its 128 x 64 tile
  // (16 KiB) in one 32-deep stage or in half of a 64-deep stage
  {
    __syncthreads();
    uint16_t* st = wave == 0 ? R0 : wave == 1 ? R1 : wave == 2 ? R2 : wave == 3 ? R3
                 : (wave < 6 ? W0 : W1) + (wave & 1) * (128 * 64);
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
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
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

static bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

void launch_gemm_bf16(bool nn, const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return;
  const bool tiled = gemm_tiled_shape(g.N, g.K, g.lda, g.ldb, g.sA, g.sB) && aligned8(g.A) && aligned8(g.B);
  if (tiled) {
    const int tn = (g.N + GBN - 1) / GBN, tm = (g.M + GBM - 1) / GBM;
    const int nt = tn * tm * g.batch;
    const int grid = ((nt + 7) / 8) * 8;
    const bool small = (g.K + 31) / 32 < GST - 1;
#define GEMM_LAUNCH(NN_, BT_)                                                                                  \
  {                                                                                                           \
    if (small) hipLaunchKernelGGL((gemm_bf16_kernel<NN_, BT_, true>), dim3(grid), dim3(512), 0, s, g, tm, tn, nt); \
    else hipLaunchKernelGGL((gemm_bf16_kernel<NN_, BT_, false>), dim3(grid), dim3(512), 0, s, g, tm, tn, nt); \
  }
    // measured on the layer set's products (K = 2048 and 5632): NT
    // 8192 x 2048 x 5632 in 142-147 instead of 159-165 us, and 0.08 ms less
    // per training step for NT and NN together.  Short K keeps the 4-stage
    // ring (shorter prologue).
    const bool wide = g.batch == 1 && g.K % 64 == 0 && g.K >= 2048;
    if (wide && nn) hipLaunchKernelGGL((gemm_wide_kernel<true, false>), dim3(grid), dim3(512), 0, s, g, tm, tn, nt);
    else if (wide) hipLaunchKernelGGL((gemm_wide_kernel<false, false>), dim3(grid), dim3(512), 0, s, g, tm, tn, nt);
    else if (nn) GEMM_LAUNCH(true, false)
    else if (g.batch > 1) GEMM_LAUNCH(false, true)
    else GEMM_LAUNCH(false, false)
#undef GEMM_LAUNCH
  } else {
    dim3 grid((unsigned)((g.N + 15) / 16), (unsigned)((g.M + 15) / 16), (unsigned)g.batch);
    if (nn) hipLaunchKernelGGL(gemm_bf16_generic_kernel<true>, grid, dim3(256), 0, s, g);
    else hipLaunchKernelGGL(gemm_bf16_generic_kernel<false>, grid, dim3(256), 0, s, g);
  }
}

bool gemm_rside_applies(bool nn, const void* A, const void* W, const void* Q, const void* C, int64_t M, int64_t N,
                        int64_t K, int b) {
  return (b == 64 || b == 128 || b == 256) && K % 64 == 0 && K >= 2048 && N % GBN == 0 && M > 0 && N > 0 &&
         gemm_tiled_shape(N, K, K, nn ? N : K, 0, 0) && aligned8(A) && aligned8(W) && aligned8(Q) && aligned8(C);
}

void launch_gemm_rside(bool nn, const uint16_t* A, const uint16_t* W, const uint16_t* Q, uint16_t* C, int64_t M,
                       int64_t N, int64_t K, int b, hipStream_t s) {
  GemmArgs g{};
  g.A = A; g.B = W; g.C = C; g.Qr = Q; g.qb = b;
  g.M = (int)M; g.N = (int)N; g.K = (int)K;
  g.lda = K; g.ldb = nn ? N : K; g.ldc = N;
  g.batch = 1;
  const int tn = (int)(N / GBN), tm = (g.M + GBM - 1) / GBM;
  const int nt = tn * tm;
  const int grid = ((nt + 7) / 8) * 8;
  if (nn) hipLaunchKernelGGL((gemm_wide_kernel<true, true>), dim3(grid), dim3(512), 0, s, g, tm, tn, nt);
  else hipLaunchKernelGGL((gemm_wide_kernel<false, true>), dim3(grid), dim3(512), 0, s, g, tm, tn, nt);
}

bool launch_gemm_q8(bool nn, const uint16_t* A, const int8_t* codes, const float* scales, uint16_t* C, int64_t M,
                    int64_t N, int64_t K, hipStream_t s) {
  if (M <= 0 || N <= 0) return true;
  GemmArgs g{};
  g.A = A; g.B = nullptr; g.C = C;
  g.Bq = codes; g.Bs = scales;
  g.M = (int)M; g.N = (int)N; g.K = (int)K;
  g.lda = K; g.ldb = nn ? N : K; g.ldc = N;
  g.batch = 1;
  // 16 codes per load: weight rows of a multiple of 16 bytes
  if (!gemm_tiled_shape(g.N, g.K, g.lda, g.ldb, 0, 0) || g.ldb % 16 != 0 || !aligned8(A) || !aligned8(codes) ||
      (reinterpret_cast<uintptr_t>(scales) & 3))
    return false;
  const int tn = (g.N + GBN - 1) / GBN, tm = (g.M + GBM - 1) / GBM;
  const int nt = tn * tm;
  const int grid = ((nt + 7) / 8) * 8;
  const bool small = (g.K + 31) / 32 < GST - 1;
  if (nn) {
    if (small) hipLaunchKernelGGL((gemm_bf16_kernel<true, false, true, true>), dim3(grid), dim3(512), 0, s, g, tm, tn, nt);
    else hipLaunchKernelGGL((gemm_bf16_kernel<true, false, false, true>), dim3(grid), dim3(512), 0, s, g, tm, tn, nt);
  } else {
    if (small) hipLaunchKernelGGL((gemm_bf16_kernel<false, false, true, true>), dim3(grid), dim3(512), 0, s, g, tm, tn, nt);
    else hipLaunchKernelGGL((gemm_bf16_kernel<false, false, false, true>), dim3(grid), dim3(512), 0, s, g, tm, tn, nt);
  }
  return true;
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
