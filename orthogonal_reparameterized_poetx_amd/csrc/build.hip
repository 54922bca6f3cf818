// Cayley block builder and batched small fp32 GEMM.
//
// Q = (I - S)^-1 (I + S) for skew S [P1 "POET-X：基于正交变换缩放的内存高效LLM训练方法",
// 实践 2], with S unpacked from the stored strict upper triangle
// [P3 "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
// Transformation", Methodologie item 4].  The pages' own GPU route fuses a
// truncated Neumann series; here the inverse is exact: M = (I - S)^-1 by
// Gauss-Jordan without pivoting (I - S has symmetric part I, so every leading
// block is invertible and no growth occurs), then Q = 2M - I because
// (I - S)^-1 (I + S) = (I - S)^-1 (2I - (I - S)).
#include "common.h"
#include "kernels.h"

namespace poetx {

// ----------------------------------------------------------------------------
// Register-resident blocked Gauss-Jordan, one workgroup per B x B matrix.
// Wave w owns (32*TR) x (32*TC) of the matrix in MFMA accumulator layout; a
// panel step K = [32p, 32p+32) inverts the diagonal 32x32 block in LDS, forms
// the new row panel, and updates every other tile with one rank-32 MFMA
// product.  One launch serves two independent batches (the R and the P
// sets of blocks (e.g. the R and P sides of several layers): workgroup w takes
// the segment s with start[s] <= w < start[s+1].
// ----------------------------------------------------------------------------
template <int B> struct GJShape {
  static constexpr int TR = (B >= 256) ? 2 : 1;  // MFMA tiles per wave along rows
  static constexpr int TC = (B >= 256) ? 4 : 1;  // ... along columns
  static constexpr int WPR = B / (32 * TR);      // waves along rows
  static constexpr int WPC = B / (32 * TC);      // waves along columns
  static constexpr int NW = WPR * WPC;
  static constexpr int NT = 64 * NW;
};

// MODE 0: trailing updates on fp32 MFMA (exact products).
// MODE 6: operands split three ways into bf16 (x = h + m + l, |x - h - m - l|
//         <= 2^-27 |x|) and the six products of order <= 2 accumulated on bf16
//         MFMA: fp32-level accuracy at bf16 MFMA rate.
template <int B, int MODE>
__global__ __launch_bounds__(GJShape<B>::NT) void gj_kernel(GJArgs g) {
  using S = GJShape<B>;
  constexpr int TR = S::TR, TC = S::TC, NT = S::NT, WPC = S::WPC;
  constexpr bool X6 = MODE == 6;
  constexpr int PC = 33;       // fp32 column-panel pitch (32 + 1)
  constexpr int PR = B + 4;    // fp32 row-panel pitch (16-byte rows for vector reads)
  constexpr int PT = 36;       // pitch of the transposed diagonal inverse
  constexpr int HP = 40;       // bf16 operand pitch (32 + 8): conflict-free b128 reads
  // one LDS block, carved below; while A is first formed, its start holds the
  // generator's packed triangle (the panels are not live yet)
  constexpr int SZ_OP = X6 ? 3 * B * HP * 2 : 16;
  constexpr int OFF_OPA = 0, OFF_OPB = SZ_OP, OFF_PROW = 2 * SZ_OP;
  constexpr int OFF_DMT = OFF_PROW + 32 * PR * 4, OFF_PCOL = OFF_DMT + 32 * PT * 4;
  constexpr int LDS_BYTES = OFF_PCOL + (X6 ? 16 : B * PC * 4);
  // X6: the fp32 column panel lives in OpB's space, which is dead from the end
  // of one panel's update until the new row panel is written
  static_assert(!X6 || B * PC * 4 <= SZ_OP, "the column panel fits in OpB");
  constexpr int TRI = B * (B - 1) / 2;                         // generator values per block
  constexpr bool STAGE_TRI = X6 && TRI * 4 <= OFF_DMT;
  __shared__ __align__(16) char gj_lds[LDS_BYTES];
  float* Pcol = reinterpret_cast<float*>(gj_lds + (X6 ? OFF_OPB : OFF_PCOL));   // old column panel A[:, K]
  float* Prow = reinterpret_cast<float*>(gj_lds + OFF_PROW);  // old row panel A[K, :], then the new one
  float* DmT = reinterpret_cast<float*>(gj_lds + OFF_DMT);    // inverse of the diagonal block, transposed
  bf16* OpA = reinterpret_cast<bf16*>(gj_lds + OFF_OPA);      // -A[:, K] split h|m|l, [i][kk]
  bf16* OpB = reinterpret_cast<bf16*>(gj_lds + OFF_OPB);      // new A[K, :]^T split h|m|l, [j][kk]
  static_assert(!X6 || B < 256 || STAGE_TRI, "the packed triangle fits in the panel buffers");

  if (g.skip && g.skip[blockIdx.x]) return;   // built another way (truncated series)
  int seg = 0;
  while (seg + 1 < g.nseg && (int)blockIdx.x >= g.start[seg + 1]) ++seg;
  const int blk = (int)blockIdx.x - g.start[seg];
  const GJSeg& sg = g.seg[seg];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tr = (wave / WPC) * 32 * TR;
  const int tc = (wave % WPC) * 32 * TC;
  const int lc = lane & 31;

  auto split3 = [](float x, bf16& h, bf16& m, bf16& l) {
    h = (bf16)x;
    const float r1 = x - (float)h;
    m = (bf16)r1;
    l = (bf16)(r1 - (float)m);
  };

  f32x16 acc[TR][TC];
  if (sg.theta && STAGE_TRI) {
    // ---- A = I - S: the packed strict upper triangle (row-major, theta(i, j)
    // at i B - i (i + 1) / 2 + j - i - 1) is copied to LDS with coalesced
    // loads, then every wave reads its tiles' entries from there:
    // A[i][j] = -theta(i, j) above the diagonal, theta(j, i) below it.
    const float* th = sg.theta + (int64_t)blk * TRI;
    float* T = reinterpret_cast<float*>(gj_lds);
    if ((reinterpret_cast<uintptr_t>(th) & 15) == 0) {
      for (int e = tid; e < TRI / 4; e += NT)
        reinterpret_cast<float4*>(T)[e] = reinterpret_cast<const float4*>(th)[e];
      for (int e = (TRI / 4) * 4 + tid; e < TRI; e += NT) T[e] = th[e];
    } else {
      for (int e = tid; e < TRI; e += NT) T[e] = th[e];
    }
    __syncthreads();
#pragma unroll
    for (int ti = 0; ti < TR; ++ti)
#pragma unroll
      for (int tj = 0; tj < TC; ++tj)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = tr + 32 * ti + c32_row(lane, r), j = tc + 32 * tj + lc;
          const int lo = min(i, j), hi = max(i, j);
          const float v = T[lo * B - lo * (lo + 1) / 2 + (hi - lo - 1)];
          acc[ti][tj][r] = i == j ? 1.0f : (i < j ? -v : v);
        }
    __syncthreads();
  } else {
    // ---- A = I - S (theta mode) or A from a strided matrix, element by element
#pragma unroll
    for (int ti = 0; ti < TR; ++ti)
#pragma unroll
      for (int tj = 0; tj < TC; ++tj)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = tr + 32 * ti + c32_row(lane, r);
          const int j = tc + 32 * tj + lc;
          float v;
          if (sg.theta) {
            const float* th = sg.theta + (int64_t)blk * (B * (B - 1) / 2);
            if (i == j) v = 1.0f;
            else if (i < j) v = -th[i * B - i * (i + 1) / 2 + (j - i - 1)];
            else v = th[j * B - j * (j + 1) / 2 + (i - j - 1)];
          } else {
            v = g.in[(int64_t)blk * g.in_stride + (int64_t)i * g.in_ld + j];
          }
          acc[ti][tj][r] = v;
        }
  }

  for (int p = 0; p < B / 32; ++p) {
    const int K0 = 32 * p;
    // ---- (a) publish the old column and row panels
#pragma unroll
    for (int ti = 0; ti < TR; ++ti)
#pragma unroll
      for (int tj = 0; tj < TC; ++tj) {
        const int I0 = tr + 32 * ti, J0 = tc + 32 * tj;
        if (J0 == K0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = I0 + c32_row(lane, r);
            Pcol[i * PC + lc] = acc[ti][tj][r];
          }
        }
        if (I0 == K0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) Prow[c32_row(lane, r) * PR + J0 + lc] = acc[ti][tj][r];
        }
      }
    __syncthreads();
    // ---- (b) invert the diagonal 32x32 block D in place (Gauss-Jordan, no
    // pivoting) on wave 0: lane (cb, rb) = (lane & 7, lane >> 3) holds the
    // 4x4 sub-block rows 4rb.., columns 4cb.. in registers.  Step k needs the
    // pivot column on this lane's rows and the pivot row on its columns, four
    // values each, fetched from their owners with lane permutes.  With the
    // pivot column cleared (its diagonal entry set to 1) and multipliers
    // c_r = D[r][k] (r != k), c_k = p - 1, the step is one uniform rank-1
    // update D -= c n^T with n_j = D[k][j] / p (j != k), n_k = 1 / p:
    // rows r != k get D[r][j] - D[r][k] D[k][j] / p and -D[r][k] / p in column
    // k; row k gets D[k][j] / p and 1 / p.
    if (wave == 0) {
      const int cb = lane & 7, rb = lane >> 3;
      float d[4][4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float4 v = *reinterpret_cast<const float4*>(&Prow[(4 * rb + a) * PR + K0 + 4 * cb]);
        d[a][0] = v.x; d[a][1] = v.y; d[a][2] = v.z; d[a][3] = v.w;
      }
#pragma unroll 1
      for (int kb = 0; kb < 8; ++kb) {
        const int srcc = (rb * 8 + kb) * 4, srcr = (kb * 8 + cb) * 4;   // byte lane addresses
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          float col[4], row[4];
#pragma unroll
          for (int a = 0; a < 4; ++a)
            col[a] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(srcc, __builtin_bit_cast(int, d[a][kc])));
#pragma unroll
          for (int c = 0; c < 4; ++c)
            row[c] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(srcr, __builtin_bit_cast(int, d[kc][c])));
          const float p = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, d[kc][kc]), kb * 9));
          // 1/p: the hardware reciprocal and one Newton step (within an ulp
          // of the quotient; the division's full sequence sat on the pivot
          // chain, which is sequential over all b pivots)
          const float r0 = __builtin_amdgcn_rcpf(p);
          const float pinv = fmaf(fmaf(-p, r0, 1.0f), r0, r0);
          float n[4], cm[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) n[c] = (cb == kb && c == kc) ? pinv : row[c] * pinv;
#pragma unroll
          for (int a = 0; a < 4; ++a) cm[a] = (rb == kb && a == kc) ? p - 1.0f : col[a];
          if (cb == kb) {
#pragma unroll
            for (int a = 0; a < 4; ++a) d[a][kc] = (rb == kb && a == kc) ? 1.0f : 0.0f;
          }
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int c = 0; c < 4; ++c) d[a][c] = fmaf(-cm[a], n[c], d[a][c]);
        }
      }
      // DmT[j][r] = D^-1[r][j]
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<float4*>(&DmT[(4 * cb + c) * PT + 4 * rb]) = make_float4(d[0][c], d[1][c], d[2][c], d[3][c]);
    }
    // meanwhile the other waves (wave 0 too when it is the only one) split the
    // column panel: OpA[q][i][kk] = piece q of -A[i, K0 + kk], eight k per
    // 16-byte write
    if constexpr (X6) {
      const int nh = NT > 64 ? NT - 64 : NT, h0 = NT > 64 ? tid - 64 : tid;
      for (int e = h0; e >= 0 && e < B * 4; e += nh) {
        const int i = e >> 2, k8 = (e & 3) * 8;
        uint16_t pc[3][8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          bf16 hh, mm, ll;
          split3(-Pcol[i * PC + k8 + t], hh, mm, ll);
          pc[0][t] = __builtin_bit_cast(uint16_t, hh);
          pc[1][t] = __builtin_bit_cast(uint16_t, mm);
          pc[2][t] = __builtin_bit_cast(uint16_t, ll);
        }
#pragma unroll
        for (int q = 0; q < 3; ++q)
          *reinterpret_cast<uint4*>(&OpA[q * B * HP + i * HP + k8]) =
              make_uint4(pack2(pc[q][0], pc[q][1]), pack2(pc[q][2], pc[q][3]), pack2(pc[q][4], pc[q][5]),
                         pack2(pc[q][6], pc[q][7]));
      }
    }
    __syncthreads();
    // ---- (c) new row panel: A[K, j] <- Dinv A[K, j] (j outside K), A[K, K] <- Dinv.
    if constexpr (X6) {
      // on split-bf16 MFMA like the update: wave w < B / 32 forms columns
      // 32 w .. 32 w + 31 (Dinv times its old columns, or Dinv itself in
      // the diagonal tile), reading and writing only those columns of Prow
      if (wave < B / 32) {
        const int J0 = 32 * wave, hi = lane >> 5;
        f32x16 c;
        if (J0 == K0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) c[r] = DmT[lc * PT + c32_row(lane, r)];
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) c[r] = 0.f;
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            bf16x8 a[3], bq[3];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int k = 16 * s + 8 * hi + e;
              bf16 h, m, l;
              split3(DmT[k * PT + lc], h, m, l);            // A[i = lc][k] = Dinv[lc][k]
              a[0][e] = h; a[1][e] = m; a[2][e] = l;
              split3(Prow[k * PR + J0 + lc], h, m, l);      // B[k][j = lc]
              bq[0][e] = h; bq[1][e] = m; bq[2][e] = l;
            }
            // order-2 terms first, then order 1, then the leading product
            c = mfma32(a[0], bq[2], c);
            c = mfma32(a[1], bq[1], c);
            c = mfma32(a[2], bq[0], c);
            c = mfma32(a[0], bq[1], c);
            c = mfma32(a[1], bq[0], c);
            c = mfma32(a[0], bq[0], c);
          }
        }
        // Prow rows i = c32_row(lane, r), column J0 + lc; OpB[q][J0 + lc][i]
        // as four consecutive rows per 8-byte write
#pragma unroll
        for (int r = 0; r < 16; ++r) Prow[c32_row(lane, r) * PR + J0 + lc] = c[r];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          uint16_t hm[3][4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            bf16 h, m, l;
            split3(c[4 * g4 + t], h, m, l);
            hm[0][t] = __builtin_bit_cast(uint16_t, h);
            hm[1][t] = __builtin_bit_cast(uint16_t, m);
            hm[2][t] = __builtin_bit_cast(uint16_t, l);
          }
          const int i0 = 8 * g4 + 4 * hi;
#pragma unroll
          for (int q = 0; q < 3; ++q)
            *reinterpret_cast<uint2*>(&OpB[q * B * HP + (J0 + lc) * HP + i0]) =
                make_uint2(pack2(hm[q][0], hm[q][1]), pack2(hm[q][2], hm[q][3]));
        }
      }
      __syncthreads();
    } else {
      // fp32: each thread owns RB rows x CB columns of the 32 x B panel.
      constexpr int CB = 4;
      constexpr int RB = 32 * B / (NT * CB);
      const int cg = tid % (B / CB), rg = tid / (B / CB);
      float nv[RB][CB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) nv[rb][cb] = 0.f;
      const bool diag = (cg * CB >= K0) && (cg * CB < K0 + 32);
      if (!diag) {
#pragma unroll 4
        for (int t = 0; t < 32; ++t) {
          float dv[RB], pv[CB];
          if constexpr (RB == 4) {
            const float4 v = *reinterpret_cast<const float4*>(&DmT[t * PT + rg * RB]);
            dv[0] = v.x; dv[1] = v.y; dv[2] = v.z; dv[3] = v.w;
          } else {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) dv[rb] = DmT[t * PT + rg * RB + rb];
          }
          {
            const float4 v = *reinterpret_cast<const float4*>(&Prow[t * PR + cg * CB]);
            pv[0] = v.x; pv[1] = v.y; pv[2] = v.z; pv[3] = v.w;
          }
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) nv[rb][cb] += dv[rb] * pv[cb];
        }
      } else {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) nv[rb][cb] = DmT[(cg * CB + cb - K0) * PT + rg * RB + rb];
      }
      __syncthreads();
      // Prow rows as 16-byte writes; OpB as RB consecutive k of one column
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        *reinterpret_cast<float4*>(&Prow[(rg * RB + rb) * PR + cg * CB]) =
            make_float4(nv[rb][0], nv[rb][1], nv[rb][2], nv[rb][3]);
      if constexpr (X6) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          uint16_t hm[3][RB];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            bf16 hh, mm, ll;
            split3(nv[rb][cb], hh, mm, ll);
            hm[0][rb] = __builtin_bit_cast(uint16_t, hh);
            hm[1][rb] = __builtin_bit_cast(uint16_t, mm);
            hm[2][rb] = __builtin_bit_cast(uint16_t, ll);
          }
          const int o = (cg * CB + cb) * HP + rg * RB;
#pragma unroll
          for (int q = 0; q < 3; ++q) {
            bf16* dst = &OpB[q * B * HP + o];
            if constexpr (RB == 4) *reinterpret_cast<uint2*>(dst) = make_uint2(pack2(hm[q][0], hm[q][1]), pack2(hm[q][2], hm[q][3]));
            else if constexpr (RB == 2) *reinterpret_cast<uint32_t*>(dst) = pack2(hm[q][0], hm[q][1]);
            else {
#pragma unroll
              for (int rb = 0; rb < RB; ++rb) reinterpret_cast<uint16_t*>(dst)[rb] = hm[q][rb];
            }
          }
        }
      }
      __syncthreads();
    }
    // ---- (d) update every tile.  Rows outside K: A[i, j] -= A[i, K] newrow[K, j],
    // where for j in K the new row panel holds Dinv and the tile starts from
    // zero, giving A[i, K] <- -A[i, K] Dinv.  Rows in K: the new row panel.
#pragma unroll
    for (int ti = 0; ti < TR; ++ti) {
      const int I0 = tr + 32 * ti;
#pragma unroll
      for (int tj = 0; tj < TC; ++tj) {
        const int J0 = tc + 32 * tj;
        if (I0 == K0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[ti][tj][r] = Prow[c32_row(lane, r) * PR + J0 + lc];
        } else {
          if (J0 == K0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[ti][tj][r] = 0.f;
          }
          if constexpr (X6) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const int ko = 16 * s + 8 * (lane >> 5);
              bf16x8 a[3], b[3];
#pragma unroll
              for (int q = 0; q < 3; ++q) {
                a[q] = *reinterpret_cast<const bf16x8*>(&OpA[q * B * HP + (I0 + lc) * HP + ko]);
                b[q] = *reinterpret_cast<const bf16x8*>(&OpB[q * B * HP + (J0 + lc) * HP + ko]);
              }
              // order-2 terms first, then order 1, then the leading product
              acc[ti][tj] = mfma32(a[0], b[2], acc[ti][tj]);
              acc[ti][tj] = mfma32(a[1], b[1], acc[ti][tj]);
              acc[ti][tj] = mfma32(a[2], b[0], acc[ti][tj]);
              acc[ti][tj] = mfma32(a[0], b[1], acc[ti][tj]);
              acc[ti][tj] = mfma32(a[1], b[0], acc[ti][tj]);
              acc[ti][tj] = mfma32(a[0], b[0], acc[ti][tj]);
            }
          } else {
#pragma unroll
            for (int s = 0; s < 16; ++s) {
              const int kk = 2 * s + (lane >> 5);
              const float a = -Pcol[(I0 + lc) * PC + kk];
              const float bb = Prow[kk * PR + J0 + lc];
              acc[ti][tj] = mfma32f(a, bb, acc[ti][tj]);
            }
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- outputs: M to a strided matrix, or Q = 2M - I in the requested layouts
#pragma unroll
  for (int ti = 0; ti < TR; ++ti)
#pragma unroll
    for (int tj = 0; tj < TC; ++tj) {
      const int I0 = tr + 32 * ti, J0 = tc + 32 * tj;
      const int j = J0 + lc;
      if (g.out) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = I0 + c32_row(lane, r);
          g.out[(int64_t)blk * g.out_stride + (int64_t)i * g.out_ld + j] = acc[ti][tj][r];
        }
      }
      const int64_t base = (int64_t)blk * B * B;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        uint16_t qb[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int r = 4 * r4 + rr;
          const int i = I0 + c32_row(lane, r);
          const float q = 2.0f * acc[ti][tj][r] - (i == j ? 1.0f : 0.0f);
          if (sg.q32) sg.q32[base + (int64_t)i * B + j] = q;
          qb[rr] = f32_to_bits(q);
          if (sg.qbf) sg.qbf[base + (int64_t)i * B + j] = qb[rr];
        }
        if (sg.qtbf) {
          const int i0 = I0 + c32_row(lane, 4 * r4);
          uint2 v;
          v.x = pack2(qb[0], qb[1]);
          v.y = pack2(qb[2], qb[3]);
          *reinterpret_cast<uint2*>(&sg.qtbf[base + (int64_t)j * B + i0]) = v;
        }
      }
    }
}

// one batch item of a BGemmArgs launch: its operands, leading dimensions
struct BGemmItem {
  const float* A; const float* B; float* C;
  int lda, ldb, ldc;
};
__device__ __forceinline__ BGemmItem bgemm_item(const BGemmArgs& a, int64_t bz) {
  BGemmItem t;
  if (bz >= a.nb0) {
    const int64_t z = bz - a.nb0;
    const int64_t sA = a.sA1 ? a.sA1 : a.sA, sB = a.sB1 ? a.sB1 : a.sB, sC = a.sC1 ? a.sC1 : a.sC;
    t.A = a.A1 ? a.A1 + z * sA : a.A + bz * a.sA;
    t.B = a.B1 ? a.B1 + z * sB : a.B + bz * a.sB;
    t.C = a.C1 ? a.C1 + z * sC : a.C + bz * a.sC;
    t.lda = (a.A1 && a.lda1) ? a.lda1 : a.lda;
    t.ldb = (a.B1 && a.ldb1) ? a.ldb1 : a.ldb;
    t.ldc = (a.C1 && a.ldc1) ? a.ldc1 : a.ldc;
  } else {
    t.A = a.A + bz * a.sA;
    t.B = a.B + bz * a.sB;
    t.C = a.C + bz * a.sC;
    t.lda = a.lda; t.ldb = a.ldb; t.ldc = a.ldc;
  }
  return t;
}

// ----------------------------------------------------------------------------
// Batched small fp32 GEMM: C = alpha * opA * opB + beta * C per batch item,
// opA = A or A^T (+ I), opB = B or B^T (+ I).  64x64 tiles, 4 waves of 32x32,
// K in chunks of 32.  MODE 0: fp32 MFMA; MODE 3 / 6: operands split into 2 / 3
// bf16 pieces and the 3 / 6 leading cross products accumulated on bf16 MFMA
// (relative error about 2^-17 / 2^-26 per product).
// M, N, K are multiples of 32.
// ----------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(256) void bgemm_kernel(BGemmArgs a) {
  constexpr int HP = 40;
  constexpr int FP = 33;
  constexpr int NS = MODE == 0 ? 0 : (MODE == 3 ? 2 : 3);   // bf16 pieces per operand
  __shared__ bf16 Ah[NS ? NS * 64 * HP : 2];
  __shared__ bf16 Bh[NS ? NS * 64 * HP : 2];
  __shared__ float Af[NS ? 1 : 64 * FP];
  __shared__ float Bf[NS ? 1 : 64 * FP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const int row0 = blockIdx.y * 64, col0 = blockIdx.x * 64;
  const int64_t bz = blockIdx.z;
  if (a.run && !a.run[bz]) return;
  const BGemmItem it = bgemm_item(a, bz);
  const float* A = it.A;
  const float* Bm = it.B;
  float* C = it.C;
  const int lda = it.lda, ldb = it.ldb, ldc = it.ldc;
  const bool active = (row0 + 32 * wi < a.M) && (col0 + 32 * wj < a.N);
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  auto put = [&](bf16* dst, int idx, float v) {
    const bf16 h = (bf16)v;
    dst[idx] = h;
    if constexpr (NS >= 2) {
      const float r1 = v - (float)h;
      const bf16 m = (bf16)r1;
      dst[64 * HP + idx] = m;
      if constexpr (NS == 3) dst[2 * 64 * HP + idx] = (bf16)(r1 - (float)m);
    }
  };
  // next K chunk is fetched into registers while the current one is multiplied
  float va[8], vb[8];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = tid + 256 * q;
      // element of opA: consecutive threads walk the contiguous dimension
      const int ia = a.transA ? (e & 63) : (e >> 5);
      const int ka = a.transA ? (e >> 6) : (e & 31);
      const int gi = row0 + ia, gka = k0 + ka;
      float x = 0.f;
      if (gi < a.M) {
        x = a.transA ? A[(int64_t)gka * lda + gi] : A[(int64_t)gi * lda + gka];
        if (a.addIA && gi == gka) x += 1.0f;
      }
      va[q] = x;
      // element of opB
      const int jb = a.transB ? (e >> 5) : (e & 63);
      const int kb = a.transB ? (e & 31) : (e >> 6);
      const int gj = col0 + jb, gkb = k0 + kb;
      float y = 0.f;
      if (gj < a.N) {
        y = a.transB ? Bm[(int64_t)gj * ldb + gkb] : Bm[(int64_t)gkb * ldb + gj];
        if (a.addIB && gkb == gj) y += 1.0f;
      }
      vb[q] = y;
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = tid + 256 * q;
      const int ia = a.transA ? (e & 63) : (e >> 5);
      const int ka = a.transA ? (e >> 6) : (e & 31);
      const int jb = a.transB ? (e >> 5) : (e & 63);
      const int kb = a.transB ? (e & 31) : (e >> 6);
      if constexpr (NS) {
        put(Ah, ia * HP + ka, va[q]);
        put(Bh, jb * HP + kb, vb[q]);
      } else {
        Af[ia * FP + ka] = va[q];
        Bf[jb * FP + kb] = vb[q];
      }
    }
  };
  fetch(0);
  for (int k0 = 0; k0 < a.K; k0 += 32) {
    stash();
    __syncthreads();
    if (k0 + 32 < a.K) fetch(k0 + 32);
    if (active) {
      const int lc = lane & 31;
      if constexpr (NS) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int ko = 16 * s + 8 * (lane >> 5);
          bf16x8 x[NS], y[NS];
#pragma unroll
          for (int q = 0; q < NS; ++q) {
            x[q] = *reinterpret_cast<const bf16x8*>(&Ah[q * 64 * HP + (32 * wi + lc) * HP + ko]);
            y[q] = *reinterpret_cast<const bf16x8*>(&Bh[q * 64 * HP + (32 * wj + lc) * HP + ko]);
          }
          if constexpr (NS == 3) {
            acc = mfma32(x[0], y[2], acc);
            acc = mfma32(x[1], y[1], acc);
            acc = mfma32(x[2], y[0], acc);
          }
          acc = mfma32(x[0], y[1], acc);
          acc = mfma32(x[1], y[0], acc);
          acc = mfma32(x[0], y[0], acc);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          const int kk = 2 * s + (lane >> 5);
          acc = mfma32f(Af[(32 * wi + lc) * FP + kk], Bf[(32 * wj + lc) * FP + kk], acc);
        }
      }
    }
    __syncthreads();
  }
  if (active) {
    const int j = col0 + 32 * wj + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = row0 + 32 * wi + c32_row(lane, r);
      float* cp = C + (int64_t)i * ldc + j;
      const float old = (a.beta != 0.f) ? *cp : 0.f;
      *cp = a.alpha * acc[r] + a.beta * old;
    }
  }
}

// ----------------------------------------------------------------------------
// The split-bf16 x6 batched GEMM for sizes in multiples of 128 (the products
// of the b = 512 Schur solve, and the truncated series at b >= 128):
// TM x 128 tiles (TM = 128, or 64 where 128-row tiles would leave CUs idle),
// 8 waves of 32 x (32 TJ) (two waves per SIMD, so one splits and stores while
// the other multiplies), K = 32 NC in chunks of 32, fully unrolled.  Each
// chunk is loaded as 16-byte vectors two chunks ahead into registers, split
// into its three bf16 pieces on the way to one of two LDS buffers, and
// multiplied from there; one barrier per chunk.  Operands are not
// transposed; A + I / B + I as in bgemm_kernel.  The products are accumulated
// in the order of bgemm_kernel<6>, so the results agree with it bit for bit.
// ----------------------------------------------------------------------------
namespace {
constexpr int X6P = 40;                       // LDS pitch in bf16 (32 k + 8)
}  // namespace

template <int NC, int TM>
__global__ __launch_bounds__(512) void bgemm_x6_t128_kernel(BGemmArgs a) {
  constexpr int WR = TM / 32, WC = 8 / WR;    // waves along rows, along columns
  constexpr int TJ = 128 / WC / 32;           // 32-column MFMA tiles per wave
  constexpr int NA = TM * 8 / 512;            // A float4 per thread per chunk
  constexpr int PA = TM * X6P, PB = 128 * X6P;          // one piece of A, of B
  constexpr int BUF = 3 * PA + 3 * PB;
  __shared__ __align__(16) bf16 L[2 * BUF];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave / WC, wc = wave % WC;
  const int row0 = blockIdx.y * TM, col0 = blockIdx.x * 128;
  const int64_t bz = blockIdx.z;
  if (a.run && !a.run[bz]) return;
  const BGemmItem it = bgemm_item(a, bz);

  // loads of one chunk: A row row0 + (e >> 3), float4 (e & 7) of the chunk's
  // 32 k; B rows k0 + 2 (tid & 15) and the next, float4 (tid >> 4) of the 128
  // columns (k fastest across lanes, so that the transposed LDS writes of a
  // wave fall on distinct banks)
  const int kp = tid & 15, jq = tid >> 4;
  float4 ra[2][NA], rb[2][2];
  auto load = [&](int c, int set) {
    const int k0 = 32 * c;
#pragma unroll
    for (int o = 0; o < NA; ++o) {
      const int e = tid + 512 * o, r = e >> 3, q = e & 7;
      ra[set][o] = *reinterpret_cast<const float4*>(it.A + (int64_t)(row0 + r) * it.lda + k0 + 4 * q);
    }
    const float* src = it.B + (int64_t)(k0 + 2 * kp) * it.ldb + col0 + 4 * jq;
    rb[set][0] = *reinterpret_cast<const float4*>(src);
    rb[set][1] = *reinterpret_cast<const float4*>(src + it.ldb);
  };
  auto split3 = [](float x, uint16_t& h, uint16_t& m, uint16_t& l) {
    const bf16 hh = (bf16)x;
    const float r1 = x - (float)hh;
    const bf16 mm = (bf16)r1;
    h = __builtin_bit_cast(uint16_t, hh);
    m = __builtin_bit_cast(uint16_t, mm);
    l = __builtin_bit_cast(uint16_t, (bf16)(r1 - (float)mm));
  };
  // A piece q at [q][row][k]; B piece q at [q][col][k] after the A pieces
  auto stash = [&](int c, int set, bf16* buf) {
    const int k0 = 32 * c;
#pragma unroll
    for (int o = 0; o < NA; ++o) {
      const int e = tid + 512 * o, r = e >> 3, q = e & 7;
      const float v[4] = {ra[set][o].x, ra[set][o].y, ra[set][o].z, ra[set][o].w};
      uint16_t pc[3][4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float x = v[t];
        if (a.addIA && row0 + r == k0 + 4 * q + t) x += 1.0f;
        split3(x, pc[0][t], pc[1][t], pc[2][t]);
      }
#pragma unroll
      for (int pq = 0; pq < 3; ++pq)
        *reinterpret_cast<uint2*>(buf + pq * PA + r * X6P + 4 * q) =
            make_uint2(pack2(pc[pq][0], pc[pq][1]), pack2(pc[pq][2], pc[pq][3]));
    }
    const float v0[4] = {rb[set][0].x, rb[set][0].y, rb[set][0].z, rb[set][0].w};
    const float v1[4] = {rb[set][1].x, rb[set][1].y, rb[set][1].z, rb[set][1].w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int j = 4 * jq + t, k = 2 * kp;
      float x0 = v0[t], x1 = v1[t];
      if (a.addIB) {
        if (col0 + j == k0 + k) x0 += 1.0f;
        if (col0 + j == k0 + k + 1) x1 += 1.0f;
      }
      uint16_t p0[3], p1[3];
      split3(x0, p0[0], p0[1], p0[2]);
      split3(x1, p1[0], p1[1], p1[2]);
#pragma unroll
      for (int pq = 0; pq < 3; ++pq)
        *reinterpret_cast<uint32_t*>(buf + 3 * PA + pq * PB + j * X6P + k) = pack2(p0[pq], p1[pq]);
    }
  };

  f32x16 acc[TJ];
#pragma unroll
  for (int tj = 0; tj < TJ; ++tj)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[tj][r] = 0.f;
  const int lc = lane & 31;
  auto compute = [&](const bf16* buf) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int ko = 16 * s + 8 * (lane >> 5);
      bf16x8 x[3], y[TJ][3];
#pragma unroll
      for (int pq = 0; pq < 3; ++pq) {
        x[pq] = *reinterpret_cast<const bf16x8*>(buf + pq * PA + (32 * wr + lc) * X6P + ko);
#pragma unroll
        for (int t = 0; t < TJ; ++t)
          y[t][pq] = *reinterpret_cast<const bf16x8*>(buf + 3 * PA + pq * PB + (32 * TJ * wc + 32 * t + lc) * X6P + ko);
      }
#pragma unroll
      for (int tj = 0; tj < TJ; ++tj) {
        f32x16 c = acc[tj];
        c = mfma32(x[0], y[tj][2], c);
        c = mfma32(x[1], y[tj][1], c);
        c = mfma32(x[2], y[tj][0], c);
        c = mfma32(x[0], y[tj][1], c);
        c = mfma32(x[1], y[tj][0], c);
        c = mfma32(x[0], y[tj][0], c);
        acc[tj] = c;
      }
    }
  };

  // chunk c sits in register set c % 2 from two chunks before its stash
  load(0, 0);
  if (NC > 1) load(1, 1);
  stash(0, 0, L);
  if (NC > 2) load(2, 0);
  __syncthreads();
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    compute(L + (c & 1) * BUF);
    if (c + 1 < NC) {
      stash(c + 1, (c + 1) & 1, L + ((c + 1) & 1) * BUF);
      if (c + 3 < NC) load(c + 3, (c + 1) & 1);
    }
    __syncthreads();
  }

#pragma unroll
  for (int tj = 0; tj < TJ; ++tj) {
    const int j = col0 + 32 * TJ * wc + 32 * tj + lc;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = row0 + 32 * wr + c32_row(lane, r);
      float* cp = it.C + (int64_t)i * it.ldc + j;
      const float old = (a.beta != 0.f) ? *cp : 0.f;
      *cp = a.alpha * acc[tj][r] + a.beta * old;
    }
  }
}

// I - S for a batch of b x b blocks (b = 512 route), fp32 [blk][b][b].  One
// workgroup per pair of 32x32 tiles (I, J) and (J, I), I <= J: the upper
// tile's entries are rows of the packed triangle (theta(i, j), j > i, is
// contiguous in j), read once, written negated to (I, J) and, transposed
// through LDS, to (J, I), so every read and write is along rows.
__global__ __launch_bounds__(256) void unpack_eye_minus_s_kernel(const float* __restrict__ theta, int b,
                                                                 float* __restrict__ A) {
  __shared__ float t[32][33];
  const int blk = blockIdx.y;
  const int nt = b / 32;
  // tile pair p -> (I, J), I <= J, row by row of the upper tile triangle
  int p = blockIdx.x, I = 0;
  while (p >= nt - I) { p -= nt - I; ++I; }
  const int J = I + p;
  const float* th = theta + (int64_t)blk * (b * (b - 1) / 2);
  float* Ab = A + (int64_t)blk * b * b;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 8 rows per pass
  for (int r = ty; r < 32; r += 8) {
    const int i = 32 * I + r, j = 32 * J + tx;
    float v = 0.f;
    if (j > i) v = th[i * b - i * (i + 1) / 2 + (j - i - 1)];
    t[r][tx] = v;
    // upper tile: -theta above the diagonal, 1 on it; in a diagonal tile the
    // entries below it are the mirror, written in the second pass
    if (I != J || j >= i) Ab[(int64_t)i * b + j] = (i == j) ? 1.f : -v;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int i = 32 * J + r, j = 32 * I + tx;   // entry (i, j) of the lower tile = theta(j, i)
    if (I != J || i > j) Ab[(int64_t)i * b + j] = t[tx][r];
  }
}

// Q = 2M - I from M [blk][b][b] into Q32 / Qbf16 / QTbf16 (32x32 LDS transpose)
__global__ __launch_bounds__(256) void finalize_q_kernel(const float* __restrict__ M, int b, float* q32,
                                                         uint16_t* qbf, uint16_t* qtbf) {
  __shared__ uint16_t t[32][33];
  const int blk = blockIdx.z;
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 8 rows per pass
  const int64_t base = (int64_t)blk * b * b;
  for (int r = ty; r < 32; r += 8) {
    const int i = i0 + r, j = j0 + tx;
    const float q = 2.f * M[base + (int64_t)i * b + j] - (i == j ? 1.f : 0.f);
    if (q32) q32[base + (int64_t)i * b + j] = q;
    const uint16_t h = f32_to_bits(q);
    if (qbf) qbf[base + (int64_t)i * b + j] = h;
    t[r][tx] = h;
  }
  __syncthreads();
  if (qtbf)
    for (int r = ty; r < 32; r += 8) qtbf[base + (int64_t)(j0 + r) * b + i0 + tx] = t[tx][r];
}

// ----------------------------------------------------------------------------
// host launchers
// ----------------------------------------------------------------------------
template <int B, int MODE>
static void launch_gj_t(int nblk, const GJArgs& g, hipStream_t s) {
  hipLaunchKernelGGL((gj_kernel<B, MODE>), dim3(nblk), dim3(GJShape<B>::NT), 0, s, g);
}

void launch_gj(int B, int mode, int nblk, const GJArgs& g, hipStream_t s) {
  if (nblk <= 0) return;
  const bool x6 = mode == 6;
  switch (B) {
    case 32: x6 ? launch_gj_t<32, 6>(nblk, g, s) : launch_gj_t<32, 0>(nblk, g, s); break;
    case 64: x6 ? launch_gj_t<64, 6>(nblk, g, s) : launch_gj_t<64, 0>(nblk, g, s); break;
    case 128: x6 ? launch_gj_t<128, 6>(nblk, g, s) : launch_gj_t<128, 0>(nblk, g, s); break;
    case 256: x6 ? launch_gj_t<256, 6>(nblk, g, s) : launch_gj_t<256, 0>(nblk, g, s); break;
    default: break;
  }
}

// the 128x128-tile kernel applies: split x6, no transposes, M and N multiples
// of 128, K = 128 or 256, 16-byte aligned rows of A and B in every segment
static bool bgemm_t128_applies(int mode, const BGemmArgs& a) {
  if (mode != 6 || a.transA || a.transB || a.M % 128 || a.N % 128 || (a.K != 128 && a.K != 256)) return false;
  auto al = [](const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  auto al4 = [](int64_t v) { return (v & 3) == 0; };
  return al(a.A) && al(a.B) && al(a.A1) && al(a.B1) && al4(a.lda) && al4(a.ldb) && al4(a.lda1) && al4(a.ldb1) &&
         al4(a.sA) && al4(a.sB) && al4(a.sA1) && al4(a.sB1);
}

void launch_bgemm(int mode, int batch, const BGemmArgs& a, hipStream_t s) {
  if (batch <= 0) return;
  if (bgemm_t128_applies(mode, a)) {
    // 128-row tiles where 64-row ones would need a second round of
    // workgroups (29 blocks at b = 512: 64-row tiles 14 us, 128-row 19 us;
    // 58: 27 and 22 us)
    const bool tall = 2 * (int64_t)batch * (a.M / 128) * (a.N / 128) > 256;
    dim3 grid(a.N / 128, a.M / (tall ? 128 : 64), batch);
    if (a.K == 256) {
      if (tall) hipLaunchKernelGGL((bgemm_x6_t128_kernel<8, 128>), grid, dim3(512), 0, s, a);
      else hipLaunchKernelGGL((bgemm_x6_t128_kernel<8, 64>), grid, dim3(512), 0, s, a);
    } else {
      if (tall) hipLaunchKernelGGL((bgemm_x6_t128_kernel<4, 128>), grid, dim3(512), 0, s, a);
      else hipLaunchKernelGGL((bgemm_x6_t128_kernel<4, 64>), grid, dim3(512), 0, s, a);
    }
    return;
  }
  dim3 grid((a.N + 63) / 64, (a.M + 63) / 64, batch);
  if (mode == 6) hipLaunchKernelGGL(bgemm_kernel<6>, grid, dim3(256), 0, s, a);
  else if (mode == 3) hipLaunchKernelGGL(bgemm_kernel<3>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(bgemm_kernel<0>, grid, dim3(256), 0, s, a);
}

void launch_unpack_eye_minus_s(const float* theta, int b, int nblk, float* A, hipStream_t s) {
  if (nblk <= 0 || b % 32) return;
  const int nt = b / 32;
  dim3 grid((unsigned)(nt * (nt + 1) / 2), nblk);
  hipLaunchKernelGGL(unpack_eye_minus_s_kernel, grid, dim3(256), 0, s, theta, b, A);
}

void launch_finalize_q(const float* M, int b, int nblk, float* q32, uint16_t* qbf, uint16_t* qtbf, hipStream_t s) {
  if (nblk <= 0) return;
  dim3 grid(b / 32, b / 32, nblk);
  hipLaunchKernelGGL(finalize_q_kernel, grid, dim3(256), 0, s, M, b, q32, qbf, qtbf);
}


}  // namespace poetx
