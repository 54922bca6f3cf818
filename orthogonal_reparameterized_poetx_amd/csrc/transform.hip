// Permuted block-diagonal transforms of token rows (the P and R sides).
//
// The orthogonal factors are permutation x block-diagonal x permutation; the
// permutations are applied as index maps, never as matrices, and the blocks
// are treated as a batch of independent b x b products
// [P3 "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
// Transformation", Methodologie items 2 and 3].
//
// Two kernels cover the four uses:
//  gather-in  (P forward, R backward): a token row in true coordinates is
//    gathered through the permutation, then block l is multiplied;
//    the result is written contiguously in the permuted ("working") layout.
//  scatter-out (R forward, P backward): a working-layout row is multiplied
//    block by block and scattered back to true coordinates.
//
// Design for gfx950: a workgroup owns T tokens and every block of the row, so
// each activation byte crosses HBM once.  Full rows are staged in LDS (in as
// many passes as LDS holds), the gather/scatter is done on LDS addresses, and
// the gathered MFMA operand fragments (gather-in) or the finished results
// (scatter-out) are held in VGPRs across the passes.  Blocks are split over
// waves (NS consecutive blocks per wave); products use 16x16x32 bf16 MFMA
// with fp32 accumulation.
#include "common.h"
#include "kernels.h"

namespace poetx {

constexpr int LDS_ELEMS = 79 * 1024;  // 158 KiB of bf16

__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__host__ __device__ __forceinline__ int row_pitch(int W) { return ((W + 127) / 128) * 128 + 2; }

// Stage rows [t0+p0, t0+p0+np) of src [N][W] bf16 into lds[r*pitch + c].
__device__ __forceinline__ void stage_rows(const uint16_t* __restrict__ src, int64_t N, int W, int pitch,
                                           int64_t tbase, int np, uint16_t* lds, int tid, int nt) {
  if ((W & 7) == 0) {
    const int nch = W >> 3;
    const int tot = np * nch;
    for (int e = tid; e < tot; e += nt) {
      const int r = e / nch, c = e - r * nch;
      const int64_t t = tbase + r;
      if (t < N) {
        const uint4 v = ldg16(src + t * W + (int64_t)c * 8);
        uint32_t* d = reinterpret_cast<uint32_t*>(lds + r * pitch + c * 8);
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
      }
    }
  } else {
    const int tot = np * W;
    for (int e = tid; e < tot; e += nt) {
      const int r = e / W, c = e - r * W;
      const int64_t t = tbase + r;
      if (t < N) lds[r * pitch + c] = src[t * W + c];
    }
  }
}

// Write lds rows back to dst [N][W] (true layout), coalesced.
__device__ __forceinline__ void unstage_rows(uint16_t* __restrict__ dst, int64_t N, int W, int pitch,
                                             int64_t tbase, int np, const uint16_t* lds, int tid, int nt) {
  if ((W & 7) == 0) {
    const int nch = W >> 3;
    const int tot = np * nch;
    for (int e = tid; e < tot; e += nt) {
      const int r = e / nch, c = e - r * nch;
      const int64_t t = tbase + r;
      if (t < N) {
        const uint32_t* s = reinterpret_cast<const uint32_t*>(lds + r * pitch + c * 8);
        uint4 v;
        v.x = s[0]; v.y = s[1]; v.z = s[2]; v.w = s[3];
        stg16(dst + t * W + (int64_t)c * 8, v);
      }
    }
  } else {
    const int tot = np * W;
    for (int e = tid; e < tot; e += nt) {
      const int r = e / W, c = e - r * W;
      const int64_t t = tbase + r;
      if (t < N) dst[t * W + c] = lds[r * pitch + c];
    }
  }
}

// ---------------------------------------------------------------------------
// gather-in
// ---------------------------------------------------------------------------
template <int B, int TT, int NS, int MAXT>
__global__ __launch_bounds__(MAXT) void gather_in_kernel(XformArgs a) {
  constexpr int T = 16 * TT;
  constexpr int KC = B / 32;             // 32-wide k chunks per block
  constexpr int CW = B < 64 ? B : 64;    // output columns staged per chunk
  constexpr int SP = 72;                 // stage pitch (elements)
  __shared__ __align__(16) uint16_t lds[LDS_ELEMS];
  const uint16_t* __restrict__ in = static_cast<const uint16_t*>(a.in);
  uint16_t* __restrict__ out = static_cast<uint16_t*>(a.out);
  uint16_t* __restrict__ emit = static_cast<uint16_t*>(a.emit);
  const uint16_t* __restrict__ bq = static_cast<const uint16_t*>(a.bq);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nt = blockDim.x;
  const int W = a.W, k = a.k;
  const int64_t N = a.N;
  const int64_t t0 = (int64_t)blockIdx.x * T;
  const int pitch = row_pitch(W);
  const int TP = min(T, LDS_ELEMS / pitch);
  const int tail0 = k * B;
  const bool vec = (W & 7) == 0;

  bf16x8 frag[NS][TT][KC];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) frag[s][tt][kc] = as_bf16x8(make_uint4(0, 0, 0, 0));

  // ---- phase G: stage rows, gather operand fragments
  for (int p0 = 0; p0 < T; p0 += TP) {
    const int np = min(TP, T - p0);
    stage_rows(in, N, W, pitch, t0 + p0, np, lds, tid, nt);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int l = wave * NS + s;
      if (l < k) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          const int tl = tt * 16 + (lane & 15);
          if (tl >= p0 && tl < p0 + np) {
            const uint16_t* row = lds + (tl - p0) * pitch;
            const int64_t t = t0 + tl;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
              const int kk0 = kc * 32 + 8 * (lane >> 4);
              const int4 pa = *reinterpret_cast<const int4*>(a.perm + l * B + kk0);
              const int4 pb = *reinterpret_cast<const int4*>(a.perm + l * B + kk0 + 4);
              uint4 v;
              v.x = pack2(row[pa.x], row[pa.y]);
              v.y = pack2(row[pa.z], row[pa.w]);
              v.z = pack2(row[pb.x], row[pb.y]);
              v.w = pack2(row[pb.z], row[pb.w]);
              frag[s][tt][kc] = as_bf16x8(v);
              if (emit && t < N) {
                uint16_t* e = emit + t * W + l * B + kk0;
                if (vec) stg16(e, v);
                else {
                  e[0] = v.x & 0xffff; e[1] = v.x >> 16; e[2] = v.y & 0xffff; e[3] = v.y >> 16;
                  e[4] = v.z & 0xffff; e[5] = v.z >> 16; e[6] = v.w & 0xffff; e[7] = v.w >> 16;
                }
              }
            }
          }
        }
      }
    }
    // identity tail: plain gather
    const int tail = W - tail0;
    if (tail > 0) {
      for (int e = tid; e < np * tail; e += nt) {
        const int r = e / tail, i = tail0 + (e - r * tail);
        const int64_t t = t0 + p0 + r;
        if (t < N) {
          const uint16_t v = lds[r * pitch + a.perm[i]];
          out[t * W + i] = v;
          if (emit) emit[t * W + i] = v;
        }
      }
    }
    __syncthreads();
  }

  // ---- phase C: block products, staged per CW columns for coalesced stores
  uint16_t* stage = lds + wave * (T * SP);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int l = wave * NS + s;
    if (l < k) {
      const uint16_t* bql = bq + (int64_t)l * B * B;
      for (int cg = 0; cg < B / CW; ++cg) {
#pragma unroll
        for (int c4 = 0; c4 < CW / 16; ++c4) {
          const int c = cg * (CW / 16) + c4;
          f32x4 acc[TT];
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
          const uint16_t* bp = bql + (int64_t)(c * 16 + (lane & 15)) * B + 8 * (lane >> 4);
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) {
            const bf16x8 bv = as_bf16x8(ldg16(bp + kc * 32));
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) acc[tt] = mfma16(frag[s][tt][kc], bv, acc[tt]);
          }
#pragma unroll
          for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              stage[(tt * 16 + 4 * (lane >> 4) + r) * SP + c4 * 16 + (lane & 15)] = f32_to_bits(acc[tt][r]);
        }
        lds_fence();
        // copy T x CW to out
        constexpr int CH = CW / 8;
        for (int e = lane; e < T * CH; e += 64) {
          const int r = e / CH, cc = e - r * CH;
          const int64_t t = t0 + r;
          if (t < N) {
            const uint16_t* sp = stage + r * SP + cc * 8;
            uint16_t* op = out + t * W + l * B + cg * CW + cc * 8;
            if (vec) {
              const uint4 v = *reinterpret_cast<const uint4*>(sp);
              stg16(op, v);
            } else {
#pragma unroll
              for (int q = 0; q < 8; ++q) op[q] = sp[q];
            }
          }
        }
        lds_fence();
      }
    }
  }
}

// ---------------------------------------------------------------------------
// scatter-out
// ---------------------------------------------------------------------------
template <int B, int TT, int NS, int MAXT>
__global__ __launch_bounds__(MAXT) void scatter_out_kernel(XformArgs a) {
  constexpr int T = 16 * TT;
  constexpr int KC = B / 32;
  constexpr int NC = B / 16;    // 16-wide output column tiles per block
  __shared__ __align__(16) uint16_t lds[LDS_ELEMS];
  const uint16_t* __restrict__ in = static_cast<const uint16_t*>(a.in);
  uint16_t* __restrict__ out = static_cast<uint16_t*>(a.out);
  const uint16_t* __restrict__ bq = static_cast<const uint16_t*>(a.bq);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nt = blockDim.x;
  const int W = a.W, k = a.k;
  const int64_t N = a.N;
  const int64_t t0 = (int64_t)blockIdx.x * T;
  const int pitch = row_pitch(W);
  const int TP = min(T, LDS_ELEMS / pitch);
  const int tail0 = k * B;
  const bool vec = (W & 7) == 0;

  // ---- phase C: results for all of this wave's blocks, bf16 in registers
  uint32_t res[NS][NC][TT][2];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int l = wave * NS + s;
#pragma unroll
    for (int cp = 0; cp < NC / 2; ++cp) {
      f32x4 acc[2][TT];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[c2][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (l < k) {
        // two k chunks in flight: fully unrolled, the loads of every chunk
        // would be issued up front and not fit beside the held results
#pragma unroll 2
        for (int kc = 0; kc < KC; ++kc) {
          bf16x8 af[TT];
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            const int64_t t = t0 + tt * 16 + (lane & 15);
            const int col = l * B + kc * 32 + 8 * (lane >> 4);
            uint4 v = make_uint4(0, 0, 0, 0);
            if (t < N) {
              const uint16_t* ip = in + t * W + col;
              if (vec) v = ldg16(ip);
              else {
                v.x = pack2(ip[0], ip[1]); v.y = pack2(ip[2], ip[3]);
                v.z = pack2(ip[4], ip[5]); v.w = pack2(ip[6], ip[7]);
              }
            }
            af[tt] = as_bf16x8(v);
          }
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2) {
            const int c = 2 * cp + c2;
            const bf16x8 bv = as_bf16x8(ldg16(bq + (int64_t)l * B * B + (int64_t)(c * 16 + (lane & 15)) * B +
                                              kc * 32 + 8 * (lane >> 4)));
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) acc[c2][tt] = mfma16(af[tt], bv, acc[c2][tt]);
          }
        }
      }
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          res[s][2 * cp + c2][tt][0] = pack2(f32_to_bits(acc[c2][tt][0]), f32_to_bits(acc[c2][tt][1]));
          res[s][2 * cp + c2][tt][1] = pack2(f32_to_bits(acc[c2][tt][2]), f32_to_bits(acc[c2][tt][3]));
          // materialise the packed bf16 pair here (not as fp32 until the scatter)
          asm volatile("" : "+v"(res[s][2 * cp + c2][tt][0]), "+v"(res[s][2 * cp + c2][tt][1]));
        }
    }
  }

  // ---- phase S: scatter results into LDS rows (true layout), write rows out
  for (int p0 = 0; p0 < T; p0 += TP) {
    const int np = min(TP, T - p0);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int l = wave * NS + s;
      if (l < k) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int col = a.perm[l * B + c * 16 + (lane & 15)];
#pragma unroll
          for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int tl = tt * 16 + 4 * (lane >> 4) + r;
              if (tl >= p0 && tl < p0 + np) {
                const uint32_t w = res[s][c][tt][r >> 1];
                lds[(tl - p0) * pitch + col] = (r & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffff);
              }
            }
        }
      }
    }
    const int tail = W - tail0;
    if (tail > 0) {
      for (int e = tid; e < np * tail; e += nt) {
        const int r = e / tail, i = tail0 + (e - r * tail);
        const int64_t t = t0 + p0 + r;
        if (t < N) lds[r * pitch + a.perm[i]] = in[t * W + i];
      }
    }
    __syncthreads();
    unstage_rows(out, N, W, pitch, t0 + p0, np, lds, tid, nt);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// configuration table: (B, TT, NS, MAXT); a shape takes the first entry whose
// capacity NS * MAXT/64 covers its block count, preferring more tokens per tile.
// ---------------------------------------------------------------------------
struct XCfg { int B, TT, NS, MAXT; };
static const XCfg kCfgs[] = {
    {256, 4, 1, 512}, {256, 2, 1, 1024}, {256, 2, 2, 768}, {256, 1, 4, 768},
    {512, 2, 1, 512}, {512, 1, 1, 1024}, {512, 1, 2, 768},
    {128, 2, 2, 1024}, {128, 1, 6, 1024},
    {64, 2, 4, 1024}, {64, 1, 11, 1024},
    {32, 4, 2, 1024}, {32, 2, 8, 1024},
};

template <int B, int TT, int NS, int MAXT>
static void launch_xf(bool gather, const XformArgs& a, int nw, hipStream_t s) {
  const int T = 16 * TT;
  dim3 grid((unsigned)((a.N + T - 1) / T));
  if (gather) hipLaunchKernelGGL((gather_in_kernel<B, TT, NS, MAXT>), grid, dim3(64 * nw), 0, s, a);
  else hipLaunchKernelGGL((scatter_out_kernel<B, TT, NS, MAXT>), grid, dim3(64 * nw), 0, s, a);
}

static bool launch_xform_bf16(bool gather, const XformArgs& a, hipStream_t s) {
  if (a.N <= 0) return true;
  for (const XCfg& c : kCfgs) {
    if (c.B != a.B) continue;
    const int cap = c.NS * (c.MAXT / 64);
    if (a.k > cap) continue;
    int nw = (a.k + c.NS - 1) / c.NS;
    if (nw < 4) nw = 4 < c.MAXT / 64 ? 4 : c.MAXT / 64;  // enough threads for staging
#define XF_CASE(B_, TT_, NS_, MT_) \
  if (c.B == B_ && c.TT == TT_ && c.NS == NS_ && c.MAXT == MT_) { launch_xf<B_, TT_, NS_, MT_>(gather, a, nw, s); return true; }
    XF_CASE(256, 4, 1, 512) XF_CASE(256, 2, 1, 1024) XF_CASE(256, 2, 2, 768) XF_CASE(256, 1, 4, 768)
    XF_CASE(512, 2, 1, 512) XF_CASE(512, 1, 1, 1024) XF_CASE(512, 1, 2, 768)
    XF_CASE(128, 2, 2, 1024) XF_CASE(128, 1, 6, 1024)
    XF_CASE(64, 2, 4, 1024) XF_CASE(64, 1, 11, 1024)
    XF_CASE(32, 4, 2, 1024) XF_CASE(32, 2, 8, 1024)
#undef XF_CASE
  }
  return false;
}

bool launch_gather_in_bf16(const XformArgs& a, hipStream_t s) { return launch_xform_bf16(true, a, s); }
bool launch_scatter_out_bf16(const XformArgs& a, hipStream_t s) { return launch_xform_bf16(false, a, s); }

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
