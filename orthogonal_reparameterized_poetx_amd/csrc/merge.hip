// Merge W0 <- R W0 P with generator reset and re-permutation
// [P3 "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
// Transformation", Methodologie item 1: the weight update W <- R_i W P_i].
//
// In the working layout (W0p = W0 with rows permuted by sigma and columns by
// tau, [P3 item 2]) R and P become block-diagonal, so the merge is an
// independent b x b tile product W0p[I, J] <- Q_R,I W0p[I, J] Q_P,J (identity
// on tail rows/columns).  The result is then relaid to the new permutations.
// New permutations are drawn on the device from SplitMix64 keys
// (Steele, Lea & Flood 2014) sorted by counting rank.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace poetx {

// ---------------------------------------------------------------------------
// bf16 tile merge.  Workgroup = (row group I, column slab of SW columns inside
// column group J).  Step 1: U^T[slab][rows of I] = Q_P,J^T[slab][:] W[I, J]^T
// (MFMA, rounded to bf16 into LDS; tail column group: U = W).  Step 2:
// V[I, slab] = Q_R,I U[:, slab] (tail row group: V = U).
// ---------------------------------------------------------------------------
constexpr int MRG_MAXB = 512;
constexpr int MRG_UP = MRG_MAXB + 8;  // LDS pitch of U^T rows

__global__ __launch_bounds__(256) void merge_tiles_bf16_kernel(const uint16_t* __restrict__ W, uint16_t* __restrict__ V,
                                                               const uint16_t* __restrict__ qr,
                                                               const uint16_t* __restrict__ qpt, int m, int n, int b,
                                                               int kR, int kP, int SW, int slabs_per_row) {
  __shared__ __align__(16) uint16_t Ut[64 * MRG_UP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int I = blockIdx.y;                      // row group
  const int slab = blockIdx.x;                   // global column slab index
  const int c0 = slab * SW;                      // first column of the slab
  if (c0 >= n) return;
  const int J = c0 / b;                          // column group (J == kP: tail)
  const int r0 = I * b;
  const int rows = min(b, m - r0);               // rows in this row group
  const int cols = min(SW, n - c0);              // columns in this slab
  const bool fullJ = J < kP, fullI = I < kR;
  const int lc = lane & 31, hi = lane >> 5;

  // ---- step 1: Ut[cc][r] = sum_kk QPt[J][c0-J*b+cc][kk] * W[r0+r][J*b+kk]
  const int rtiles = (rows + 31) / 32, ctiles = (cols + 31) / 32;
  if (fullJ) {
    const uint16_t* qpj = qpt + (int64_t)J * b * b;
    const int cb = c0 - J * b;
    for (int p = wave; p < rtiles * ctiles; p += 4) {
      const int rt = p % rtiles, ct = p / rtiles;
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
      const int cc = ct * 32 + lc;            // A-operand row (slab column)
      const int rr = rt * 32 + lc;            // B-operand column (weight row)
      const bool cok = cc < cols, rok = rr < rows;
      for (int ks = 0; ks < b / 16; ++ks) {
        const int kk = ks * 16 + 8 * hi;
        const uint4 av = cok ? ldg16(qpj + (int64_t)(cb + cc) * b + kk) : make_uint4(0, 0, 0, 0);
        const uint4 bv = rok ? ldg16(W + (int64_t)(r0 + rr) * n + J * b + kk) : make_uint4(0, 0, 0, 0);
        acc = mfma32(as_bf16x8(av), as_bf16x8(bv), acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int crow = ct * 32 + c32_row(lane, r);
        Ut[crow * MRG_UP + rt * 32 + lc] = f32_to_bits(acc[r]);
      }
    }
  } else {
    for (int e = tid; e < cols * rows; e += 256) {
      const int r = e / cols, cc = e - r * cols;
      Ut[cc * MRG_UP + r] = W[(int64_t)(r0 + r) * n + c0 + cc];
    }
  }
  __syncthreads();

  // ---- step 2: V[r0+i][c0+cc] = sum_r QR[I][i][r] * Ut[cc][r]
  if (fullI) {
    const uint16_t* qri = qr + (int64_t)I * b * b;
    const int itiles = b / 32;
    for (int p = wave; p < itiles * ctiles; p += 4) {
      const int it = p % itiles, ct = p / itiles;
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
      const int ii = it * 32 + lc;
      const int cc = ct * 32 + lc;
      for (int ks = 0; ks < b / 16; ++ks) {
        const int kk = ks * 16 + 8 * hi;
        const uint4 av = ldg16(qri + (int64_t)ii * b + kk);
        const uint4 bv = *reinterpret_cast<const uint4*>(&Ut[cc * MRG_UP + kk]);
        acc = mfma32(as_bf16x8(av), as_bf16x8(bv), acc);
      }
      if (cc < cols) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = it * 32 + c32_row(lane, r);
          V[(int64_t)(r0 + i) * n + c0 + cc] = f32_to_bits(acc[r]);
        }
      }
    }
  } else {
    for (int e = tid; e < rows * cols; e += 256) {
      const int r = e / cols, cc = e - r * cols;
      V[(int64_t)(r0 + r) * n + c0 + cc] = Ut[cc * MRG_UP + r];
    }
  }
}

// fp32 merge in two element-wise passes (U = W D_P, V = D_R U)
__global__ void merge_right_f32_kernel(const float* __restrict__ W, float* __restrict__ U, const float* __restrict__ qp,
                                       int m, int n, int b, int kP) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)m * n) return;
  const int r = (int)(e / n), c = (int)(e % n);
  const int J = c / b;
  if (J >= kP) { U[e] = W[e]; return; }
  const int cc = c - J * b;
  const float* q = qp + (int64_t)J * b * b;
  float s = 0.f;
  for (int kk = 0; kk < b; ++kk) s = fmaf(W[(int64_t)r * n + J * b + kk], q[(int64_t)kk * b + cc], s);
  U[e] = s;
}

__global__ void merge_left_f32_kernel(const float* __restrict__ U, float* __restrict__ V, const float* __restrict__ qr,
                                      int m, int n, int b, int kR) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)m * n) return;
  const int r = (int)(e / n), c = (int)(e % n);
  const int I = r / b;
  if (I >= kR) { V[e] = U[e]; return; }
  const int ii = r - I * b;
  const float* q = qr + (int64_t)I * b * b;
  float s = 0.f;
  for (int kk = 0; kk < b; ++kk) s = fmaf(q[(int64_t)ii * b + kk], U[(int64_t)(I * b + kk) * n + c], s);
  V[e] = s;
}

void launch_merge_tiles(bool f32, const void* W, void* V, const void* qr, const void* qpt, int64_t m, int64_t n, int b,
                        int kR, int kP, hipStream_t s) {
  if (m <= 0 || n <= 0) return;
  if (f32) {
    // V doubles as the intermediate: U into V, then in place is not possible,
    // so the caller passes V with room for two matrices.
    float* U = static_cast<float*>(V) + m * n;
    const int64_t tot = m * n;
    hipLaunchKernelGGL(merge_right_f32_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s,
                       static_cast<const float*>(W), U, static_cast<const float*>(qpt), (int)m, (int)n, b, kP);
    hipLaunchKernelGGL(merge_left_f32_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, U,
                       static_cast<float*>(V), static_cast<const float*>(qr), (int)m, (int)n, b, kR);
    return;
  }
  const int SW = b < 64 ? b : 64;
  const int slabs = (int)((n + SW - 1) / SW);
  const int rgroups = (int)((m + b - 1) / b);
  hipLaunchKernelGGL(merge_tiles_bf16_kernel, dim3(slabs, rgroups), dim3(256), 0, s, static_cast<const uint16_t*>(W),
                     static_cast<uint16_t*>(V), static_cast<const uint16_t*>(qr), static_cast<const uint16_t*>(qpt),
                     (int)m, (int)n, b, kR, kP, SW, slabs);
}

// ---------------------------------------------------------------------------
// permutations
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t mix64_dev(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ void perm_keys_kernel(uint64_t seed, uint64_t merge_index, int side, int64_t n, uint64_t* keys) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint64_t g = 0x9E3779B97F4A7C15ull;
  const uint64_t base = mix64_dev(seed + g * (2 * merge_index + (uint64_t)side + 1));
  keys[i] = mix64_dev(base + g * (uint64_t)(i + 1));
}

// out[rank(i)] = i with rank(i) = #{j : (key_j, j) < (key_i, i)}.  Each of
// the 16 indices of a workgroup is ranked by 16 lanes that split the scan
// over j and sum their counts with cross-lane shuffles.
constexpr int RANK_I = 16, RANK_J = 16, RANK_TILE = 2048;
__global__ __launch_bounds__(RANK_I * RANK_J) void perm_rank_kernel(const uint64_t* __restrict__ keys, int64_t n,
                                                                    int32_t* out) {
  __shared__ uint64_t tile[RANK_TILE];
  const int li = threadIdx.x / RANK_J, lj = threadIdx.x % RANK_J;
  const int64_t i = (int64_t)blockIdx.x * RANK_I + li;
  const uint64_t ki = i < n ? keys[i] : 0;
  int rank = 0;
  for (int64_t j0 = 0; j0 < n; j0 += RANK_TILE) {
    const int cnt = (int)min((int64_t)RANK_TILE, n - j0);
    __syncthreads();
    for (int e = threadIdx.x; e < cnt; e += RANK_I * RANK_J) tile[e] = keys[j0 + e];
    __syncthreads();
    for (int e = lj; e < cnt; e += RANK_J) {
      const uint64_t kj = tile[e];
      const int64_t j = j0 + e;
      rank += (kj < ki) || (kj == ki && j < i);
    }
  }
#pragma unroll
  for (int off = RANK_J / 2; off > 0; off >>= 1) rank += __shfl_xor(rank, off, RANK_J);
  if (i < n && lj == 0) out[rank] = (int32_t)i;
}

void launch_perm_keys_rank(uint64_t seed, uint64_t merge_index, int side, int64_t n, uint64_t* keys, int32_t* out,
                           hipStream_t s) {
  if (n <= 0) return;
  const unsigned g = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(perm_keys_kernel, dim3(g), dim3(256), 0, s, seed, merge_index, side, n, keys);
  hipLaunchKernelGGL(perm_rank_kernel, dim3((unsigned)((n + RANK_I - 1) / RANK_I)), dim3(RANK_I * RANK_J), 0, s, keys,
                     n, out);
}

// Both sides of a merge in one launch each (workgroups [0, blocks0) take the
// row side, the rest the column side): the counting rank computes the keys as
// it goes instead of reading them from memory.
__device__ __forceinline__ uint64_t perm_key(uint64_t base, int64_t j) {
  return mix64_dev(base + 0x9E3779B97F4A7C15ull * (uint64_t)(j + 1));
}
__global__ __launch_bounds__(RANK_I * RANK_J) void perm_rank2_kernel(uint64_t seed, uint64_t merge_index, int64_t n0,
                                                                     int64_t n1, int32_t* out0, int32_t* out1,
                                                                     int blocks0) {
  __shared__ uint64_t tile[RANK_TILE];
  const int side = (int)blockIdx.x < blocks0 ? 0 : 1;
  const int64_t n = side ? n1 : n0;
  int32_t* out = side ? out1 : out0;
  const int64_t blk = side ? (int64_t)blockIdx.x - blocks0 : (int64_t)blockIdx.x;
  const uint64_t base = mix64_dev(seed + 0x9E3779B97F4A7C15ull * (2 * merge_index + (uint64_t)side + 1));
  const int li = threadIdx.x / RANK_J, lj = threadIdx.x % RANK_J;
  const int64_t i = blk * RANK_I + li;
  const uint64_t ki = i < n ? perm_key(base, i) : 0;
  int rank = 0;
  for (int64_t j0 = 0; j0 < n; j0 += RANK_TILE) {
    const int cnt = (int)min((int64_t)RANK_TILE, n - j0);
    __syncthreads();
    for (int e = threadIdx.x; e < cnt; e += RANK_I * RANK_J) tile[e] = perm_key(base, j0 + e);
    __syncthreads();
    for (int e = lj; e < cnt; e += RANK_J) {
      const uint64_t kj = tile[e];
      const int64_t j = j0 + e;
      rank += (kj < ki) || (kj == ki && j < i);
    }
  }
#pragma unroll
  for (int off = RANK_J / 2; off > 0; off >>= 1) rank += __shfl_xor(rank, off, RANK_J);
  if (i < n && lj == 0) out[rank] = (int32_t)i;
}
// inv0 = p0^-1 (first n0 threads), inv1 = p1^-1
__global__ void invert_perm2_kernel(const int32_t* __restrict__ p0, int64_t n0, int32_t* __restrict__ inv0,
                                    const int32_t* __restrict__ p1, int64_t n1, int32_t* __restrict__ inv1) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e < n0) inv0[p0[e]] = (int32_t)e;
  else if (e < n0 + n1) inv1[p1[e - n0]] = (int32_t)(e - n0);
}
// commit the new permutations and turn them into the relayout's maps:
// cur[i] <- nw[i], nw[i] <- inv[nw[i]] (per side)
__global__ void commit_perm2_kernel(int32_t* nw0, int32_t* cur0, const int32_t* __restrict__ inv0, int64_t n0,
                                    int32_t* nw1, int32_t* cur1, const int32_t* __restrict__ inv1, int64_t n1) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e < n0) {
    const int32_t v = nw0[e];
    cur0[e] = v;
    nw0[e] = inv0[v];
  } else if (e < n0 + n1) {
    const int64_t i = e - n0;
    const int32_t v = nw1[i];
    cur1[i] = v;
    nw1[i] = inv1[v];
  }
}
void launch_merge_permutations(uint64_t seed, uint64_t merge_index, int32_t* sigma, int32_t* tau, int64_t m, int64_t n,
                               int32_t* snew, int32_t* tnew, int32_t* sinv, int32_t* tinv, hipStream_t s) {
  if (m <= 0 && n <= 0) return;
  const int b0 = (int)((m + RANK_I - 1) / RANK_I), b1 = (int)((n + RANK_I - 1) / RANK_I);
  hipLaunchKernelGGL(perm_rank2_kernel, dim3((unsigned)(b0 + b1)), dim3(RANK_I * RANK_J), 0, s, seed, merge_index, m, n,
                     snew, tnew, b0);
  const unsigned g = (unsigned)((m + n + 255) / 256);
  hipLaunchKernelGGL(invert_perm2_kernel, dim3(g), dim3(256), 0, s, sigma, m, sinv, tau, n, tinv);
  hipLaunchKernelGGL(commit_perm2_kernel, dim3(g), dim3(256), 0, s, snew, sigma, sinv, m, tnew, tau, tinv, n);
}

__global__ void invert_perm_kernel(const int32_t* __restrict__ p, int64_t n, int32_t* __restrict__ inv) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) inv[p[i]] = (int32_t)i;
}

void launch_invert_perm(const int32_t* p, int64_t n, int32_t* inv, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(invert_perm_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, inv);
}

// W[i][j] = V[sinv_old[snew[i]]][tinv_old[tnew[j]]], one row per workgroup.
// bf16 rows (n <= 32768) are staged in LDS so the column gather hits LDS; the
// fp32 path (small layers) gathers straight from the cached source row.
__global__ __launch_bounds__(256) void relayout_bf16_kernel(const uint16_t* __restrict__ V, uint16_t* __restrict__ W,
                                                            const int32_t* __restrict__ sinv,
                                                            const int32_t* __restrict__ snew,
                                                            const int32_t* __restrict__ tinv,
                                                            const int32_t* __restrict__ tnew, int n) {
  __shared__ __align__(16) uint16_t row[32768];
  const int i = blockIdx.x;
  const int src = sinv[snew[i]];
  for (int c = threadIdx.x; c < n; c += blockDim.x) row[c] = V[(int64_t)src * n + c];
  __syncthreads();
  for (int j = threadIdx.x; j < n; j += blockDim.x) W[(int64_t)i * n + j] = row[tinv[tnew[j]]];
}

__global__ __launch_bounds__(256) void relayout_f32_kernel(const float* __restrict__ V, float* __restrict__ W,
                                                           const int32_t* __restrict__ sinv,
                                                           const int32_t* __restrict__ snew,
                                                           const int32_t* __restrict__ tinv,
                                                           const int32_t* __restrict__ tnew, int n) {
  const int i = blockIdx.x;
  const float* src = V + (int64_t)sinv[snew[i]] * n;
  for (int j = threadIdx.x; j < n; j += blockDim.x) W[(int64_t)i * n + j] = src[tinv[tnew[j]]];
}

void launch_relayout(bool f32, const void* V, void* W, const int32_t* sinv_old, const int32_t* snew,
                     const int32_t* tinv_old, const int32_t* tnew, int64_t m, int64_t n, hipStream_t s) {
  if (m <= 0 || n <= 0) return;
  if (f32)
    hipLaunchKernelGGL(relayout_f32_kernel, dim3((unsigned)m), dim3(256), 0, s, static_cast<const float*>(V),
                       static_cast<float*>(W), sinv_old, snew, tinv_old, tnew, (int)n);
  else
    hipLaunchKernelGGL(relayout_bf16_kernel, dim3((unsigned)m), dim3(256), 0, s, static_cast<const uint16_t*>(V),
                       static_cast<uint16_t*>(W), sinv_old, snew, tinv_old, tnew, (int)n);
}

// dst[r][:] = src[r][:] for r < rows (16-byte chunks; n multiple of 8)
__global__ void copy_rows_bf16_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t chunks) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < chunks; e += (int64_t)gridDim.x * blockDim.x)
    dst[e] = src[e];
}
void launch_copy_rows_bf16(const uint16_t* src, uint16_t* dst, int64_t rows, int64_t n, hipStream_t s) {
  const int64_t chunks = rows * n / 8;
  if (chunks <= 0) return;
  const int64_t g = std::min<int64_t>((chunks + 255) / 256, 4096);
  hipLaunchKernelGGL(copy_rows_bf16_kernel, dim3((unsigned)g), dim3(256), 0, s, reinterpret_cast<const uint4*>(src),
                     reinterpret_cast<uint4*>(dst), chunks);
}

// W[i][j] = V[rmap[i]][cmap[j]] for bf16 rows of n columns (n multiple of 8,
// 16-byte aligned rows): R source rows per workgroup are staged in LDS with
// asynchronous 16-byte loads (one contiguous KiB per wave instruction), then
// every thread gathers 8-column chunks through LDS, reading each chunk's 8
// column indices once for all R rows, and writes them as 16-byte stores.
constexpr int RL_THREADS = 256;
__global__ __launch_bounds__(RL_THREADS) void relayout_rows_bf16_kernel(const uint16_t* __restrict__ V,
                                                                        uint16_t* __restrict__ W,
                                                                        const int32_t* __restrict__ rmap,
                                                                        const int32_t* __restrict__ cmap, int64_t m,
                                                                        int n, int R) {
  extern __shared__ __align__(16) uint16_t rows[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t t0 = (int64_t)blockIdx.x * R;
  const int nr = (int)min((int64_t)R, m - t0);
  const int cpr = (n + 511) >> 9;   // 1 KiB chunks per row
  for (int c = wave; c < nr * cpr; c += RL_THREADS / 64) {
    const int r = c / cpr, j = c - r * cpr;
    const int e0 = (j << 9) + lane * 8;
    if (e0 < n)
      __builtin_amdgcn_global_load_lds(V + (int64_t)rmap[t0 + r] * n + e0,
                                       (__attribute__((address_space(3))) void*)(rows + r * n + (j << 9)), 16, 0, 0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  uint16_t* __restrict__ out = W + t0 * n;
  for (int c = tid; c < (n >> 3); c += RL_THREADS) {
    const int4 pa = *reinterpret_cast<const int4*>(cmap + c * 8);
    const int4 pb = *reinterpret_cast<const int4*>(cmap + c * 8 + 4);
    for (int r = 0; r < nr; ++r) {
      const uint16_t* row = rows + r * n;
      uint4 v;
      v.x = pack2(row[pa.x], row[pa.y]);
      v.y = pack2(row[pa.z], row[pa.w]);
      v.z = pack2(row[pb.x], row[pb.y]);
      v.w = pack2(row[pb.z], row[pb.w]);
      stg16(out + (int64_t)r * n + c * 8, v);
    }
  }
}
bool launch_relayout_rows_bf16(const uint16_t* V, uint16_t* W, const int32_t* rmap, const int32_t* cmap, int64_t m,
                               int64_t n, hipStream_t s) {
  if (m <= 0 || n <= 0) return true;
  if ((n & 7) || n > 32768 || (reinterpret_cast<uintptr_t>(V) & 15) || (reinterpret_cast<uintptr_t>(W) & 15) ||
      (reinterpret_cast<uintptr_t>(cmap) & 15))
    return false;
  int R = (int)(32768 / n);
  R = R < 1 ? 1 : (R > 16 ? 16 : R);
  const size_t lds = (size_t)R * n * sizeof(uint16_t);
  hipLaunchKernelGGL(relayout_rows_bf16_kernel, dim3((unsigned)((m + R - 1) / R)), dim3(RL_THREADS), lds, s, V, W,
                     rmap, cmap, m, (int)n, R);
  return true;
}

__global__ void copy_i32_kernel(const int32_t* __restrict__ src, int32_t* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}
void launch_copy_i32(const int32_t* src, int32_t* dst, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(copy_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, dst, n);
}

__global__ void fill_f32_kernel(float* p, float v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}
void launch_fill_f32(float* p, float v, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, v, n);
}

// Adam (Kingma & Ba 2015, Algorithm 1), bias corrections passed in
__global__ void adam_kernel(float* __restrict__ th, const float* __restrict__ g, float* __restrict__ m,
                            float* __restrict__ v, int64_t n, float lr, float b1, float b2, float eps, float bc1,
                            float bc2) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float gi = g[i];
  const float mi = b1 * m[i] + (1.f - b1) * gi;
  const float vi = b2 * v[i] + (1.f - b2) * gi * gi;
  m[i] = mi;
  v[i] = vi;
  th[i] = th[i] - lr * (mi / bc1) / (sqrtf(vi / bc2) + eps);
}
void launch_adam(float* theta, const float* grad, float* m, float* v, int64_t n, float lr, float b1, float b2,
                 float eps, float bc1, float bc2, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(adam_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, theta, grad, m, v, n, lr, b1, b2,
                     eps, bc1, bc2);
}

}  // namespace poetx
