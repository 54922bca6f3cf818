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
// The item of a batched launch that workgroup g belongs to (starts[k] is
// its first workgroup).
__device__ __forceinline__ int batch_item(const MergeBatch& b, int g) {
  int k = 0;
  while (k + 1 < b.count && g >= b.start[k + 1]) ++k;
  return k;
}

// Per item: workgroups [0, b0) rank the row side, [b0, b0 + b1) the column
// side, and the rest invert the old permutations (sinv = sigma^-1, tinv =
// tau^-1), which the same launch can do: they read only sigma, tau.
__global__ __launch_bounds__(RANK_I * RANK_J) void perm_rank2_kernel(MergeBatch bt) {
  __shared__ uint64_t tile[RANK_TILE];
  const int kb = batch_item(bt, (int)blockIdx.x);
  const MergeItem& it = bt.it[kb];
  const int lb = (int)blockIdx.x - bt.start[kb];
  const int64_t n0 = it.m, n1 = it.n;
  const int blocks0 = (int)((n0 + RANK_I - 1) / RANK_I), blocks01 = blocks0 + (int)((n1 + RANK_I - 1) / RANK_I);
  if (lb >= blocks01) {
    const int64_t e = (int64_t)(lb - blocks01) * (RANK_I * RANK_J) + threadIdx.x;
    if (e < n0) it.sinv[it.sigma[e]] = (int32_t)e;
    else if (e < n0 + n1) it.tinv[it.tau[e - n0]] = (int32_t)(e - n0);
    return;
  }
  const int side = lb < blocks0 ? 0 : 1;
  const int64_t n = side ? n1 : n0;
  int32_t* out = side ? it.tnew : it.snew;
  const int64_t blk = side ? (int64_t)lb - blocks0 : (int64_t)lb;
  const uint64_t base = mix64_dev(it.seed + 0x9E3779B97F4A7C15ull * (2 * it.merge_index + (uint64_t)side + 1));
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
// commit the new permutations and turn them into the relayout's maps:
// cur[i] <- nw[i], nw[i] <- inv[nw[i]] (per side)
__global__ void commit_perm2_kernel(MergeBatch bt) {
  const int k = batch_item(bt, (int)blockIdx.x);
  const MergeItem& it = bt.it[k];
  const int64_t e = (int64_t)((int)blockIdx.x - bt.start[k]) * blockDim.x + threadIdx.x;
  if (e < it.m) {
    const int32_t v = it.snew[e];
    it.sigma[e] = v;
    it.snew[e] = it.sinv[v];
  } else if (e < it.m + it.n) {
    const int64_t i = e - it.m;
    const int32_t v = it.tnew[i];
    it.tau[i] = v;
    it.tnew[i] = it.tinv[v];
  }
}
void launch_merge_permutations_batch(const MergeBatch& b, hipStream_t s) {
  if (b.count <= 0) return;
  MergeBatch t = b;
  int tot = 0;
  for (int k = 0; k < t.count; ++k) {
    t.start[k] = tot;
    const MergeItem& it = t.it[k];
    tot += (int)((it.m + RANK_I - 1) / RANK_I) + (int)((it.n + RANK_I - 1) / RANK_I) +
           (int)((it.m + it.n + RANK_I * RANK_J - 1) / (RANK_I * RANK_J));
  }
  t.start[t.count] = tot;
  if (tot > 0) hipLaunchKernelGGL(perm_rank2_kernel, dim3((unsigned)tot), dim3(RANK_I * RANK_J), 0, s, t);
  tot = 0;
  for (int k = 0; k < t.count; ++k) {
    t.start[k] = tot;
    tot += (int)((t.it[k].m + t.it[k].n + 255) / 256);
  }
  t.start[t.count] = tot;
  if (tot > 0) hipLaunchKernelGGL(commit_perm2_kernel, dim3((unsigned)tot), dim3(256), 0, s, t);
}
void launch_merge_permutations(uint64_t seed, uint64_t merge_index, int32_t* sigma, int32_t* tau, int64_t m, int64_t n,
                               int32_t* snew, int32_t* tnew, int32_t* sinv, int32_t* tinv, hipStream_t s) {
  if (m <= 0 && n <= 0) return;
  MergeBatch b{};
  b.count = 1;
  MergeItem& it = b.it[0];
  it.sigma = sigma; it.tau = tau; it.snew = snew; it.tnew = tnew; it.sinv = sinv; it.tinv = tinv;
  it.m = m; it.n = n; it.seed = seed; it.merge_index = merge_index;
  launch_merge_permutations_batch(b, s);
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

// ---------------------------------------------------------------------------
// In-place merge: the products act on W0p where it lies, and the relayout
// W'[i][j] = W[rho(i)][kappa(j)] moves rows along the cycles of rho.
// ---------------------------------------------------------------------------

// P side, bf16, any b: W[r][J b + c] <- bf16(sum_k W[r][J b + k] Q_P,J[k][c])
// for full column groups J < kP.  Workgroup = (32 rows, group J): the rows'
// segment of group J is staged in LDS before anything is written, and no
// other workgroup reads or writes it, so the update is in place.  Same
// operands and MFMA order as merge_tiles_bf16_kernel's first step.
constexpr int PROW_R = 32;
__global__ __launch_bounds__(256) void merge_prow_bf16_kernel(uint16_t* W, const uint16_t* __restrict__ qpt, int m,
                                                              int n, int b, int kP) {
  __shared__ __align__(16) uint16_t seg[PROW_R * (MRG_MAXB + 8)];
  const int pitch = b + 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int J = blockIdx.y;
  const int r0 = blockIdx.x * PROW_R;
  const int rows = min(PROW_R, m - r0);
  if (J >= kP || rows <= 0) return;
  for (int e = tid; e < rows * b; e += 256) {
    const int r = e / b, k = e - r * b;
    seg[r * pitch + k] = W[(int64_t)(r0 + r) * n + (int64_t)J * b + k];
  }
  __syncthreads();
  const uint16_t* qpj = qpt + (int64_t)J * b * b;
  const int lc = lane & 31, hi = lane >> 5;
  const int ctiles = b / 32;
  for (int ct = wave; ct < ctiles; ct += 4) {
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    const int cc = ct * 32 + lc;            // A-operand row: output column within the group
    const bool rok = lc < rows;             // B-operand column: weight row
    for (int ks = 0; ks < b / 16; ++ks) {
      const int kk = ks * 16 + 8 * hi;
      const uint4 av = ldg16(qpj + (int64_t)cc * b + kk);
      const uint4 bv = rok ? *reinterpret_cast<const uint4*>(&seg[lc * pitch + kk]) : make_uint4(0, 0, 0, 0);
      acc = mfma32(as_bf16x8(av), as_bf16x8(bv), acc);
    }
    if (rok) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int col = ct * 32 + c32_row(lane, r);
        W[(int64_t)(r0 + lc) * n + (int64_t)J * b + col] = f32_to_bits(acc[r]);
      }
    }
  }
}

// R side, bf16, any b: W[I b + i][c] <- bf16(sum_k Q_R,I[i][k] W[I b + k][c])
// for full row groups I < kR.  Workgroup = (group I, slab of 64 columns):
// the slab of the group's rows is staged in LDS first; same operands and MFMA
// order as merge_tiles_bf16_kernel's second step.
constexpr int RCOL_SW = 64;
__global__ __launch_bounds__(256) void merge_rcol_bf16_kernel(uint16_t* W, const uint16_t* __restrict__ qr, int m, int n,
                                                              int b, int kR) {
  __shared__ __align__(16) uint16_t Ut[RCOL_SW * MRG_UP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int I = blockIdx.y;
  const int c0 = blockIdx.x * RCOL_SW;
  const int cols = min(RCOL_SW, n - c0);
  if (I >= kR || cols <= 0) return;
  const int r0 = I * b;
  for (int e = tid; e < cols * b; e += 256) {
    const int r = e / cols, cc = e - r * cols;
    Ut[cc * MRG_UP + r] = W[(int64_t)(r0 + r) * n + c0 + cc];
  }
  __syncthreads();
  const uint16_t* qri = qr + (int64_t)I * b * b;
  const int lc = lane & 31, hi = lane >> 5;
  const int itiles = b / 32, ctiles = (cols + 31) / 32;
  for (int p = wave; p < itiles * ctiles; p += 4) {
    const int it = p % itiles, ct = p / itiles;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    const int ii = it * 32 + lc;
    const int cc = ct * 32 + lc;
    const bool cok = cc < cols;
    for (int ks = 0; ks < b / 16; ++ks) {
      const int kk = ks * 16 + 8 * hi;
      const uint4 av = ldg16(qri + (int64_t)ii * b + kk);
      const uint4 bv = cok ? *reinterpret_cast<const uint4*>(&Ut[cc * MRG_UP + kk]) : make_uint4(0, 0, 0, 0);
      acc = mfma32(as_bf16x8(av), as_bf16x8(bv), acc);
    }
    if (cok) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = it * 32 + c32_row(lane, r);
        W[(int64_t)(r0 + i) * n + c0 + cc] = f32_to_bits(acc[r]);
      }
    }
  }
}

// fp32, in place: P side one row per workgroup (the row staged in LDS), R
// side one (row group, 32-column slab) per workgroup (the slab staged); the
// sums run in the order of merge_right_f32_kernel / merge_left_f32_kernel.
__global__ __launch_bounds__(256) void merge_prow_f32_kernel(float* W, const float* __restrict__ qp, int n, int b,
                                                             int kP) {
  __shared__ float row[32768];
  const int r = blockIdx.x;
  float* w = W + (int64_t)r * n;
  for (int c = threadIdx.x; c < kP * b; c += 256) row[c] = w[c];
  __syncthreads();
  for (int c = threadIdx.x; c < kP * b; c += 256) {
    const int J = c / b, cc = c - J * b;
    const float* q = qp + (int64_t)J * b * b;
    float s = 0.f;
    for (int kk = 0; kk < b; ++kk) s = fmaf(row[J * b + kk], q[(int64_t)kk * b + cc], s);
    w[c] = s;
  }
}
constexpr int RCOL_F32_SW = 32;
__global__ __launch_bounds__(256) void merge_rcol_f32_kernel(float* W, const float* __restrict__ qr, int n, int b,
                                                             int kR) {
  __shared__ float slab[MRG_MAXB * RCOL_F32_SW];
  const int I = blockIdx.y;
  const int c0 = blockIdx.x * RCOL_F32_SW;
  const int cols = min(RCOL_F32_SW, n - c0);
  if (I >= kR || cols <= 0) return;
  const int64_t r0 = (int64_t)I * b;
  for (int e = threadIdx.x; e < b * cols; e += 256) {
    const int k = e / cols, cc = e - k * cols;
    slab[k * RCOL_F32_SW + cc] = W[(r0 + k) * n + c0 + cc];
  }
  __syncthreads();
  const float* q = qr + (int64_t)I * b * b;
  for (int e = threadIdx.x; e < b * cols; e += 256) {
    const int ii = e / cols, cc = e - ii * cols;
    float s = 0.f;
    for (int kk = 0; kk < b; ++kk) s = fmaf(q[(int64_t)ii * b + kk], slab[kk * RCOL_F32_SW + cc], s);
    W[(r0 + ii) * n + c0 + cc] = s;
  }
}

void launch_merge_products_inplace(bool f32, void* W, const void* qr, const void* qpt, int64_t m, int64_t n, int b,
                                   int kR, int kP, hipStream_t s) {
  if (m <= 0 || n <= 0) return;
  if (f32) {
    if (kP > 0)
      hipLaunchKernelGGL(merge_prow_f32_kernel, dim3((unsigned)m), dim3(256), 0, s, static_cast<float*>(W),
                         static_cast<const float*>(qpt), (int)n, b, kP);
    if (kR > 0)
      hipLaunchKernelGGL(merge_rcol_f32_kernel, dim3((unsigned)((n + RCOL_F32_SW - 1) / RCOL_F32_SW), (unsigned)kR),
                         dim3(256), 0, s, static_cast<float*>(W), static_cast<const float*>(qr), (int)n, b, kR);
    return;
  }
  if (kP > 0)
    hipLaunchKernelGGL(merge_prow_bf16_kernel, dim3((unsigned)((m + PROW_R - 1) / PROW_R), (unsigned)kP), dim3(256), 0,
                       s, static_cast<uint16_t*>(W), static_cast<const uint16_t*>(qpt), (int)m, (int)n, b, kP);
  if (kR > 0)
    hipLaunchKernelGGL(merge_rcol_bf16_kernel, dim3((unsigned)((n + RCOL_SW - 1) / RCOL_SW), (unsigned)kR), dim3(256),
                       0, s, static_cast<uint16_t*>(W), static_cast<const uint16_t*>(qr), (int)m, (int)n, b, kR);
}

// ---- relayout along the cycles of rho ----------------------------------
// Plan (one workgroup, the map in LDS as 16-bit indices, m <= 32768):
// pointer jumping gives every i its cycle's minimum c (15 doubling rounds),
// then its distance d(i) along rho to c (list ranking with a self-loop at c).
// Heads are the i with d(i) % L == 0, so every cycle is cut into segments of
// at most L positions, each starting at a head and ending just before the
// next one.  A head whose cycle has another head is "saved": its row is
// copied aside before any row moves, because the segment ending at it reads
// it after its own segment has overwritten it.  A cycle with a single head
// (length <= L) keeps that row in its walker's LDS instead.  Saved heads
// number at most sum over long cycles of ceil(len / L) < 2 m / L.
// KP = rows per thread (one of a few counts with 1024 KP >= m): the
// doubling rounds touch only slots that exist (a thread's slots past m are
// skipped in every loop).
constexpr int CP_THREADS = 1024, CP_MAXM = 32768, CP_WAVES = CP_THREADS / 64;
// One workgroup per item of the batch (rho = its snew).
template <int KP>
__global__ __launch_bounds__(CP_THREADS) void cycle_plan_kernel(MergeBatch bt, int L) {
  const MergeItem& it = bt.it[blockIdx.x];
  const int32_t* __restrict__ rho = it.snew;
  const int m = (int)it.m;
  int32_t* __restrict__ dist = it.dist;
  int32_t* __restrict__ hlist = it.hlist;
  int32_t* __restrict__ slot = it.slot;
  int32_t* __restrict__ slist = it.slist;
  int32_t* __restrict__ counts = it.counts;
  int32_t* __restrict__ nxt = it.nxt;
  __shared__ uint16_t A[CP_MAXM], B[CP_MAXM];
  __shared__ int wsH[CP_WAVES], wsS[CP_WAVES];
  const int tid = threadIdx.x;
  int rounds = 0;
  while ((1 << rounds) < m) ++rounds;
  for (int i = tid; i < m; i += CP_THREADS) {
    A[i] = (uint16_t)i;
    B[i] = (uint16_t)rho[i];
  }
  __syncthreads();
  // A(i) = min over i, rho(i), ..., rho^(2^r - 1)(i); B(i) = rho^(2^r)(i)
  for (int r = 0; r < rounds; ++r) {
    uint16_t na[KP], nb[KP];
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int i = tid + k * CP_THREADS;
      if (i < m) {
        const int j = B[i];
        na[k] = min(A[i], A[j]);
        nb[k] = B[j];
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int i = tid + k * CP_THREADS;
      if (i < m) {
        A[i] = na[k];
        B[i] = nb[k];
      }
    }
    __syncthreads();
  }
  // list ranking: A(i) <- 0 at the cycle minimum, 1 elsewhere; B(i) <- rho(i),
  // or i itself at the minimum; then A(i) += A(B(i)), B(i) <- B(B(i))
  for (int i = tid; i < m; i += CP_THREADS) {
    const bool c = A[i] == i;
    A[i] = c ? 0 : 1;
    B[i] = c ? (uint16_t)i : (uint16_t)rho[i];
  }
  __syncthreads();
  for (int r = 0; r < rounds; ++r) {
    uint16_t na[KP], nb[KP];
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int i = tid + k * CP_THREADS;
      if (i < m) {
        const int j = B[i];
        na[k] = (uint16_t)(A[i] + A[j]);
        nb[k] = B[j];
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int i = tid + k * CP_THREADS;
      if (i < m) {
        A[i] = na[k];
        B[i] = nb[k];
      }
    }
    __syncthreads();
  }
  // distances out (coalesced); then, with rho back in B, per row the flags
  // head (d % L == 0) and saved head (a head whose cycle has another head:
  // d > 0, or rho(i)'s distance >= L) into B, and nxt(i) = rho(i), with the
  // sign bit set when rho(i) is a head
  __syncthreads();
  for (int i = tid; i < m; i += CP_THREADS) {
    const int d = A[i];
    dist[i] = d;
    B[i] = (uint16_t)rho[i];
  }
  __syncthreads();
  uint16_t fl[KP];
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const int i = tid + k * CP_THREADS;
    if (i < m) {
      const int d = A[i], q = B[i], dq = A[q];
      const bool h = d % L == 0;
      fl[k] = (uint16_t)(h ? (d > 0 || dq >= L ? 3 : 1) : 0);
      nxt[i] = (dq % L == 0) ? (int32_t)((uint32_t)q | 0x80000000u) : q;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const int i = tid + k * CP_THREADS;
    if (i < m) B[i] = fl[k];
  }
  __syncthreads();
  // heads and saved heads, listed in index order: thread t owns
  // [t * KP, (t + 1) * KP); the slots go through A (as 16 bits,
  // 0xffff for none) so that slot[] is written along rows
  int ch = 0, cs = 0;
  for (int k = 0; k < KP; ++k) {
    const int i = tid * KP + k;
    if (i >= m) break;
    const int f = B[i];
    ch += f & 1;
    cs += f >> 1;
  }
  // prefix sums over the threads: within each wave by lane shifts, then
  // over the wave totals
  const int lane = tid & 63, wave = tid >> 6;
  int ih = ch, is = cs;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int h2 = __shfl_up(ih, off), s2 = __shfl_up(is, off);
    if (lane >= off) {
      ih += h2;
      is += s2;
    }
  }
  if (lane == 63) {
    wsH[wave] = ih;
    wsS[wave] = is;
  }
  __syncthreads();
  if (wave == 0) {
    int th = lane < CP_WAVES ? wsH[lane] : 0, ts = lane < CP_WAVES ? wsS[lane] : 0;
#pragma unroll
    for (int off = 1; off < CP_WAVES; off <<= 1) {
      const int h2 = __shfl_up(th, off), s2 = __shfl_up(ts, off);
      if (lane >= off) {
        th += h2;
        ts += s2;
      }
    }
    if (lane < CP_WAVES) {
      wsH[lane] = th;
      wsS[lane] = ts;
    }
  }
  __syncthreads();
  int oh = (wave ? wsH[wave - 1] : 0) + ih - ch, os = (wave ? wsS[wave - 1] : 0) + is - cs;   // exclusive prefix
  for (int k = 0; k < KP; ++k) {
    const int i = tid * KP + k;
    if (i >= m) break;
    const int f = B[i];
    uint16_t sl = 0xffff;
    if (f & 1) {
      hlist[oh++] = i;
      if (f & 2) {
        sl = (uint16_t)os;
        slist[os++] = i;
      }
    }
    A[i] = sl;
  }
  if (tid == CP_THREADS - 1) {
    counts[0] = wsH[CP_WAVES - 1];
    counts[1] = wsS[CP_WAVES - 1];
  }
  __syncthreads();
  for (int i = tid; i < m; i += CP_THREADS) {
    const int sl = A[i];
    slot[i] = sl == 0xffff ? -1 : sl;
  }
}

// saved[s][:] = W[slist[s]][:] for s < counts[1]; one row per workgroup,
// item blockIdx.y of the batch
template <typename T>
__global__ __launch_bounds__(256) void save_heads_kernel(MergeBatch bt) {
  const MergeItem& it = bt.it[blockIdx.y];
  const int sidx = blockIdx.x;
  if (sidx >= it.counts[1]) return;
  const int n = (int)it.n;
  const T* src = static_cast<const T*>(it.W) + (int64_t)it.slist[sidx] * n;
  T* dst = static_cast<T*>(it.saved) + (int64_t)sidx * n;
  for (int c = threadIdx.x; c < n; c += 256) dst[c] = src[c];
}

// One segment per workgroup: from head h, positions p = h, rho(h), ... while
// rho(p) is not a head: W[p][j] <- W[rho(p)][kappa(j)] (row rho(p) is still
// untouched: only this walker writes it, at its next position); at the last
// position the source is the next head's saved row, or, for a cycle with a
// single head, the head's own row kept in LDS before the first write.
// Barriers separate the positions, so a row is read completely before the
// next position overwrites it.
template <typename T>
__global__ __launch_bounds__(256) void walk_rows_kernel(T* W, const T* __restrict__ saved,
                                                        const int32_t* __restrict__ rho,
                                                        const int32_t* __restrict__ kappa,
                                                        const int32_t* __restrict__ dist,
                                                        const int32_t* __restrict__ hlist,
                                                        const int32_t* __restrict__ slot,
                                                        const int32_t* __restrict__ counts, int n, int L) {
  __shared__ T keep[32768];
  const int g = blockIdx.x;
  if (g >= counts[0]) return;
  const int h = hlist[g];
  const bool single = slot[h] < 0;
  if (single) {
    for (int c = threadIdx.x; c < n; c += 256) keep[c] = W[(int64_t)h * n + c];
    __syncthreads();
  }
  int p = h;
  // a segment has at most L positions (the bound also ends the walk if rho
  // were not a permutation)
  for (int step = 0; step < L; ++step) {
    const int q = rho[p];
    const bool last = dist[q] % L == 0;
    T* dst = W + (int64_t)p * n;
    if (last && single) {
      for (int j = threadIdx.x; j < n; j += 256) dst[j] = keep[kappa[j]];
    } else {
      const T* src = last ? saved + (int64_t)slot[q] * n : W + (int64_t)q * n;
      for (int j = threadIdx.x; j < n; j += 256) dst[j] = src[kappa[j]];
    }
    __syncthreads();
    if (last) break;
    p = q;
  }
}

// The segment walk for bf16 rows of a multiple of 8 columns, 16-byte aligned:
// one thread first chases the segment's positions p_0 = h, p_1, ... (nxt
// flags the next head), then the rows move in chunks through LDS: a chunk's
// source rows (p_{t+1}, or for the last position the next head's saved row,
// or, in a cycle with a single head, the head's own row loaded before any
// write) are all loaded before any of its destinations is written, and a
// destination is never a source of a later chunk.  Each 8-column group reads
// its column indices once for all rows of the chunk.
constexpr int WK_MAXL = 64;
constexpr int WK_SLOTS_BYTES = 144 * 1024;
// Item blockIdx.y of the batch (kappa = its tnew), segment blockIdx.x.
__global__ __launch_bounds__(256) void walk_rows_staged_bf16_kernel(MergeBatch bt, int L) {
  __shared__ __align__(16) uint16_t rows[WK_SLOTS_BYTES / 2];
  __shared__ int pos[WK_MAXL + 1];
  __shared__ int meta[2];
  const MergeItem& it = bt.it[blockIdx.y];
  uint16_t* W = static_cast<uint16_t*>(it.W);
  const uint16_t* __restrict__ saved = static_cast<const uint16_t*>(it.saved);
  const int32_t* __restrict__ nxt = it.nxt;
  const int32_t* __restrict__ hlist = it.hlist;
  const int32_t* __restrict__ slot = it.slot;
  const int32_t* __restrict__ counts = it.counts;
  const int32_t* __restrict__ kappa = it.tnew;
  const int n = (int)it.n;
  const int g = blockIdx.x;
  if (g >= counts[0]) return;
  const int tid = threadIdx.x;
  const int h = hlist[g];
  if (tid == 0) {
    int p = h, c = 0, q = h;
    pos[0] = h;
    for (int step = 0; step < L; ++step) {
      const int v = nxt[p];
      q = v & 0x7fffffff;
      ++c;
      if (v < 0) break;
      pos[c] = q;
      p = q;
    }
    meta[0] = c;   // positions p_0 .. p_{c-1}
    meta[1] = q;   // the next head
  }
  __syncthreads();
  const int c = meta[0], F = meta[1];
  const int sF = slot[F];
  const bool single = sF < 0;     // then F == h: the cycle has this one head
  const int n8 = n >> 3;
  const int C = WK_SLOTS_BYTES / (n * 2);   // row slots (>= 4 for n <= 16384, >= 2 up to 32768)
  auto load_row = [&](const uint16_t* src, int k) {
    uint4* d = reinterpret_cast<uint4*>(rows + (int64_t)k * n);
    const uint4* sv = reinterpret_cast<const uint4*>(src);
    for (int e = tid; e < n8; e += 256) d[e] = sv[e];
  };
  // rows of the chunk [t0, t0 + cnt) go from slot sl(k) to p_{t0 + k}
  auto write_rows = [&](int t0, int cnt, int keep_slot) {
    for (int e = tid; e < n8; e += 256) {
      const int4 pa = *reinterpret_cast<const int4*>(kappa + e * 8);
      const int4 pb = *reinterpret_cast<const int4*>(kappa + e * 8 + 4);
      for (int k = 0; k < cnt; ++k) {
        const int t = t0 + k;
        const int sl = (t == c - 1 && keep_slot >= 0) ? keep_slot : k;
        const uint16_t* row = rows + (int64_t)sl * n;
        uint4 v;
        v.x = pack2(row[pa.x], row[pa.y]);
        v.y = pack2(row[pa.z], row[pa.w]);
        v.z = pack2(row[pb.x], row[pb.y]);
        v.w = pack2(row[pb.z], row[pb.w]);
        stg16(W + (int64_t)pos[t] * n + e * 8, v);
      }
    }
  };
  if (single && c <= C) {
    // the whole cycle fits: slot t holds row p_t, p_t <- p_{(t+1) mod c}
    for (int k = 0; k < c; ++k) load_row(W + (int64_t)pos[k] * n, k);
    __syncthreads();
    for (int e = tid; e < n8; e += 256) {
      const int4 pa = *reinterpret_cast<const int4*>(kappa + e * 8);
      const int4 pb = *reinterpret_cast<const int4*>(kappa + e * 8 + 4);
      for (int t = 0; t < c; ++t) {
        const uint16_t* row = rows + (int64_t)((t + 1 == c) ? 0 : t + 1) * n;
        uint4 v;
        v.x = pack2(row[pa.x], row[pa.y]);
        v.y = pack2(row[pa.z], row[pa.w]);
        v.z = pack2(row[pb.x], row[pb.y]);
        v.w = pack2(row[pb.z], row[pb.w]);
        stg16(W + (int64_t)pos[t] * n + e * 8, v);
      }
    }
    return;
  }
  int keep_slot = -1, cap = C;
  if (single) {
    // keep the head's row in the last slot before p_0 is overwritten
    keep_slot = C - 1;
    cap = C - 1;
    load_row(W + (int64_t)h * n, keep_slot);
  }
  for (int t0 = 0; t0 < c; t0 += cap) {
    const int cnt = min(cap, c - t0);
    for (int k = 0; k < cnt; ++k) {
      const int t = t0 + k;
      if (t + 1 < c) load_row(W + (int64_t)pos[t + 1] * n, k);
      else if (!single) load_row(saved + (int64_t)sF * n, k);
    }
    __syncthreads();
    write_rows(t0, cnt, keep_slot);
    __syncthreads();
  }
}

bool walk_staged_ok(int64_t n, int L, const void* W, const void* saved, const int32_t* kappa) {
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  return (n & 7) == 0 && n <= 32768 && L <= WK_MAXL && al(W) && al(saved) && al(kappa);
}

void launch_cycle_plans_batch(const MergeBatch& b, int L, hipStream_t s) {
  int64_t mmax = 0;
  for (int k = 0; k < b.count; ++k) mmax = std::max(mmax, b.it[k].m);
  if (b.count <= 0 || mmax <= 0) return;
  const int kp = (int)((mmax + CP_THREADS - 1) / CP_THREADS);
#define POETX_CP(K) hipLaunchKernelGGL(cycle_plan_kernel<K>, dim3((unsigned)b.count), dim3(CP_THREADS), 0, s, b, L)
  if (kp <= 1) POETX_CP(1);
  else if (kp <= 2) POETX_CP(2);
  else if (kp <= 3) POETX_CP(3);
  else if (kp <= 4) POETX_CP(4);
  else if (kp <= 6) POETX_CP(6);
  else if (kp <= 8) POETX_CP(8);
  else if (kp <= 11) POETX_CP(11);
  else if (kp <= 16) POETX_CP(16);
  else if (kp <= 22) POETX_CP(22);
  else POETX_CP(32);
#undef POETX_CP
}

void launch_relayout_staged_batch(const MergeBatch& b, int L, hipStream_t s) {
  int64_t smax = 0, mmax = 0;
  for (int k = 0; k < b.count; ++k) {
    smax = std::max(smax, b.it[k].max_saved);
    mmax = std::max(mmax, b.it[k].m);
  }
  if (b.count <= 0 || mmax <= 0) return;
  if (smax > 0)
    hipLaunchKernelGGL(save_heads_kernel<uint16_t>, dim3((unsigned)smax, (unsigned)b.count), dim3(256), 0, s, b);
  hipLaunchKernelGGL(walk_rows_staged_bf16_kernel, dim3((unsigned)mmax, (unsigned)b.count), dim3(256), 0, s, b, L);
}

void launch_relayout_inplace(bool f32, void* W, void* saved, const int32_t* rho, const int32_t* kappa, int64_t m,
                             int64_t n, int L, int32_t* dist, int32_t* hlist, int32_t* slot, int32_t* slist,
                             int32_t* counts, int32_t* nxt, int64_t max_saved, hipStream_t s) {
  if (m <= 0 || n <= 0) return;
  MergeBatch b{};
  b.count = 1;
  MergeItem& it = b.it[0];
  it.W = W; it.saved = saved;
  it.snew = const_cast<int32_t*>(rho); it.tnew = const_cast<int32_t*>(kappa);
  it.dist = dist; it.hlist = hlist; it.slot = slot; it.slist = slist; it.counts = counts; it.nxt = nxt;
  it.m = m; it.n = n; it.max_saved = max_saved;
  launch_cycle_plans_batch(b, L, s);
  if (!f32 && walk_staged_ok(n, L, W, saved, kappa)) {
    launch_relayout_staged_batch(b, L, s);
    return;
  }
  if (f32) {
    if (max_saved > 0)
      hipLaunchKernelGGL(save_heads_kernel<float>, dim3((unsigned)max_saved, 1), dim3(256), 0, s, b);
    hipLaunchKernelGGL(walk_rows_kernel<float>, dim3((unsigned)m), dim3(256), 0, s, static_cast<float*>(W),
                       static_cast<const float*>(saved), rho, kappa, dist, hlist, slot, counts, (int)n, L);
  } else {
    if (max_saved > 0)
      hipLaunchKernelGGL(save_heads_kernel<uint16_t>, dim3((unsigned)max_saved, 1), dim3(256), 0, s, b);
    hipLaunchKernelGGL(walk_rows_kernel<uint16_t>, dim3((unsigned)m), dim3(256), 0, s, static_cast<uint16_t*>(W),
                       static_cast<const uint16_t*>(saved), rho, kappa, dist, hlist, slot, counts, (int)n, L);
  }
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

// two arrays set to v in one launch (the first n0 threads take p0)
__global__ void fill2_f32_kernel(float* p0, int64_t n0, float* p1, int64_t n1, float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n0) p0[i] = v;
  else if (i - n0 < n1) p1[i - n0] = v;
}
// thR, thP <- 0 of item blockIdx.y
__global__ void zero_generators_kernel(MergeBatch bt) {
  const MergeItem& it = bt.it[blockIdx.y];
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < it.nthR) it.thR[i] = 0.f;
  else if (i - it.nthR < it.nthP) it.thP[i - it.nthR] = 0.f;
}
void launch_zero_generators_batch(const MergeBatch& b, hipStream_t s) {
  int64_t tmax = 0;
  for (int k = 0; k < b.count; ++k) tmax = std::max(tmax, b.it[k].nthR + b.it[k].nthP);
  if (b.count <= 0 || tmax <= 0) return;
  hipLaunchKernelGGL(zero_generators_kernel, dim3((unsigned)((tmax + 255) / 256), (unsigned)b.count), dim3(256), 0, s,
                     b);
}
void launch_fill2_f32(float* p0, int64_t n0, float* p1, int64_t n1, float v, hipStream_t s) {
  if (n0 < 0) n0 = 0;
  if (n1 < 0) n1 = 0;
  if (n0 + n1 <= 0) return;
  hipLaunchKernelGGL(fill2_f32_kernel, dim3((unsigned)((n0 + n1 + 255) / 256)), dim3(256), 0, s, p0, n0, p1, n1, v);
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
