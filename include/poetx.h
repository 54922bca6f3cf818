/*
 * poetx.h -- C ABI of the POET-X layer hot path on AMD Instinct MI355X (gfx950).
 *
 * One linear layer uses the weight W = R * W0 * P.  W0 (m x n, out x in) is
 * frozen; R (m x m) and P (n x n) are permuted block-diagonal orthogonal
 * matrices whose b x b blocks are Cayley transforms of trainable
 * skew-symmetric generators.  The library computes the forward product
 * y = R (W0 (P x)), the backward onto the generators (and the input) with the
 * blocks and intermediate activations recomputed instead of stored, and the
 * periodic merge W0 <- R W0 P with generator reset and re-permutation.
 *
 * Sources (cited by page title and section):
 *  [P3] "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
 *       Transformation", gist.science summary of arXiv 2603.05500,
 *       "Technische samenvatting" > "Methodologie" items 1-5.
 *  [P1] "POET-X：基于正交变换缩放的内存高效LLM训练方法" (ai-stack.site),
 *       实践 2 (Cayley transform), 实践 4 (recompute), 实践 5 (fp32 accumulation).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller, row-major,
 *    unless a parameter says "host".  The library never allocates or frees
 *    device memory; scratch space is the caller's workspace `ws` of at least
 *    poetx_workspace_bytes(...) bytes, 256-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on `stream` and returns; none synchronizes the host.
 *  - Tokens are rows: X is N x n, Y and dY are N x m, so Y = X W^T.
 *  - Block structure: k_R = m / b blocks on the R side, k_P = n / b on the P
 *    side (integer division).  The m - k_R*b (resp. n - k_P*b) leftover
 *    coordinates form an identity tail with no generator.
 *  - Generators ("theta"): fp32, [k][b(b-1)/2], the strict upper triangle of
 *    each skew block S in row-major order: S[i][j] = theta[p], S[j][i] = -theta[p]
 *    for i < j, p = i*b - i*(i+1)/2 + (j-i-1).  Only this triangle is stored
 *    [P3 item 4].  Block l of R is Q_l = (I - S_l)^-1 (I + S_l) [P1 实践 2].
 *  - Permutations: int32 index maps, never matrices [P3 item 2].  sigma (length
 *    m) and tau (length n): block l of R acts on the true coordinates
 *    sigma[l*b .. l*b+b-1], the tail on sigma[k_R*b ..]; likewise tau for P.
 *  - Working weight layout: the two permutations next to W0 are folded into
 *    the stored weight [P3 item 2, second bullet]: the buffer W0p holds
 *    W0p[i][j] = W0[sigma[i]][tau[j]].  poetx_merge with zero generators is a
 *    pure relayout, which is how a caller packs a true-coordinate W0 (start
 *    from identity sigma, tau) and unpacks it again.
 *  - dtype (poetx_layer.dtype) applies to W0p, X, Y, dY and dX: POETX_F32 or
 *    POETX_BF16.  With bf16 every product runs on bf16 MFMA with fp32
 *    accumulation [P1 实践 5]; intermediate activations are stored in bf16.
 *    Generators, their gradients and the Cayley solve are fp32.
 *  - Results are deterministic: identical inputs give bit-identical outputs.
 *  - Errors: a negative poetx_status; poetx_last_error() then describes it.
 *    Arguments are validated on the host before anything is enqueued, so an
 *    error leaves every output untouched.  A failed kernel launch returns
 *    POETX_EHIP.  No exception crosses the ABI.
 *  - Sizes: 1 <= m, n <= 32768; 0 <= N < 2^31; b in {32, 64, 128, 256, 512}.
 *    N == 0 is a valid empty call (nothing is enqueued except the gradient
 *    reset of poetx_backward when POETX_ACCUMULATE_GRAD is not set).
 */
#ifndef POETX_H
#define POETX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  POETX_OK = 0,
  POETX_EINVAL = -1,     /* null pointer, bad enum, bad block size          */
  POETX_ESHAPE = -2,     /* m, n, N or a count out of range                 */
  POETX_EDTYPE = -3,     /* unsupported dtype                                */
  POETX_EWORKSPACE = -4, /* workspace too small or misaligned                */
  POETX_EHIP = -5        /* a HIP runtime call or kernel launch failed       */
} poetx_status;

typedef enum { POETX_F32 = 0, POETX_BF16 = 1 } poetx_dtype;

/* poetx_layer.flags */
#define POETX_ACCUMULATE_GRAD 1u /* backward adds into dthR/dthP instead of overwriting */
#define POETX_W0_INT8 2u         /* W0p in the INT8 weight format (bf16 layers), below */
/* bf16, b in {64, 128, 256}: the forward's R-side block product as a pass
 * of its own instead of in the epilogue of the GEMM before it.  Results are
 * bit-identical either way; for verification. */
#define POETX_SEPARATE_BLOCK_PRODUCTS 4u
/* bf16 layers: W0p also holds its transpose (format below) */
#define POETX_W0_TRANSPOSED 8u
/* bf16 layers: the X argument of the forward and backward calls holds
 * x' = Pi_tau x, the input already gathered into the working layout
 * (poetx_permute_input below), instead of x */
#define POETX_X_PERMUTED 16u

/* op codes for poetx_workspace_bytes */
#define POETX_OP_FORWARD 0
#define POETX_OP_BACKWARD 1
#define POETX_OP_MERGE 2
#define POETX_OP_FORWARD_BLOCKS 3  /* poetx_forward_blocks  */
#define POETX_OP_BACKWARD_BLOCKS 4 /* poetx_backward_blocks */
#define POETX_OP_MERGE_BLOCKS 5    /* poetx_merge_blocks    */
#define POETX_OP_BACKWARD_DQ 6     /* poetx_backward_blocks_dq */

typedef struct {
  int64_t m;      /* rows of W0 = output features                         */
  int64_t n;      /* columns of W0 = input features                       */
  int32_t b;      /* block size of R and P                                */
  int32_t dtype;  /* poetx_dtype of W0p, X, Y, dY, dX                     */
  uint32_t flags; /* POETX_ACCUMULATE_GRAD, POETX_W0_INT8,
                     POETX_SEPARATE_BLOCK_PRODUCTS, POETX_W0_TRANSPOSED,
                     POETX_X_PERMUTED                                     */
  uint32_t reserved; /* must be 0                                         */
} poetx_layer;

/*
 * Bytes of workspace that op (POETX_OP_*) needs for this layer and N tokens.
 * Returns 0 and sets the last error if the layer is invalid.  Host only.
 */
size_t poetx_workspace_bytes(const poetx_layer* layer, int64_t N, int op);

/*
 * POET-XQ weight storage [P3 item 5: base weights stored quantized, e.g.
 * INT8, and dequantized on the fly].  With POETX_W0_INT8 in layer->flags
 * (bf16 layers only) every W0p argument of this library points to the INT8
 * weight format instead of bf16 [m][n]:
 *   bytes [0, m*n)            int8 codes q[i][j], row-major, working layout
 *   bytes [off, off + 4m)     fp32 scales s[i], off = m*n rounded up to 256
 * The weight a pass uses is w[i][j] = bf16(s[i] * q[i][j]) (fp32 product,
 * both roundings to nearest even), so its results equal those of the bf16
 * layer whose W0p holds those values, bit for bit.  When n % 16 == 0 and
 * m % 8 == 0 the passes' GEMMs can read the codes and scales directly and
 * form w as they stage their tiles, with no bf16 copy of the weight (W0p must
 * then be 16-byte aligned, else POETX_EINVAL).  They do so by default unless
 * n or m is a multiple of 64 of at least 2048 (there a dequantized copy in
 * the workspace feeding the wide bf16 GEMM is faster); those layers, and
 * other shapes, dequantize w into the pass's workspace first (the workspace
 * sizes include that buffer), transposed for the forward product and its
 * recompute (read as NN GEMMs, as with POETX_W0_TRANSPOSED below) and
 * [m][n] for the backward product.  poetx_forward_blocks_noalloc always reads the
 * codes directly.  A
 * merge merges the dequantized weight and stores it again as codes:
 *   s[i] = max_j |w[i][j]| / 127, q[i][j] = clamp(rne(w[i][j] / s[i]), -127, 127)
 * in fp32 (s[i] = 0, q[i] = 0 for a row of zeros).
 *
 * poetx_w0_bytes: bytes of the W0p buffer of this layer (any format);
 *   0 and the last error set if the layer is invalid.  Host only.
 * poetx_quantize_w0: W0q (INT8 format) from a bf16 [m][n] weight W0bf16 in
 *   the same layout, by the rule above.  Device pointers; no workspace.
 * poetx_dequantize_w0: the bf16 [m][n] weight a pass would use.
 * Both return POETX_EINVAL when layer->flags lacks POETX_W0_INT8.
 */
size_t poetx_w0_bytes(const poetx_layer* layer);
int poetx_quantize_w0(const poetx_layer* layer, const void* W0bf16, void* W0q, void* stream);
int poetx_dequantize_w0(const poetx_layer* layer, const void* W0q, void* W0bf16, void* stream);

/*
 * Weight with its transpose (POETX_W0_TRANSPOSED, bf16 layers, not with
 * POETX_W0_INT8): every W0p argument points to
 *   bytes [0, 2mn)            bf16 W0p [m][n], working layout, as without the flag
 *   bytes [off, off + 2mn)    bf16 W0p^T [n][m], off = 2mn rounded up to 256
 * The forward product z2' = z1' W0p^T (and its recompute in the backward
 * pass) then reads W0p^T, whose rows run along the output features: the
 * GEMM's weight operand in the layout of the backward product, which the
 * GEMM kernels stage faster.  Results are bit-identical to the layer
 * without the flag [P3 "POET-X: Memory-efficient LLM Training by Scaling
 * Orthogonal Transformation", Methodologie item 1: the weight-sized product
 * the input-centric form keeps].  Every merge writes both halves.
 *
 * poetx_transpose_w0: writes the second half from the first (after the
 *   caller has written W0p itself).  POETX_EINVAL without the flag.
 */
int poetx_transpose_w0(const poetx_layer* layer, void* W0p, void* stream);

/*
 * The input in the working layout [P3 "POET-X: Memory-efficient LLM Training
 * by Scaling Orthogonal Transformation", Methodologie items 2-3: the
 * permutation of P regroups the input coordinates into the blocks that act
 * on them]:
 *   Xp[t][j] = X[t][tau[j]]   (t < N, j < n, the identity tail included)
 * For layers with POETX_X_PERMUTED (bf16 only), every forward and backward
 * call takes Xp where it takes X, and skips its own gather of X: the pass
 * then starts with the P-side block product.  A caller can so gather the
 * input while the blocks are being built (the gather does not need them),
 * and keep Xp instead of X for the backward pass (same bytes; its recompute
 * then gathers nothing).  Results are bit-identical to the layer without the
 * flag on X.
 *   tau  [n] int32 (a permutation; not checked); X, Xp [N][n] bf16, device,
 *   not overlapping.  The layer's flags need not include POETX_X_PERMUTED.
 * Errors: POETX_EINVAL (NULL argument), POETX_EDTYPE (fp32 layer),
 * POETX_ESHAPE (N out of range), POETX_EHIP (launch failed).
 */
int poetx_permute_input(const poetx_layer* layer, const int32_t* tau, const void* X, int64_t N, void* Xp,
                        void* stream);

/*
 * One batch of Cayley blocks for poetx_build_block_sets: the generators of
 * nblocks blocks and where their Q goes (layouts as in poetx_build_blocks).
 */
typedef struct {
  const float* theta; /* [nblocks][b(b-1)/2] fp32, device                  */
  int64_t nblocks;    /* >= 0                                              */
  float* Q32;         /* [nblocks][b][b] fp32 Q, device, nullable          */
  void* Qbf16;        /* [nblocks][b][b] bf16 Q, device, nullable          */
  void* QTbf16;       /* [nblocks][b][b] bf16 Q^T, device, nullable        */
} poetx_block_set;

/*
 * Prebuilt Cayley blocks of one layer for poetx_forward_blocks and
 * poetx_backward_blocks, each [k][b][b] row-major on the device (R side:
 * k = k_R, P side: k = k_P).  Which are read:
 *   fp32 layer, forward and backward: Q32R, Q32P;
 *   bf16 layer, forward:  QR, QP (bf16 Q);
 *   bf16 layer, backward: Q32R, Q32P (fp32 Q, for the chain rule), QP,
 *                         QTR, QTP (bf16 Q^T);
 *   merge: Q32R, Q32P (fp32 layer) or QR, QTP (bf16 layer).
 * The others may be NULL.
 */
typedef struct {
  const float* Q32R;
  const float* Q32P;
  const void* QR;
  const void* QP;
  const void* QTR;
  const void* QTP;
} poetx_blocks;

/*
 * Bytes of workspace poetx_build_blocks needs for nblocks blocks of size b;
 * for poetx_build_block_sets, pass the total nblocks of its sets (at b = 512
 * the blocks of all sets go through one pass of the 2x2 Schur-complement
 * solve together).  Zero for b <= 256.
 */
size_t poetx_build_workspace_bytes(int64_t nblocks, int32_t b);

/*
 * a1-a2: batched Cayley builder [P1 实践 2; P3 item 4].
 * For each block l < nblocks: S_l from theta[l] (layout above), then
 * Q_l = (I - S_l)^-1 (I + S_l), computed as 2 (I - S_l)^-1 - I with an exact
 * fp32 Gauss-Jordan solve (no pivoting: I - S has symmetric part I).
 *   theta  [nblocks][b(b-1)/2] fp32, device
 *   Q32    [nblocks][b][b] fp32 row-major, device, nullable
 *   Qbf16  [nblocks][b][b] bf16 Q, row-major, device, nullable
 *   QTbf16 [nblocks][b][b] bf16 Q^T, row-major, device, nullable
 *   ws     workspace of poetx_build_workspace_bytes(nblocks, b) bytes
 * nblocks == 0 is a no-op.
 */
int poetx_build_blocks(const float* theta, int64_t nblocks, int32_t b, float* Q32,
                       void* Qbf16, void* QTbf16, void* ws, size_t ws_bytes, void* stream);

/*
 * a1-a2 over several independent batches at once (e.g. the R and P sides of
 * every layer of a model): the same blocks poetx_build_blocks gives for each
 * set, with the sets of one call sharing kernel launches so that the grid
 * covers the blocks of all of them.  The pages fuse the block builds to cut
 * launches and data movement [P3 item 4; P1 实践 2].
 *   sets   host array of count poetx_block_set (count in [0, 4096]); every
 *          set has the same block size b
 *   ws     poetx_build_workspace_bytes(total nblocks over the sets, b) bytes
 * Output buffers must not overlap each other or any theta.
 */
int poetx_build_block_sets(const poetx_block_set* sets, int32_t count, int32_t b, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * poetx_build_block_sets with the truncated Neumann (CNP) form of the Cayley
 * map where it is accurate enough [P3 item 4]: (I - S)^-1 = I + S + S^2 + ...
 * for ||S|| < 1, so Q = I + 2 (S + S^2 + ... + S^terms) with `terms` powers
 * kept.  A block takes this form only when the dropped tail is provably
 * small: f = ||S||_F < 1 and 2 f^(terms+1) / (1 - f) <= 2^-22 (a bound on
 * its spectral norm); every other block gets the exact solve, bit for bit as
 * poetx_build_block_sets builds it.  The powers are fp32-accurate products.
 * With the generators at zero (right after a merge) every block takes the
 * series.
 *   terms  1..16
 *   b      32, 64, 128 or 256; at most 65535 blocks per set and per call
 *   ws     poetx_build_cnp_workspace_bytes(total blocks of the call, b)
 */
size_t poetx_build_cnp_workspace_bytes(int64_t total_blocks, int32_t b);
int poetx_build_block_sets_cnp(const poetx_block_set* sets, int32_t count, int32_t b, int32_t terms,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * a3-a5: forward Y = X W^T, W = R W0 P, computed input-centrically as
 * P, then W0, then R on each token [P3 item 1], with P and R applied as
 * gathers/scatters and batched block products [P3 items 2-3].
 *   W0p   [m][n] dtype, working layout
 *   thR   [k_R][b(b-1)/2] fp32;  thP [k_P][b(b-1)/2] fp32
 *   sigma [m] int32, tau [n] int32 (must be permutations; not checked)
 *   X     [N][n] dtype;  Y [N][m] dtype (written)
 */
int poetx_forward(const poetx_layer* layer, const void* W0p, const float* thR,
                  const float* thP, const int32_t* sigma, const int32_t* tau,
                  const void* X, int64_t N, void* Y, void* ws, size_t ws_bytes,
                  void* stream);

/*
 * poetx_forward with the Cayley blocks built beforehand (poetx_build_blocks
 * or poetx_build_block_sets from the layer's current generators): a3-a5
 * only.  Same arguments and results as poetx_forward, with the generators
 * replaced by the blocks (poetx_blocks above).  Workspace:
 * poetx_workspace_bytes(layer, N, POETX_OP_FORWARD_BLOCKS).
 */
int poetx_forward_blocks(const poetx_layer* layer, const void* W0p, const poetx_blocks* blocks,
                         const int32_t* sigma, const int32_t* tau, const void* X, int64_t N,
                         void* Y, void* ws, size_t ws_bytes, void* stream);

/*
 * poetx_forward_blocks for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes no workspace and allocates nothing: its intermediates
 * live in a static device array of POETX_NOALLOC_SCRATCH_BYTES (64 MiB) that
 * every GPU the library runs on holds until the process ends (its device
 * address is looked up once per device, on the first call with that device
 * current; the stream must belong to the current device).  Tokens go
 * through in chunks of the largest multiple of 128 whose forward
 * intermediates fit the array (N * (n + m + max(m, n)) * 2 bytes for bf16,
 * N * (n + m) * 4 for fp32); the results are bit-identical to
 * poetx_forward_blocks.  Calls on one GPU share the array, which keeps the
 * last call's contents: calls that overlap on one GPU (concurrent streams,
 * threads) race and must be serialized by the caller.  Errors: those of
 * poetx_forward_blocks; POETX_EINVAL for POETX_W0_INT8 layers whose GEMMs
 * cannot read the codes directly (n % 16 or m % 8 nonzero: their dequantized
 * weight does not fit beside the chunk); POETX_ESHAPE if 128
 * tokens of the layer exceed the array; POETX_EHIP if the array's address
 * cannot be obtained.
 */
#define POETX_NOALLOC_SCRATCH_BYTES (64ull << 20)
int poetx_forward_blocks_noalloc(const poetx_layer* layer, const void* W0p,
                                 const poetx_blocks* blocks, const int32_t* sigma,
                                 const int32_t* tau, const void* X, int64_t N, void* Y,
                                 void* stream);

/*
 * a0, a6-a9: backward of L = <dY, Y> with W0 frozen.  The Cayley blocks and
 * the intermediate activations are recomputed from X rather than stored
 * (POET-Xmem gradient checkpointing, [P3 item 5]); the gradient reaches the
 * stored generators through the Cayley map [P1 实践 2 step 3]:
 * dL/dS = 1/2 (I + Q^T) G (I + Q^T) with G = dL/dQ, and
 * dL/dtheta_p = G_S[i][j] - G_S[j][i].
 *   dY   [N][m] dtype
 *   dX   [N][n] dtype, written; nullable (then not computed)
 *   dthR [k_R][b(b-1)/2] fp32, dthP [k_P][b(b-1)/2] fp32: overwritten, or
 *        accumulated into when layer->flags has POETX_ACCUMULATE_GRAD
 */
int poetx_backward(const poetx_layer* layer, const void* W0p, const float* thR,
                   const float* thP, const int32_t* sigma, const int32_t* tau,
                   const void* X, const void* dY, int64_t N, void* dX, float* dthR,
                   float* dthP, void* ws, size_t ws_bytes, void* stream);

/*
 * poetx_backward with the Cayley blocks built beforehand (the caller
 * rebuilds them from the generators for the backward pass, which keeps the
 * blocks recomputed rather than held from the forward pass [P3 item 5]):
 * a0, a6-a9 with the same arguments and results as poetx_backward, the
 * generators replaced by the blocks.  Workspace:
 * poetx_workspace_bytes(layer, N, POETX_OP_BACKWARD_BLOCKS).
 */
int poetx_backward_blocks(const poetx_layer* layer, const void* W0p, const poetx_blocks* blocks,
                          const int32_t* sigma, const int32_t* tau, const void* X, const void* dY,
                          int64_t N, void* dX, float* dthR, float* dthP, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * a0, a6-a8 without the chain rule: poetx_backward_blocks up to the gradient
 * with respect to the orthogonal blocks, G_l = dL/dQ_l, which it writes
 * instead of the generator gradients.  The chain rule through the Cayley
 * map [P1 实践 2 step 3] then runs for many layers at once in
 * poetx_chain_rule_sets, so its small per-block products fill the GPU.
 *   GR [k_R][b][b], GP [k_P][b][b] fp32, device, overwritten
 * bf16 layers only; layer->flags must not carry POETX_ACCUMULATE_GRAD (it
 * belongs to poetx_chain_rule_sets).  N == 0 writes zeros.  Workspace:
 * poetx_workspace_bytes(layer, N, POETX_OP_BACKWARD_DQ).
 */
int poetx_backward_blocks_dq(const poetx_layer* layer, const void* W0p, const poetx_blocks* blocks,
                             const int32_t* sigma, const int32_t* tau, const void* X, const void* dY,
                             int64_t N, void* dX, float* GR, float* GP, void* ws, size_t ws_bytes,
                             void* stream);

/*
 * The variant without activation recompute: POET-Xmem recomputes the
 * intermediate activations in the backward pass to save memory [P3 item 5];
 * keeping the weight product's output z2' = z1' W0p^T from the forward pass
 * instead saves the backward pass the P-side block product and the forward
 * GEMM, for N * m * 2 bytes per layer.
 *
 * poetx_forward_blocks that also writes z2' to Z2:
 *   Z2  [N][m] bf16, the working (sigma-permuted) layout, device, written;
 *       must not overlap any other argument
 * bf16 layers only (POETX_EDTYPE otherwise); N == 0 writes nothing.
 * Workspace: poetx_workspace_bytes(layer, N, POETX_OP_FORWARD_BLOCKS).
 */
int poetx_forward_blocks_z2(const poetx_layer* layer, const void* W0p, const poetx_blocks* blocks,
                            const int32_t* sigma, const int32_t* tau, const void* X, int64_t N,
                            void* Y, void* Z2, void* ws, size_t ws_bytes, void* stream);

/*
 * poetx_backward_blocks_dq with z2' read from Z2 instead of recomputed:
 *   Z2  [N][m] bf16, as poetx_forward_blocks_z2 wrote it for the same X,
 *       W0p and generators (the blocks are rebuilt from the same generators,
 *       so the results are identical to poetx_backward_blocks_dq's)
 * x' = Pi_tau x is still gathered again for dL/dQ_P.  bf16 layers only.
 * Workspace: poetx_workspace_bytes(layer, N, POETX_OP_BACKWARD_DQ).
 */
int poetx_backward_blocks_dq_z2(const poetx_layer* layer, const void* W0p, const poetx_blocks* blocks,
                                const int32_t* sigma, const int32_t* tau, const void* X, const void* dY,
                                const void* Z2, int64_t N, void* dX, float* GR, float* GP, void* ws,
                                size_t ws_bytes, void* stream);

/* One batch of blocks for poetx_chain_rule_sets. */
typedef struct {
  const float* Q32; /* [nblocks][b][b] fp32 Cayley blocks Q, device           */
  const float* G;   /* [nblocks][b][b] fp32 dL/dQ, device                      */
  int64_t nblocks;  /* >= 0                                                    */
  float* dtheta;    /* [nblocks][b(b-1)/2] fp32 generator gradient, device     */
} poetx_chain_set;

/*
 * a9 over many batches at once: for every block,
 * G_S = 1/2 (I + Q^T) G (I + Q^T) and dtheta_p = G_S[i][j] - G_S[j][i] on the
 * stored upper triangle [P1 实践 2 step 3; P3 item 4].  The products are
 * fp32-accurate (bf16 MFMA on a hi/lo split of each fp32 operand, fp32
 * accumulation), as in poetx_backward for bf16 layers, and bit-identical to
 * it block for block.
 *   sets   host array of count poetx_chain_set (count in [0, 65536]), one
 *          block size b for all
 *   flags  POETX_ACCUMULATE_GRAD: add into dtheta instead of overwriting
 *   ws     poetx_chain_workspace_bytes(total blocks over the sets, b) bytes
 * G and Q are only read.
 */
int poetx_chain_rule_sets(const poetx_chain_set* sets, int32_t count, int32_t b, uint32_t flags,
                          void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of poetx_chain_rule_sets for total_blocks blocks of size b. */
size_t poetx_chain_workspace_bytes(int64_t total_blocks, int32_t b);

/*
 * a10-a11: merge W0 <- R W0 P [P3 item 1], then theta_R, theta_P <- 0 and
 * new permutations sigma' = perm(seed, merge_index, side 0),
 * tau' = perm(seed, merge_index, side 1) (see poetx_make_permutation), with
 * W0p rewritten in place into the new working layout:
 * W0p'[i][j] = (R W0 P)[sigma'[i]][tau'[j]].
 *   W0p        [m][n] dtype, in/out
 *   thR, thP   fp32, zeroed on return
 *   sigma, tau int32, in: current permutations; out: the new ones
 * The permutations are drawn on the device; nothing is copied to or from the
 * host.  With zero generators the result is an exact relayout.
 */
int poetx_merge(const poetx_layer* layer, void* W0p, float* thR, float* thP, int32_t* sigma,
                int32_t* tau, uint64_t perm_seed, uint64_t merge_index, void* ws,
                size_t ws_bytes, void* stream);

/*
 * poetx_merge with the Cayley blocks built beforehand from the layer's
 * current generators (poetx_build_block_sets lets a merge of many layers
 * share builder launches).  Same arguments and results as poetx_merge, the
 * blocks (poetx_blocks above) added.  Workspace:
 * poetx_workspace_bytes(layer, 0, POETX_OP_MERGE_BLOCKS).
 */
int poetx_merge_blocks(const poetx_layer* layer, void* W0p, const poetx_blocks* blocks, float* thR,
                       float* thP, int32_t* sigma, int32_t* tau, uint64_t perm_seed,
                       uint64_t merge_index, void* ws, size_t ws_bytes, void* stream);

/* One layer's arguments of poetx_merge_blocks, for poetx_merge_blocks_sets. */
typedef struct {
  const poetx_layer* layer;
  void* W0p;
  const poetx_blocks* blocks;
  float* thR;
  float* thP;
  int32_t* sigma;
  int32_t* tau;
  uint64_t perm_seed;
  uint64_t merge_index;
} poetx_merge_set;

/*
 * a10-a11 for several layers at once: the global merge of a model [P3
 * item 1: every layer merged at the same step].  The results are those of
 * poetx_merge_blocks on each set in turn, bit for bit; the permutation
 * draws, the relayout plans, the relayouts and the generator resets of up to
 * 16 sets share one launch per stage (bf16 layers whose rows are a multiple
 * of 8 columns and 16-byte aligned; other layers are merged one by one
 * inside the call).  The sets' buffers must be disjoint.  count == 0 is a
 * no-op.
 *   ws  workspace of poetx_merge_sets_workspace_bytes(sets, count) bytes
 * Errors are detected on the host, before any launch, for every set.
 */
int poetx_merge_blocks_sets(const poetx_merge_set* sets, int32_t count, void* ws, size_t ws_bytes,
                            void* stream);

/* Workspace bytes of poetx_merge_blocks_sets (0 with the error set for an
 * invalid layer). */
size_t poetx_merge_sets_workspace_bytes(const poetx_merge_set* sets, int32_t count);

/*
 * a11 on the host: the permutation poetx_merge draws for (seed, merge_index,
 * side), written to host_out[0..n-1].  The pages only say the permutations are
 * index maps [P3 item 2]; the generator adopted for "uniform random from a
 * seed" is: mix64 = SplitMix64's output function (Steele, Lea & Flood 2014),
 * gamma = 0x9E3779B97F4A7C15,
 * base = mix64(seed + gamma*(2*merge_index + side + 1)),
 * key_i = mix64(base + gamma*(i+1)), and the permutation lists 0..n-1 in
 * ascending (key_i, i) order.  side: 0 = sigma (R), 1 = tau (P).
 */
int poetx_make_permutation(uint64_t seed, uint64_t merge_index, int32_t side, int64_t n,
                           int32_t* host_out);

/*
 * a12: one Adam step (Kingma & Ba 2015, with bias correction, no weight
 * decay) on count fp32 generators, in place:
 *   m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2;
 *   theta <- theta - lr * (m / (1-b1^step)) / (sqrt(v / (1-b2^step)) + eps).
 * step >= 1.  Not on the pages (they leave the generator optimizer open).
 */
int poetx_adam_step(float* theta, const float* grad, float* m, float* v, int64_t count,
                    int64_t step, float lr, float beta1, float beta2, float eps,
                    void* stream);

/* Message of the last error on this thread ("" if none). */
const char* poetx_last_error(void);

/*
 * Diagnostics (not part of the method): per-kernel timing for measurement.
 * poetx_timing_enable(1) clears the record and starts recording a HIP event
 * pair on the caller's stream around every kernel the library launches,
 * together with the launch's algorithmic flops and HBM bytes; (0) stops.
 * poetx_timing_summary synchronizes the recorded events and writes one line
 * per kernel class, "name launches total_ms flops bytes" and a newline, into buf (host,
 * len bytes, NUL-terminated); returns the number of classes or a negative
 * status.  Recording adds host work per launch; leave it off when timing
 * whole steps.  Not thread-safe.
 */
int poetx_timing_enable(int on);
int poetx_timing_summary(char* buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* POETX_H */
