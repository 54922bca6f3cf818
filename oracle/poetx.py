"""POET-X layer hot path in float64, true coordinates, numpy only.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Notation (the pages give none; this is the plainest reading of them):

* ``W0`` is the frozen base weight, shape (m, n) = (out, in), as in a linear
  layer; tokens are rows, so ``Y = X @ W.T`` with ``W = R @ W0 @ P``.
  [P3 "Methodologie" item 1: W is changed by an orthogonal equivalence
  transform, W <- R W P, applied input-centrically as a chain of linear maps on
  the input; P2 section 1.2: such transforms leave the spectrum unchanged.]
* ``R`` (m x m) and ``P`` (n x n) are permuted block-diagonal orthogonal
  matrices [P3 "Methodologie" items 2-3].  With block size ``b``, ``R`` has
  ``k_R = m // b`` blocks; the ``m - k_R*b`` leftover coordinates form an
  identity tail.  The permutation ``sigma`` (for R) groups coordinates:
  block ``l`` acts on the true coordinates ``sigma[l*b:(l+1)*b]`` and the tail
  on ``sigma[k_R*b:]``.  Equivalently ``R = Pi^T diag(Q_0..Q_{k-1}, I) Pi``
  with the gather ``(Pi v)_i = v[sigma[i]]``.  ``P`` is the same with ``tau``.
* Each block ``Q_l`` is the Cayley transform of a skew-symmetric ``S_l`` whose
  strict upper triangle is the trainable generator ``theta_l`` (row-major,
  ``b(b-1)/2`` numbers) [P3 "Methodologie" item 4; P1 实践 2].

``contract=True`` inserts round-to-nearest-even to bfloat16 at the points where
a bf16 pipeline stores a value (low-precision storage and products with fp32
accumulation [P1 实践 5]): the Q operands of every bf16 product, z1, z2, Y,
gZ2, gZ1, dX, and the merged weight (and its half-merged intermediate).
Everything else is float64.  ``contract=False`` is the exact definition.
"""

import numpy as np

GOLDEN_GAMMA = 0x9E3779B97F4A7C15
_MASK64 = (1 << 64) - 1


# --------------------------------------------------------------------------
# Rounding used by the bf16 precision contract
# --------------------------------------------------------------------------
def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits and float32's exponent range, so a
    number in [2**(e-1), 2**e) is rounded to a multiple of 2**(e-8); below the
    smallest normal 2**-126 the spacing stays 2**-133.  Returned as float64.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    q = np.ldexp(1.0, e - 8)
    return np.rint(x / q) * q


def _identity(x):
    return x


# --------------------------------------------------------------------------
# a1, a2: generator -> skew matrix -> Cayley block
# --------------------------------------------------------------------------
def triu_pairs(b):
    """(rows, cols) of the strict upper triangle of a b x b matrix, row-major.

    Generator entry p sits at (i, j) with i < j and
    p = i*b - i*(i+1)/2 + (j - i - 1).  Only this triangle is stored, which
    halves the parameter count [P3 "Methodologie" item 4, first bullet].
    """
    return np.triu_indices(b, k=1)


def unpack_skew(theta_l, b):
    """Skew-symmetric S with S[i, j] = theta[p(i, j)] and S[j, i] = -theta[p]."""
    theta_l = np.asarray(theta_l, dtype=np.float64)
    if theta_l.shape != (b * (b - 1) // 2,):
        raise ValueError("generator has %s entries, expected b(b-1)/2 = %d"
                         % (theta_l.shape, b * (b - 1) // 2))
    S = np.zeros((b, b), dtype=np.float64)
    r, c = triu_pairs(b)
    S[r, c] = theta_l
    S[c, r] = -theta_l
    return S


def cayley(S):
    """Q = (I - S)^-1 (I + S) by an LU solve [P1 实践 2, step 2].

    For skew S this Q is orthogonal with det +1 [P1 实践 4, step 3].  The
    pages' GPU route replaces the inverse by a truncated Neumann series
    [P3 "Methodologie" item 4]: ``cayley_neumann`` below.
    """
    b = S.shape[0]
    eye = np.eye(b)
    return np.linalg.solve(eye - S, eye + S)


def cayley_neumann(S, k):
    """The truncated Neumann form of the Cayley map [P3 "Methodologie" item 4,
    CNP]: (I - S)^-1 is the series I + S + S^2 + ... for ||S|| < 1, so
    Q = (I - S)^-1 (I + S) = I + 2 (S + S^2 + ...); keep the first k powers.
    Plain powers, float64."""
    S = np.asarray(S, dtype=np.float64)
    b = S.shape[0]
    P = np.eye(b)
    acc = np.zeros((b, b))
    for _ in range(k):
        P = P @ S
        acc = acc + P
    return np.eye(b) + 2.0 * acc


def cnp_error_bound(S, k):
    """Bound on ||cayley(S) - cayley_neumann(S, k)||_2: the dropped tail
    2 (S^{k+1} + S^{k+2} + ...) has norm at most 2 f^{k+1} / (1 - f) with
    f = ||S||_F >= ||S||_2; infinite when f >= 1 (no convergence bound)."""
    f = float(np.linalg.norm(np.asarray(S, dtype=np.float64)))
    return 2.0 * f ** (k + 1) / (1.0 - f) if f < 1.0 else np.inf


def block_count(dim, b):
    """Number of full b x b blocks along a side of size dim; the rest is an
    identity tail."""
    return dim // b


def _qs(theta, b):
    theta = np.asarray(theta, dtype=np.float64)
    return [cayley(unpack_skew(theta[l], b)) for l in range(theta.shape[0])]


def _groups(perm, b):
    perm = np.asarray(perm, dtype=np.int64)
    k = len(perm) // b
    return [perm[l * b:(l + 1) * b] for l in range(k)]


def dense_orthogonal(theta, perm, b):
    """The full permuted block-diagonal matrix Pi^T diag(Q_0..Q_{k-1}, I) Pi.

    Built from an explicit permutation matrix; only for brute-force checks on
    small sizes.
    """
    perm = np.asarray(perm, dtype=np.int64)
    dim = len(perm)
    Pi = np.zeros((dim, dim))
    Pi[np.arange(dim), perm] = 1.0
    D = np.eye(dim)
    for l, Q in enumerate(_qs(theta, b)):
        D[l * b:(l + 1) * b, l * b:(l + 1) * b] = Q
    return Pi.T @ D @ Pi


# --------------------------------------------------------------------------
# a3-a5: forward  y = R (W0 (P x))
# --------------------------------------------------------------------------
def forward(W0, thR, thP, sigma, tau, X, b, contract=False, intermediates=False):
    """Input-centric forward [P3 "Methodologie" item 1]: P, then W0, then R.

    Z1 = P applied to each token; Z2 = Z1 W0^T; Y = R applied to Z2.
    Block products act on the coordinate groups given by the permutations,
    never on an explicit permutation matrix [P3 "Methodologie" items 2-3].
    """
    rnd = round_bf16 if contract else _identity
    W0 = np.asarray(W0, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    QR, QP = _qs(thR, b), _qs(thP, b)
    QRm = [rnd(q) for q in QR]
    QPm = [rnd(q) for q in QP]
    Z1 = X.copy()
    for l, J in enumerate(_groups(tau, b)):
        Z1[:, J] = rnd(X[:, J] @ QPm[l].T)
    Z2 = rnd(Z1 @ W0.T)
    Y = Z2.copy()
    for l, I in enumerate(_groups(sigma, b)):
        Y[:, I] = rnd(Z2[:, I] @ QRm[l].T)
    if intermediates:
        return Y, dict(Z1=Z1, Z2=Z2, QR=QR, QP=QP, QRm=QRm, QPm=QPm)
    return Y


# --------------------------------------------------------------------------
# a9: chain rule from dL/dQ to dL/dtheta
# --------------------------------------------------------------------------
def chain_rule(G, Q):
    """Gradient on the stored generator from G = dL/dQ.

    With M = (I - S)^-1, dQ = 2 M dS M, so dL/dS = 2 M^T G M^T
    = 1/2 (I + Q^T) G (I + Q^T) since M = (I + Q)/2.  theta_p enters S at
    (i, j) with + and at (j, i) with -, hence
    dL/dtheta_p = G_S[i, j] - G_S[j, i]  (automatic differentiation carried to
    the generator [P1 实践 2, step 3]; upper-triangle storage [P3 item 4]).
    """
    b = Q.shape[0]
    A = np.eye(b) + Q.T
    GS = 0.5 * (A @ G @ A)
    r, c = triu_pairs(b)
    return GS[r, c] - GS[c, r]


# --------------------------------------------------------------------------
# a0, a6-a8: backward onto the generators (W0 frozen), with recompute
# --------------------------------------------------------------------------
def backward(W0, thR, thP, sigma, tau, X, gY, b, contract=False, intermediates=False):
    """Gradients of L = <gY, Y> w.r.t. X, theta_R and theta_P; W0 is frozen.

    Z1 and Z2 are recomputed from X rather than stored (gradient
    checkpointing, POET-Xmem [P3 "Methodologie" item 5]).
    Returns (dX, dthR [k_R, b(b-1)/2], dthP [k_P, b(b-1)/2]).
    """
    rnd = round_bf16 if contract else _identity
    W0 = np.asarray(W0, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    gY = np.asarray(gY, dtype=np.float64)
    _, it = forward(W0, thR, thP, sigma, tau, X, b, contract=contract, intermediates=True)
    Z2 = it["Z2"]
    gZ2 = gY.copy()
    GR = []
    for l, I in enumerate(_groups(sigma, b)):
        gZ2[:, I] = rnd(gY[:, I] @ it["QRm"][l])
        GR.append(gY[:, I].T @ Z2[:, I])
    gZ1 = rnd(gZ2 @ W0)
    dX = gZ1.copy()
    GP = []
    for l, J in enumerate(_groups(tau, b)):
        GP.append(gZ1[:, J].T @ X[:, J])
        dX[:, J] = rnd(gZ1[:, J] @ it["QPm"][l])
    nt = b * (b - 1) // 2
    dthR = np.array([chain_rule(G, Q) for G, Q in zip(GR, it["QR"])]).reshape(-1, nt)
    dthP = np.array([chain_rule(G, Q) for G, Q in zip(GP, it["QP"])]).reshape(-1, nt)
    if intermediates:
        return dX, dthR, dthP, dict(it, gZ2=gZ2, gZ1=gZ1, GR=GR, GP=GP)
    return dX, dthR, dthP


# --------------------------------------------------------------------------
# a10: merge  W0 <- R W0 P
# --------------------------------------------------------------------------
def merge(W0, thR, thP, sigma, tau, b, contract=False):
    """The merged weight R W0 P in true coordinates [P3 "Methodologie" item 1].

    P is applied first (U = W0 P, per column group), then R (per row group).
    In contract mode U and the result are each rounded to bf16 once.
    The caller then resets the generators to zero and draws new permutations.
    """
    rnd = round_bf16 if contract else _identity
    W0 = np.asarray(W0, dtype=np.float64)
    QRm = [rnd(q) for q in _qs(thR, b)]
    QPm = [rnd(q) for q in _qs(thP, b)]
    U = W0.copy()
    for l, J in enumerate(_groups(tau, b)):
        U[:, J] = rnd(W0[:, J] @ QPm[l])
    W = U.copy()
    for l, I in enumerate(_groups(sigma, b)):
        W[I, :] = rnd(QRm[l] @ U[I, :])
    return W


def pack(W0, sigma, tau):
    """Working layout with the two inner permutations folded into the weight
    [P3 "Methodologie" item 2, second bullet]: W0p[i, j] = W0[sigma[i], tau[j]]."""
    return np.asarray(W0)[np.asarray(sigma)][:, np.asarray(tau)]


def unpack(W0p, sigma, tau):
    """Inverse of pack: W0[sigma[i], tau[j]] = W0p[i, j]."""
    W0p = np.asarray(W0p)
    W0 = np.empty_like(W0p)
    W0[np.ix_(np.asarray(sigma), np.asarray(tau))] = W0p
    return W0


# --------------------------------------------------------------------------
# a11: permutations drawn from a seed
# --------------------------------------------------------------------------
def mix64(z):
    """SplitMix64's output function (Steele, Lea & Flood, OOPSLA 2014):
    xor-shift 30, multiply, xor-shift 27, multiply, xor-shift 31, mod 2**64."""
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def make_permutation(seed, merge_index, side, n):
    """Uniform random permutation of 0..n-1 from (seed, merge_index, side).

    side 0 is sigma (for R), side 1 is tau (for P); merge_index 0 is the
    initial packing and counts merges after it.  A per-(merge, side) stream
    base = mix64(seed + gamma*(2*merge_index + side + 1)) gives keys
    key_i = mix64(base + gamma*(i + 1)), i.e. the SplitMix64 stream seeded
    with base; the permutation lists 0..n-1 sorted by (key_i, i).
    The pages only say the permutations are index maps [P3 "Methodologie"
    item 2]; this generator is the reading adopted for "uniform random from
    a seed".
    """
    base = mix64((seed + GOLDEN_GAMMA * (2 * merge_index + side + 1)) & _MASK64)
    keys = [mix64((base + GOLDEN_GAMMA * (i + 1)) & _MASK64) for i in range(n)]
    return np.array(sorted(range(n), key=lambda i: (keys[i], i)), dtype=np.int64)


# --------------------------------------------------------------------------
# a12: Adam on the generators (only for the multi-layer training step)
# --------------------------------------------------------------------------
def adam_step(theta, grad, m, v, step, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8):
    """Adam with bias correction (Kingma & Ba 2015, Algorithm 1), no weight
    decay; returns the new (theta, m, v).  ``step`` counts from 1."""
    theta = np.asarray(theta, dtype=np.float64)
    g = np.asarray(grad, dtype=np.float64)
    m = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** step)
    vhat = v / (1.0 - beta2 ** step)
    return theta - lr * mhat / (np.sqrt(vhat) + eps), m, v



# --------------------------------------------------------------------------
# POET-XQ: base weights stored as INT8 codes and dequantized for each use
# [P3 "Methodologie" item 5].  The pages give no granularity; the plainest
# reading is symmetric per-row codes (one scale per output feature).  The
# codes are decided in fp32, the precision a GPU decides them in.
# --------------------------------------------------------------------------
def quantize_rows(W):
    """INT8 codes and fp32 scales of a weight [m][n] (bf16 values):
    s_i = a_i / 127 with a_i = max_j |w_ij|, q_ij = clamp(rne(w_ij / s_i),
    -127, 127), both divisions in fp32 with round-to-nearest-even; a row of
    zeros gets s_i = 0 and q_i = 0.  Returns (q int8 [m][n], s float32 [m])."""
    W32 = np.asarray(W, dtype=np.float32)
    s = np.max(np.abs(W32), axis=1) / np.float32(127.0)
    s = s.astype(np.float32)
    q = np.zeros(W32.shape, dtype=np.int8)
    nz = s > 0
    r = W32[nz] / s[nz][:, None]
    q[nz] = np.clip(np.rint(r), -127, 127).astype(np.int8)
    return q, s


def dequantize_rows(q, s):
    """bf16 weight values s_i * q_ij: the product rounded to fp32, then to
    bf16 (both round-to-nearest-even).  Returned as float64."""
    p = np.asarray(s, dtype=np.float32)[:, None] * np.asarray(q, dtype=np.float32)
    return round_bf16(p.astype(np.float32).astype(np.float64))
