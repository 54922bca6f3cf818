"""Pins of the float64 oracle against what the pages and the mathematics fix.

None of these re-types the oracle's own formula: each checks a closed form, an
invariant, a brute-force construction along a different route, finite
differences, or a published test vector.
"""

import itertools
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_theta(rng, k, b, std):
    return rng.standard_normal((k, b * (b - 1) // 2)) * std


# ---------------------------------------------------------------- rounding --
def test_round_bf16_special_values():
    r = O.round_bf16
    assert r(1.0) == 1.0
    assert r(1.0 + 2.0 ** -8) == 1.0                      # tie, 1.0 is even
    assert r(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6      # tie, rounds to even
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    assert r(-1.0 - 2.0 ** -8) == -1.0
    assert r(0.0) == 0.0
    assert r(2.0 ** -130) == 2.0 ** -130                  # subnormal, exact
    assert r(3.0 * 2.0 ** -134) == 2.0 ** -132            # subnormal tie -> even


def test_round_bf16_is_nearest_representable():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(20000) * 10.0 ** rng.uniform(-6, 6, 20000)
    y = O.round_bf16(x)
    bits = y.astype(np.float32).view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)                     # y is a bf16 value
    assert np.all(y.astype(np.float32).astype(np.float64) == y)
    up = (bits + 0x10000).view(np.float32).astype(np.float64)
    dn = (bits - 0x10000).view(np.float32).astype(np.float64)
    assert np.all(np.abs(x - y) <= np.abs(x - up))
    assert np.all(np.abs(x - y) <= np.abs(x - dn))


def test_round_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(50000) * 3).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(x.astype(np.float64)), ref)


# ------------------------------------------------------------ permutations --
def test_mix64_published_vector():
    lines = [l for l in open(os.path.join(GOLDEN, "splitmix64_seed1234567.txt"))
             if l.strip() and not l.startswith("#")]
    seed = int(lines[0].split()[1])
    expect = [int(l) for l in lines[1:]]
    got = [O.mix64(seed + O.GOLDEN_GAMMA * (i + 1)) for i in range(len(expect))]
    assert got == expect


def test_permutation_is_bijection_and_deterministic():
    for n in (1, 2, 7, 256, 5632, 11008):
        p = O.make_permutation(123, 0, 0, n)
        assert p.dtype == np.int64
        assert np.array_equal(np.sort(p), np.arange(n))
        assert np.array_equal(p, O.make_permutation(123, 0, 0, n))


def test_permutation_streams_differ():
    a = O.make_permutation(5, 0, 0, 512)
    assert not np.array_equal(a, O.make_permutation(5, 0, 1, 512))
    assert not np.array_equal(a, O.make_permutation(5, 1, 0, 512))
    assert not np.array_equal(a, O.make_permutation(6, 0, 0, 512))
    # consecutive merges are not shifts of one another
    b = O.make_permutation(5, 1, 0, 512)
    assert not np.array_equal(a[1:], b[:-1])


def test_permutation_uniform_chi2():
    # all 24 permutations of 4 items, 24000 seeds: chi^2 with 23 dof
    counts = {p: 0 for p in itertools.permutations(range(4))}
    trials = 24000
    for s in range(trials):
        counts[tuple(O.make_permutation(s, 3, 1, 4))] += 1
    exp = trials / 24
    chi2 = sum((c - exp) ** 2 / exp for c in counts.values())
    assert chi2 < 49.7          # p = 0.001 critical value for 23 dof


def test_permutation_sort_order():
    # the permutation lists indices in ascending key order, ties by index
    seed, k, side, n = 99, 2, 1, 64
    base = O.mix64(seed + O.GOLDEN_GAMMA * (2 * k + side + 1))
    keys = np.array([O.mix64(base + O.GOLDEN_GAMMA * (i + 1)) for i in range(n)], dtype=np.uint64)
    p = O.make_permutation(seed, k, side, n)
    assert np.all(keys[p][1:] > keys[p][:-1])


# ----------------------------------------------------------- unpack_skew ----
def test_unpack_skew_positions():
    b = 6
    theta = np.arange(1, b * (b - 1) // 2 + 1, dtype=np.float64)
    S = O.unpack_skew(theta, b)
    p = 0
    for i in range(b):                 # row-major walk of the strict upper triangle
        for j in range(i + 1, b):
            assert S[i, j] == theta[p] and S[j, i] == -theta[p]
            assert p == i * b - i * (i + 1) // 2 + (j - i - 1)
            p += 1
    assert np.all(np.diag(S) == 0)
    assert np.array_equal(S, -S.T)


# ----------------------------------------------------------------- Cayley ---
def test_cayley_b2_closed_form():
    for a in (0.0, 0.3, -1.7, 5.0):
        Q = O.cayley(O.unpack_skew(np.array([a]), 2))
        c, s = (1 - a * a) / (1 + a * a), 2 * a / (1 + a * a)
        assert np.allclose(Q, [[c, s], [-s, c]], atol=1e-15, rtol=0)


def test_cayley_zero_is_identity():
    for b in (2, 32, 256):
        Q = O.cayley(O.unpack_skew(np.zeros(b * (b - 1) // 2), b))
        assert np.array_equal(Q, np.eye(b))


@pytest.mark.parametrize("b,var", [(32, 1e-2), (64, 1e-3), (256, 1e-3), (512, 1e-3)])
def test_cayley_orthogonal_det_one(b, var):
    rng = np.random.default_rng(b)
    S = O.unpack_skew(rng.standard_normal(b * (b - 1) // 2) * np.sqrt(var), b)
    Q = O.cayley(S)
    assert np.linalg.norm(Q.T @ Q - np.eye(b)) <= 1e-10
    assert abs(np.linalg.det(Q) - 1.0) <= 1e-10
    # Q(-S) = Q(S)^T and Q = 2 (I - S)^-1 - I
    assert np.allclose(O.cayley(-S), Q.T, atol=1e-13, rtol=0)
    assert np.allclose(Q, 2 * np.linalg.inv(np.eye(b) - S) - np.eye(b), atol=1e-12, rtol=0)


# ---------------------------------------------------------------- forward ---
def _case(rng, m, n, b, N, wstd=0.1, tstd=0.2):
    W0 = rng.standard_normal((m, n)) * wstd
    thR = _rand_theta(rng, m // b, b, tstd)
    thP = _rand_theta(rng, n // b, b, tstd)
    sigma = O.make_permutation(int(rng.integers(1 << 62)), 0, 0, m)
    tau = O.make_permutation(int(rng.integers(1 << 62)), 0, 1, n)
    X = rng.standard_normal((N, n))
    gY = rng.standard_normal((N, m))
    return W0, thR, thP, sigma, tau, X, gY


SHAPES = [(256, 256, 32, 64), (40, 24, 8, 5), (37, 50, 6, 9), (16, 16, 16, 3), (10, 7, 4, 2)]


@pytest.mark.parametrize("m,n,b,N", SHAPES)
def test_forward_matches_dense_brute_force(m, n, b, N):
    rng = np.random.default_rng([m, n, b, N])
    W0, thR, thP, sigma, tau, X, _ = _case(rng, m, n, b, N)
    R = O.dense_orthogonal(thR, sigma, b)
    P = O.dense_orthogonal(thP, tau, b)
    Y = O.forward(W0, thR, thP, sigma, tau, X, b)
    assert np.allclose(Y, X @ (R @ W0 @ P).T, atol=1e-12, rtol=0)
    assert np.allclose(R.T @ R, np.eye(m), atol=1e-12)
    v = rng.standard_normal(m)
    assert abs(np.linalg.norm(R @ v) - np.linalg.norm(v)) < 1e-12


def test_forward_zero_generators_is_plain_matmul():
    rng = np.random.default_rng(3)
    W0, thR, thP, sigma, tau, X, _ = _case(rng, 48, 32, 8, 7)
    Y = O.forward(W0, 0 * thR, 0 * thP, sigma, tau, X, 8)
    assert np.allclose(Y, np.matmul(X, W0.T), atol=1e-13, rtol=0)


def test_tail_coordinates_untouched_by_R():
    # coordinates in the identity tail of R pass W0 P x through unchanged
    rng = np.random.default_rng(4)
    m, n, b = 21, 16, 4
    W0, thR, thP, sigma, tau, X, _ = _case(rng, m, n, b, 3)
    Y = O.forward(W0, thR, thP, sigma, tau, X, b)
    Y0 = O.forward(W0, 0 * thR, thP, sigma, tau, X, b)
    tail = sigma[(m // b) * b:]
    assert np.allclose(Y[:, tail], Y0[:, tail], atol=1e-14, rtol=0)


@pytest.mark.parametrize("m,n,b", [(64, 48, 16), (256, 256, 32), (50, 30, 7)])
def test_spectral_invariance(m, n, b):
    rng = np.random.default_rng([m, n, b, 1])
    W0, thR, thP, sigma, tau, _, _ = _case(rng, m, n, b, 1)
    W = O.dense_orthogonal(thR, sigma, b) @ W0 @ O.dense_orthogonal(thP, tau, b)
    s0 = np.linalg.svd(W0, compute_uv=False)
    s1 = np.linalg.svd(W, compute_uv=False)
    assert np.max(np.abs(s0 - s1)) <= 1e-9 * s0[0]
    s2 = np.linalg.svd(O.merge(W0, thR, thP, sigma, tau, b), compute_uv=False)
    assert np.max(np.abs(s0 - s2)) <= 1e-9 * s0[0]


# --------------------------------------------------------------- backward ---
def _loss(W0, thR, thP, sigma, tau, X, gY, b):
    return float(np.sum(gY * O.forward(W0, thR, thP, sigma, tau, X, b)))


@pytest.mark.parametrize("m,n,b,N", [(10, 7, 3, 4), (12, 9, 4, 3), (8, 8, 8, 2)])
def test_backward_generators_finite_differences(m, n, b, N):
    rng = np.random.default_rng([m, n, b, N, 9])
    W0, thR, thP, sigma, tau, X, gY = _case(rng, m, n, b, N, wstd=0.5, tstd=0.4)
    _, dR, dP = O.backward(W0, thR, thP, sigma, tau, X, gY, b)
    h = 1e-6
    for th, d, side in ((thR, dR, 0), (thP, dP, 1)):
        fd = np.zeros_like(th)
        for idx in np.ndindex(th.shape):
            tp, tm = th.copy(), th.copy()
            tp[idx] += h
            tm[idx] -= h
            args_p = (tp, thP) if side == 0 else (thR, tp)
            args_m = (tm, thP) if side == 0 else (thR, tm)
            fd[idx] = (_loss(W0, *args_p, sigma, tau, X, gY, b)
                       - _loss(W0, *args_m, sigma, tau, X, gY, b)) / (2 * h)
        assert np.allclose(d, fd, atol=1e-7, rtol=1e-6), (side, np.max(np.abs(d - fd)))


def test_backward_dx_is_dense_transpose():
    rng = np.random.default_rng(11)
    m, n, b = 37, 50, 6
    W0, thR, thP, sigma, tau, X, gY = _case(rng, m, n, b, 5)
    dX, _, _ = O.backward(W0, thR, thP, sigma, tau, X, gY, b)
    W = O.dense_orthogonal(thR, sigma, b) @ W0 @ O.dense_orthogonal(thP, tau, b)
    assert np.allclose(dX, gY @ W, atol=1e-12, rtol=0)


def test_chain_rule_b2_closed_form():
    # at b=2, Q(a) = [[c, s], [-s, c]] and dQ/da is known in closed form
    rng = np.random.default_rng(2)
    for a in (0.0, 0.7, -2.5):
        G = rng.standard_normal((2, 2))
        Q = O.cayley(O.unpack_skew(np.array([a]), 2))
        dQ = np.array([[-4 * a, 2 * (1 - a * a)], [-2 * (1 - a * a), -4 * a]]) / (1 + a * a) ** 2
        assert np.allclose(O.chain_rule(G, Q), [np.sum(G * dQ)], atol=1e-13, rtol=0)


# ------------------------------------------------------------------ merge ---
@pytest.mark.parametrize("m,n,b", [(64, 48, 16), (37, 50, 6), (256, 256, 32)])
def test_merge_is_dense_product(m, n, b):
    rng = np.random.default_rng([m, n, b, 2])
    W0, thR, thP, sigma, tau, _, _ = _case(rng, m, n, b, 1)
    W = O.merge(W0, thR, thP, sigma, tau, b)
    Wd = O.dense_orthogonal(thR, sigma, b) @ W0 @ O.dense_orthogonal(thP, tau, b)
    assert np.allclose(W, Wd, atol=1e-12, rtol=0)


def test_merge_preserves_function():
    rng = np.random.default_rng(21)
    m, n, b = 40, 24, 8
    W0, thR, thP, sigma, tau, X, _ = _case(rng, m, n, b, 6)
    before = O.forward(W0, thR, thP, sigma, tau, X, b)
    W1 = O.merge(W0, thR, thP, sigma, tau, b)
    s1, t1 = O.make_permutation(77, 1, 0, m), O.make_permutation(77, 1, 1, n)
    after = O.forward(W1, 0 * thR, 0 * thP, s1, t1, X, b)
    assert np.allclose(before, after, atol=1e-12, rtol=0)


def test_zero_merge_is_pure_relayout():
    rng = np.random.default_rng(22)
    m, n, b = 40, 24, 8
    W0, thR, thP, sigma, tau, _, _ = _case(rng, m, n, b, 1)
    for contract in (False, True):
        W = O.round_bf16(W0) if contract else W0
        assert np.array_equal(O.merge(W, 0 * thR, 0 * thP, sigma, tau, b, contract=contract), W)
    Wp = O.pack(W0, sigma, tau)
    assert np.array_equal(O.unpack(Wp, sigma, tau), W0)
    assert Wp[3, 5] == W0[sigma[3], tau[5]]


# ------------------------------------------------------ bf16 contract mode ---
def test_contract_mode_reduces_to_exact_without_rounding(monkeypatch):
    rng = np.random.default_rng(31)
    m, n, b = 24, 40, 8
    W0, thR, thP, sigma, tau, X, gY = _case(rng, m, n, b, 5)
    ref_f = O.forward(W0, thR, thP, sigma, tau, X, b)
    ref_b = O.backward(W0, thR, thP, sigma, tau, X, gY, b)
    ref_m = O.merge(W0, thR, thP, sigma, tau, b)
    import oracle.poetx as P
    monkeypatch.setattr(P, "round_bf16", lambda x: np.asarray(x, dtype=np.float64))
    assert np.array_equal(P.forward(W0, thR, thP, sigma, tau, X, b, contract=True), ref_f)
    got = P.backward(W0, thR, thP, sigma, tau, X, gY, b, contract=True)
    for g, r in zip(got, ref_b):
        assert np.array_equal(g, r)
    assert np.array_equal(P.merge(W0, thR, thP, sigma, tau, b, contract=True), ref_m)


def test_contract_mode_outputs_are_bf16_and_close():
    rng = np.random.default_rng(32)
    m, n, b = 64, 48, 16
    W0, thR, thP, sigma, tau, X, gY = _case(rng, m, n, b, 33)
    W0 = O.round_bf16(W0)
    X = O.round_bf16(X)
    gY = O.round_bf16(gY)
    Yc = O.forward(W0, thR, thP, sigma, tau, X, b, contract=True)
    Ye = O.forward(W0, thR, thP, sigma, tau, X, b)
    assert np.array_equal(O.round_bf16(Yc), Yc)
    assert np.linalg.norm(Yc - Ye) <= 2e-2 * np.linalg.norm(Ye)
    dXc, dRc, dPc = O.backward(W0, thR, thP, sigma, tau, X, gY, b, contract=True)
    dXe, dRe, dPe = O.backward(W0, thR, thP, sigma, tau, X, gY, b)
    assert np.array_equal(O.round_bf16(dXc), dXc)
    for c, e in ((dXc, dXe), (dRc, dRe), (dPc, dPe)):
        assert np.linalg.norm(c - e) <= 3e-2 * np.linalg.norm(e)


# Exact rational arithmetic for the rounding-point pin below: products of
# bf16 values are formed without error and rounded to bf16 once, by integer
# arithmetic on the fraction (no float64 step).
def _bf16_exact(x):
    from fractions import Fraction
    x = Fraction(x)
    if x == 0:
        return x
    sgn, a = (1, x) if x > 0 else (-1, -x)
    # e with 2^(e-1) <= a < 2^e, then the spacing of 8 significant bits
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** (e - 1) > a:
        e -= 1
    while Fraction(2) ** e <= a:
        e += 1
    q = Fraction(2) ** (e - 8)
    r = a / q
    fl = r.numerator // r.denominator
    rem = r - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sgn * fl * q


def _frac_mat(a):
    from fractions import Fraction
    return [[Fraction(float(v)) for v in row] for row in np.atleast_2d(a)]


def _fmatmul(A, B):
    return [[sum(A[i][k] * B[k][j] for k in range(len(B))) for j in range(len(B[0]))] for i in range(len(A))]


def _ftrans(A):
    return [list(r) for r in zip(*A)]


def _fround(A):
    return [[_bf16_exact(v) for v in row] for row in A]


def _dense_from_b2(theta, perm, dim):
    """Pi^T diag(Q_0.., I) Pi for b = 2, each Q_l in closed form as exact
    rationals, rounded to bf16: Q = [[c, s], [-s, c]], c = (1-a^2)/(1+a^2),
    s = 2a/(1+a^2) for the generator a; gather convention (Pi v)_i = v[perm[i]]."""
    from fractions import Fraction
    D = [[Fraction(int(i == j)) for j in range(dim)] for i in range(dim)]
    for l, a in enumerate(np.asarray(theta)[:, 0]):
        a = Fraction(float(a))
        c, s = (1 - a * a) / (1 + a * a), 2 * a / (1 + a * a)
        q = [[c, s], [-s, c]]
        for i in range(2):
            for j in range(2):
                D[2 * l + i][2 * l + j] = _bf16_exact(q[i][j])
    Pi = [[Fraction(int(perm[i] == j)) for j in range(dim)] for i in range(dim)]
    return _fmatmul(_ftrans(Pi), _fmatmul(D, Pi))


def test_contract_mode_rounding_points_exact():
    """Every stored bf16 intermediate of the contract mode (z1, z2, Y, gZ2,
    gZ1, dX) equals the exactly computed product of its rounded inputs,
    rounded to bf16 once, and the fp32-kept reductions G_R, G_P are the plain
    sums of products of those rounded values [P1 实践 5: low-precision storage,
    high-precision accumulation].  The route is independent of the oracle's:
    dense permuted block matrices with b = 2 blocks in closed form, exact
    rational arithmetic, and rounding by integer arithmetic.  Identity tails on
    both sides (m, n odd)."""
    rng = np.random.default_rng(77)
    m, n, b, N = 9, 7, 2, 5
    W0 = O.round_bf16(rng.standard_normal((m, n)) * 0.4)
    X = O.round_bf16(rng.standard_normal((N, n)))
    gY = O.round_bf16(rng.standard_normal((N, m)))
    thR = _rand_theta(rng, m // b, b, 0.7)
    thP = _rand_theta(rng, n // b, b, 0.7)
    sigma = O.make_permutation(91, 0, 0, m)
    tau = O.make_permutation(91, 0, 1, n)
    dXo, dRo, dPo, it = O.backward(W0, thR, thP, sigma, tau, X, gY, b, contract=True, intermediates=True)
    Yo = O.forward(W0, thR, thP, sigma, tau, X, b, contract=True)

    Rm = _dense_from_b2(thR, sigma, m)
    Pm = _dense_from_b2(thP, tau, n)
    Wf, Xf, gf = _frac_mat(W0), _frac_mat(X), _frac_mat(gY)
    Z1 = _fround(_fmatmul(Xf, _ftrans(Pm)))
    Z2 = _fround(_fmatmul(Z1, _ftrans(Wf)))
    Y = _fround(_fmatmul(Z2, _ftrans(Rm)))
    gZ2 = _fround(_fmatmul(gf, Rm))
    gZ1 = _fround(_fmatmul(gZ2, Wf))
    dX = _fround(_fmatmul(gZ1, Pm))
    as64 = lambda A: np.array([[float(v) for v in r] for r in A])
    for name, want, got in (("Z1", Z1, it["Z1"]), ("Z2", Z2, it["Z2"]), ("Y", Y, Yo), ("gZ2", gZ2, it["gZ2"]),
                            ("gZ1", gZ1, it["gZ1"]), ("dX", dX, dXo)):
        assert np.array_equal(as64(want), got), name
    # G_l = (upstream rows)^T (kept activation rows) over the group's columns
    for G, up, act, perm in ((it["GR"], gf, Z2, sigma), (it["GP"], gZ1, Xf, tau)):
        for l, Gl in enumerate(G):
            cols = perm[2 * l:2 * l + 2]
            want = [[sum(up[t][cols[i]] * act[t][cols[j]] for t in range(N)) for j in range(2)] for i in range(2)]
            assert np.allclose(as64(want), Gl, rtol=1e-14, atol=1e-14)


# ------------------------------------------------------------------- Adam ---
def test_adam_first_step_closed_form():
    g = np.array([0.5, -2.0, 1e-3, 0.0])
    th, m, v = O.adam_step(np.ones(4), g, np.zeros(4), np.zeros(4), 1, lr=0.1)
    # m_hat = g and v_hat = g^2 at step 1, so the step is lr * g / (|g| + eps)
    assert np.allclose(th, 1.0 - 0.1 * g / (np.abs(g) + 1e-8), atol=1e-15, rtol=0)
    assert np.allclose(m, 0.1 * g) and np.allclose(v, 0.001 * g * g)


def test_adam_second_step_by_hand():
    th, m, v = O.adam_step(np.array([0.0]), np.array([1.0]), np.zeros(1), np.zeros(1), 1, lr=1.0)
    th, m, v = O.adam_step(th, np.array([-1.0]), m, v, 2, lr=1.0)
    # m2 = 0.9*0.1 - 0.1 = -0.01 ; v2 = 0.999*0.001 + 0.001 = 0.001999
    mhat = -0.01 / (1 - 0.81)
    vhat = 0.001999 / (1 - 0.998001)
    assert np.allclose(th, [-(1 / (1 + 1e-8)) - mhat / (np.sqrt(vhat) + 1e-8)], atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# POET-XQ weight codes [P3 "Methodologie" item 5]: symmetric per-row INT8
# --------------------------------------------------------------------------
def test_quantize_rows_worked_examples():
    u = 2.0 ** -7
    W = np.array([[127 * u, -64 * u, 3 * u, 0.0],          # absmax 127 u: scale u exactly, codes = integers
                  [127 * u, 2.5 * u, -2.5 * u, 1.5 * u],   # ties round to even: 2, -2, 2
                  [0.0, 0.0, 0.0, 0.0],                    # zero row: scale 0, codes 0
                  [-3.0, 1.0, 0.0, 0.5]])                  # negative maximum
    q, s = O.quantize_rows(W)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert s[0] == u and s[1] == u and s[2] == 0.0
    assert s[3] == np.float32(3.0) / np.float32(127.0)
    assert q[0].tolist() == [127, -64, 3, 0]
    assert q[1].tolist() == [127, 2, -2, 2]
    assert q[2].tolist() == [0, 0, 0, 0]
    assert q[3].tolist() == [-127, 42, 0, 21]            # 127/3 = 42.33, 127/6 = 21.17
    D = O.dequantize_rows(q, s)
    assert np.array_equal(D[:3], np.array([[127 * u, -64 * u, 3 * u, 0], [127 * u, 2 * u, -2 * u, 2 * u], [0] * 4]))
    assert D[3, 0] == -3.0                               # 127 * fp32(3/127) rounds back to 3 in bf16


def test_quantize_rows_bounds_and_symmetries():
    rng = np.random.default_rng(17)
    W = O.round_bf16(rng.standard_normal((64, 300)) * np.exp(rng.uniform(-6, 2, (64, 1))))
    q, s = O.quantize_rows(W)
    sq = s.astype(np.float64)[:, None] * q
    # rounding to the nearest code: within half a step, plus the fp32
    # rounding of the quotient w / s (at most 127 * 2^-24 steps), which can
    # move a value a hair below a half-way point onto it
    assert np.all(np.abs(sq - W) <= s[:, None] * (0.5 + 127 * 2.0 ** -24) * (1 + 1e-9))
    assert np.all(np.abs(q).max(axis=1) == 127)
    # the bf16 dequantized value adds at most half a bf16 ulp of the product
    # (8 significant bits: 2^-8 relative), and the fp32 product 2^-24 more
    D = O.dequantize_rows(q, s)
    assert np.all(np.abs(D - sq) <= (2.0 ** -8 + 2.0 ** -23) * np.abs(sq))
    # odd symmetry and equivariance under row and column permutations
    qn, sn = O.quantize_rows(-W)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    pr, pc = rng.permutation(64), rng.permutation(300)
    qp, sp = O.quantize_rows(W[pr][:, pc])
    assert np.array_equal(qp, q[pr][:, pc]) and np.array_equal(sp, s[pr])


def test_dequantize_rows_matches_torch_rounding():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    q = rng.integers(-127, 128, (40, 77)).astype(np.int8)
    s = (np.abs(rng.standard_normal(40)) * 1e-2).astype(np.float32)
    ref = (torch.from_numpy(s)[:, None] * torch.from_numpy(q).to(torch.float32)).to(torch.bfloat16).to(torch.float64)
    assert np.array_equal(O.dequantize_rows(q, s), ref.numpy())


# --------------------------------------------------------------------------
# CNP: truncated Neumann form of the Cayley map [P3 "Methodologie" item 4]
# --------------------------------------------------------------------------
@pytest.mark.parametrize("k", range(1, 7))
def test_cayley_neumann_closed_form_b2(k):
    # S = [[0, a], [-a, 0]] has S^2 = -a^2 I: the odd powers are S (-a^2)^m,
    # the even ones (-a^2)^m I, so the truncated sums are geometric
    a = 0.3
    S = np.array([[0.0, a], [-a, 0.0]])
    odd = sum((-a * a) ** m for m in range((k - 1) // 2 + 1))          # j = 2m + 1 <= k
    even = sum((-a * a) ** m for m in range(1, k // 2 + 1))           # j = 2m <= k, m >= 1
    want = np.eye(2) + 2.0 * (odd * S + even * np.eye(2))
    assert np.allclose(O.cayley_neumann(S, k), want, rtol=0, atol=1e-15)


@pytest.mark.parametrize("k", range(1, 7))
def test_cnp_error_bound_two_sided_b2(k):
    """At b = 2, S = [[0, a], [-a, 0]]: the dropped tail 2 S^(k+1) (I - S)^-1
    is a scaled rotation, so its 2-norm is 2|a|^(k+1) / sqrt(1 + a^2) exactly
    ((I - S)^-1 = (I + S)/(1 + a^2)).  The bound uses f = ||S||_F = sqrt(2)|a|,
    so bound / tail = 2^((k+1)/2) sqrt(1 + a^2) / (1 - f): never below 1, and
    for small a it tends to 2^((k+1)/2), the Frobenius-to-spectral slack of S
    to the power k+1.  A bound one power too loose (f^k) would exceed that
    limit by 1/f."""
    for a in (1e-4, 0.05, 0.3, -0.2):
        S = np.array([[0.0, a], [-a, 0.0]])
        tail = np.linalg.norm(O.cayley(S) - O.cayley_neumann(S, k), 2)
        want_tail = 2.0 * abs(a) ** (k + 1) / np.sqrt(1.0 + a * a)
        # the difference of two O(1) float64 matrices: absolute error ~1e-16
        assert abs(tail - want_tail) <= 1e-14
        bound = O.cnp_error_bound(S, k)
        assert bound >= want_tail * (1 - 1e-12)
        lo = 2.0 ** ((k + 1) / 2)
        hi = lo * np.sqrt(1 + a * a) / (1 - np.sqrt(2) * abs(a))
        assert lo * (1 - 1e-12) <= bound / want_tail <= hi * (1 + 1e-12)
        if abs(a) <= 1e-4:
            assert bound / want_tail <= lo * (1 + 2e-4)


def test_cayley_neumann_limits_and_bound():
    assert np.array_equal(O.cayley_neumann(np.zeros((8, 8)), 5), np.eye(8))
    rng = np.random.default_rng(21)
    for b, scale in [(8, 0.05), (32, 0.004), (64, 0.001)]:
        S = O.unpack_skew(rng.standard_normal(b * (b - 1) // 2) * scale, b)
        assert np.array_equal(O.cayley_neumann(S, 1), np.eye(b) + 2.0 * S)
        exact = O.cayley(S)
        prev = np.inf
        for k in range(1, 9):
            err = np.linalg.norm(O.cayley_neumann(S, k) - exact, 2)
            assert err <= O.cnp_error_bound(S, k) * (1 + 1e-9) + 1e-14
            assert err <= prev + 1e-15          # more terms never hurt while ||S|| < 1
            prev = err
    big = O.unpack_skew(rng.standard_normal(64 * 63 // 2) * 0.1, 64)
    assert O.cnp_error_bound(big, 6) == np.inf
