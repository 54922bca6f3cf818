"""Seeded synthetic workloads for the POET-X layer hot path.

This module only draws numbers and stores them in the working dtypes; it holds
none of the method's arithmetic.  It is shared by the tests, the benchmark and
the smoke check, so the HIP path and the float64 oracle see identical inputs.

Shapes and distributions are those of the five workloads the layer path is
measured on (second argument of N(., .) is the variance):

1. ``c1``  one 256x256 fp32 layer, b=32, 64 tokens; W0 ~ N(0, 1/256),
   generators ~ N(0, 1e-2), X and gY ~ N(0, 1); fwd, bwd, one merge.
2. ``c2``  one 2048x2048 bf16 layer, b=256, 4096 tokens (16 x 256);
   W0 ~ N(0, 1/2048), generators ~ N(0, 1e-3) fp32; fwd+bwd, one merge.
3. ``c3``  LLaMA-1B-shaped layer set (hidden 2048): q, k, v, o 2048x2048,
   gate, up 5632x2048, down 2048x5632; bf16, b=256, 8192 tokens (32 x 256);
   W0 ~ N(0, 0.02^2), generators ~ N(0, 1e-3); fwd+bwd over all seven.
4. ``c4``  LLaMA-7B-shaped MLP projection 11008x4096 bf16, b in
   {64, 128, 256, 512} (at 512 the R side has 21 blocks and a 256-wide
   identity tail), 8192 tokens; fwd+bwd and merge.
5. ``c5``  24 layers of c3 shapes (168 matrices) resident in HBM; one training
   step (fwd all, bwd all with recompute, Adam on the generators, global
   merge with re-permutation).

No public dataset is involved: the pages pre-train LLaMA models on an unnamed
corpus, and these synthetic tensors with the layers' shapes stand in for
those activations.

Seeds: Gaussian values come from ``numpy.random.default_rng([c, j, s])`` in
float64 and are then stored in the config's dtype (round to nearest even).
``c`` is the config number, ``j`` the matrix index (q, k, v, o, gate, up,
down = 0..6; in c5 ``j = 7*layer + idx``), and ``s`` the stream: 1 W0,
2 theta_R, 3 theta_P, 4 X (keyed by the first matrix that consumes that input
width), 5 gY.  The layout permutations use ``perm_seed(c, j)``.
"""

import numpy as np

LAYER_SET = (("q", 2048, 2048), ("k", 2048, 2048), ("v", 2048, 2048), ("o", 2048, 2048),
             ("gate", 5632, 2048), ("up", 5632, 2048), ("down", 2048, 5632))


def _cfg(name, dtype, mats, b, N, w_var, theta_var, layers=1):
    return dict(name=name, dtype=dtype, mats=tuple(mats), b=b, N=N, w_var=w_var,
                theta_var=theta_var, layers=layers)


CONFIGS = {
    1: _cfg("layer256_fp32_b32", "f32", [("w", 256, 256)], 32, 64, 1.0 / 256, 1e-2),
    2: _cfg("square2048_bf16_b256", "bf16", [("w", 2048, 2048)], 256, 4096, 1.0 / 2048, 1e-3),
    3: _cfg("llama1b_layerset_bf16_b256", "bf16", LAYER_SET, 256, 8192, 0.02 ** 2, 1e-3),
    4: _cfg("llama7b_mlp_11008x4096_bf16", "bf16", [("mlp", 11008, 4096)], 512, 8192, 0.02 ** 2, 1e-3),
    5: _cfg("llama1b_24layer_stack_bf16_b256", "bf16", LAYER_SET, 256, 8192, 0.02 ** 2, 1e-3, layers=24),
}
C4_BLOCK_SIZES = (64, 128, 256, 512)


def perm_seed(c, j):
    """64-bit seed of the layout permutations of matrix j in config c."""
    return (int(c) << 32) | (int(j) << 8) | 6


def gaussian(c, j, s, shape, var):
    """float64 N(0, var) samples from the (config, matrix, stream) seed."""
    rng = np.random.default_rng([int(c), int(j), int(s)])
    return rng.standard_normal(shape) * np.sqrt(var)


def to_bf16_bits(x):
    """float64 -> bfloat16 bit patterns (uint16), round to nearest even via
    float32.  Inputs only; values are data, not part of the method."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(bits):
    """Exact float64 values of bfloat16 bit patterns."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def stored(x, dtype):
    """(storage array, exact float64 value) for x in dtype 'f32' or 'bf16'.

    The storage array is float32 for 'f32' and uint16 bit patterns for 'bf16'.
    """
    if dtype == "f32":
        s = np.asarray(x, dtype=np.float32)
        return s, s.astype(np.float64)
    if dtype == "bf16":
        s = to_bf16_bits(x)
        return s, bf16_bits_to_f64(s)
    raise ValueError(dtype)


def input_owner(cfg, j):
    """Matrix index whose seed keys the input of matrix j (first consumer of
    that input width within the layer)."""
    n = cfg["mats"][j % len(cfg["mats"])][2]
    base = j - (j % len(cfg["mats"]))
    for i, (_, _, ni) in enumerate(cfg["mats"]):
        if ni == n:
            return base + i
    raise AssertionError


def matrix_inputs(c, j, N=None, b=None, rows=None):
    """All inputs of matrix j of config c.

    Returns a dict with m, n, b, N, dtype, and for each of W0, thR, thP, X, gY
    the pair (storage, float64 value).  ``rows`` optionally restricts X and gY
    to a subset of token rows (drawn from the full-size stream, then sliced).
    Generators are fp32 [k, b(b-1)/2].
    """
    cfg = CONFIGS[c]
    name, m, n = cfg["mats"][j % len(cfg["mats"])]
    b = cfg["b"] if b is None else b
    N = cfg["N"] if N is None else N
    dt = cfg["dtype"]
    nt = b * (b - 1) // 2
    out = dict(name=name, m=m, n=n, b=b, N=N, dtype=dt, perm_seed=perm_seed(c, j))
    out["W0"] = stored(gaussian(c, j, 1, (m, n), cfg["w_var"]), dt)
    # a block size other than the config's own (the c4 sweep) gets its own draw
    tj = j if b == cfg["b"] else 1000 * b + j
    out["thR"] = stored(gaussian(c, tj, 2, (m // b, nt), cfg["theta_var"]), "f32")
    out["thP"] = stored(gaussian(c, tj, 3, (n // b, nt), cfg["theta_var"]), "f32")
    X = gaussian(c, input_owner(cfg, j), 4, (N, n), 1.0)
    gY = gaussian(c, j, 5, (N, m), 1.0)
    if rows is not None:
        X, gY = X[rows], gY[rows]
    out["X"] = stored(X, dt)
    out["gY"] = stored(gY, dt)
    return out


def small_case(seed, m, n, b, N, dtype="bf16", w_std=0.05, theta_std=0.03):
    """A small seeded case of arbitrary shape (for parity tests with ragged
    tails and edge cases).  Same structure as ``matrix_inputs``."""
    rng = np.random.default_rng([7777, int(seed), m, n, b, N])
    nt = b * (b - 1) // 2
    out = dict(name="small", m=m, n=n, b=b, N=N, dtype=dtype, perm_seed=(int(seed) << 8) | 6)
    out["W0"] = stored(rng.standard_normal((m, n)) * w_std, dtype)
    out["thR"] = stored(rng.standard_normal((m // b, nt)) * theta_std, "f32")
    out["thP"] = stored(rng.standard_normal((n // b, nt)) * theta_std, "f32")
    out["X"] = stored(rng.standard_normal((N, n)), dtype)
    out["gY"] = stored(rng.standard_normal((N, m)), dtype)
    return out
