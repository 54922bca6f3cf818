"""GPU parity: the HIP path through the C ABI against the float64 oracle.

bf16 workloads are compared with the oracle's bf16 precision contract
(rounding to bf16 at the same storage points, float64 elsewhere), fp32
workloads with its exact mode.  Tolerances (gpu_util.compare): bf16 outputs
|d| <= 1e-3 + 2e-2|ref| + 6u rms(v), v the bf16 intermediate feeding the
output through an orthogonal block (u = 2^-8); generator gradients
|d| <= 1e-3 + 2e-2|ref| + 6e-3 rms(ref); fp32 |d| <= 1e-5 max(|ref|, rms(ref));
each with a ceiling on the fraction outside the stated bound and a normwise
bound.  Permutations, packing and zero-generator merges are bit-exact.
"""

import numpy as np
import pytest

import oracle
import workloads as WL
from gpu_util import compare, from_dev, layer_floors, make_layer, oracle_perms, to_dev, torch_mod

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def run_layer_case(inp, merge=True, repeat_check=False):
    torch = torch_mod()
    dt, b = inp["dtype"], inp["b"]
    _log("case m=%d n=%d b=%d N=%d %s" % (inp["m"], inp["n"], b, inp["N"], dt))
    lay, d = make_layer(inp)
    sigma, tau = oracle_perms(inp, 0)
    W0 = inp["W0"][1]
    thR, thP = inp["thR"][1], inp["thP"][1]
    X, gY = inp["X"][1], inp["gY"][1]
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(lay.sigma), sigma)
    assert np.array_equal(from_dev(lay.tau), tau)
    assert np.array_equal(from_dev(lay.W0p), oracle.pack(W0, sigma, tau))
    Y = lay.forward(d["X"])
    dX, dR, dP = lay.backward(d["X"], d["gY"])
    torch.cuda.synchronize()
    if repeat_check:
        Y2 = lay.forward(d["X"])
        dX2, dR2, dP2 = lay.backward(d["X"], d["gY"])
        torch.cuda.synchronize()
        assert torch.equal(Y, Y2) and torch.equal(dX, dX2) and torch.equal(dR, dR2) and torch.equal(dP, dP2)
    out = []
    contract = dt == "bf16"
    dXr, dRr, dPr, it = oracle.backward(W0, thR, thP, sigma, tau, X, gY, b, contract=contract, intermediates=True)
    Yr = oracle.forward(W0, thR, thP, sigma, tau, X, b, contract=contract)
    fl = layer_floors(W0, it)
    bk, sk = ("bf16", "sum") if contract else ("f32", "f32")
    out.append(compare(from_dev(Y), Yr, bk, "Y", floor=fl["Y"] if contract else None))
    out.append(compare(from_dev(dX), dXr, bk, "dX", floor=fl["dX"] if contract else None))
    if dRr.size:
        out.append(compare(from_dev(dR), dRr, sk, "dthR", terms=inp["N"]))
    if dPr.size:
        out.append(compare(from_dev(dP), dPr, sk, "dthP", terms=inp["N"]))
    if merge:
        lay.merge()
        torch.cuda.synchronize()
        s1, t1 = oracle_perms(inp, 1)
        assert np.array_equal(from_dev(lay.sigma), s1)
        assert np.array_equal(from_dev(lay.tau), t1)
        assert not lay.thR.any().item() and not lay.thP.any().item()
        Wn = oracle.merge(W0, thR, thP, sigma, tau, b, contract=contract)
        out.append(compare(from_dev(lay.W0p), oracle.pack(Wn, s1, t1), bk, "W0p_merged",
                           floor=fl["W"] if contract else None))
    return out


SMALL = [
    # m, n, b, N  (ragged tails, N not a multiple of 16, widths not multiples of 8)
    (96, 80, 32, 37),
    (300, 200, 64, 50),
    (256, 512, 128, 33),
    (600, 520, 256, 70),
    (1100, 700, 512, 40),
    (70, 90, 32, 1),
    (20, 40, 32, 5),       # m < b: R is the identity
    (512, 256, 256, 129),
    (4360, 4104, 256, 45),  # rows of 4096+ columns with identity tails (streaming permutation)
    (2048, 2048, 256, 45),  # K >= 2048, a multiple of 64: the 64-deep GEMM ring, few tokens
    (2112, 2240, 64, 70),   # the same with a partial last tile in n and m
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("m,n,b,N", SMALL)
def test_small_layers(m, n, b, N, dtype):
    inp = WL.small_case(11, m, n, b, N, dtype=dtype)
    run_layer_case(inp, repeat_check=(m == 600))


@pytest.mark.parametrize("b", [32, 64, 128, 256, 512])
def test_build_blocks(b):
    torch = torch_mod()
    import orthogonal_reparameterized_poetx_amd as P
    nb = 5
    rng = np.random.default_rng(b)
    theta = (rng.standard_normal((nb, b * (b - 1) // 2)) * np.sqrt(1e-3 if b > 32 else 1e-2)).astype(np.float32)
    th = to_dev(theta, "f32")
    Q32 = torch.empty(nb, b, b, dtype=torch.float32, device="cuda:0")
    Qb = torch.empty(nb, b, b, dtype=torch.bfloat16, device="cuda:0")
    QT = torch.empty(nb, b, b, dtype=torch.bfloat16, device="cuda:0")
    ws = P.make_workspace(P.build_workspace_bytes(nb, b), "cuda:0")
    P.poetx_build_blocks(th, nb, b, Q32, Qb, QT, ws)
    torch.cuda.synchronize()
    q = from_dev(Q32)
    worst = 0.0
    for l in range(nb):
        ref = oracle.cayley(oracle.unpack_skew(theta[l].astype(np.float64), b))
        # the solve's accuracy is absolute (asserted below); the fraction of
        # entries within 1e-5 of their own size is not a property of it
        compare(q[l], ref, "f32", "Q32[%d]" % l, max_strict=1.0)
        assert np.linalg.norm(q[l].T @ q[l] - np.eye(b)) < 1e-4
        worst = max(worst, float(np.abs(q[l] - ref).max()))
    _log("b=%d max |Q32 - Q| = %.3g" % (b, worst))
    # fp32-level accuracy of the exact solve (|Q_ij| <= 1; measured 0.7-1.6e-6)
    assert worst <= 2.0 ** -18
    # bf16 copies are the rounding of the fp32 result, bit for bit
    assert torch.equal(Qb, Q32.to(torch.bfloat16))
    assert torch.equal(QT, Q32.to(torch.bfloat16).transpose(1, 2))


def test_zero_generator_merge_is_exact_relayout():
    torch = torch_mod()
    inp = WL.small_case(5, 384, 320, 64, 4, dtype="bf16")
    inp["thR"] = (np.zeros_like(inp["thR"][0]), np.zeros(inp["thR"][0].shape))
    inp["thP"] = (np.zeros_like(inp["thP"][0]), np.zeros(inp["thP"][0].shape))
    lay, _ = make_layer(inp)
    for k in range(1, 4):
        lay.merge()
        torch.cuda.synchronize()
        s, t = oracle_perms(inp, k)
        assert np.array_equal(from_dev(lay.W0p), oracle.pack(inp["W0"][1], s, t))


def test_accumulate_and_empty():
    torch = torch_mod()
    inp = WL.small_case(3, 256, 256, 64, 40, dtype="bf16")
    lay, d = make_layer(inp)
    _, dR, dP = lay.backward(d["X"], d["gY"])
    dR2, dP2 = dR.clone(), dP.clone()
    lay.backward(d["X"], d["gY"], dthR=dR2, dthP=dP2, want_dx=False, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(dR2, dR + dR) and torch.equal(dP2, dP + dP)
    # N = 0: forward is a no-op, backward resets the gradients
    Xe = d["X"][:0]
    lay.forward(Xe)
    _, z1, z2 = lay.backward(Xe, d["gY"][:0], dthR=dR2, dthP=dP2, want_dx=False)
    torch.cuda.synchronize()
    assert not z1.any().item() and not z2.any().item()


@pytest.mark.parametrize("c", [1, 2])
def test_config_single(c):
    inp = WL.matrix_inputs(c, 0)
    run_layer_case(inp, repeat_check=True)


@pytest.mark.parametrize("j", range(7))
def test_config3_layerset(j):
    inp = WL.matrix_inputs(3, j)
    run_layer_case(inp, merge=(j in (0, 4, 6)))


@pytest.mark.parametrize("b", WL.C4_BLOCK_SIZES)
def test_config4_mlp(b):
    inp = WL.matrix_inputs(4, 0, b=b)
    run_layer_case(inp, merge=True)
