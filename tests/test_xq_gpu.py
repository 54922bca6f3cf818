"""GPU parity of the INT8 weight storage (POET-XQ, POETX_W0_INT8).

The codes and scales are integers and fp32 values decided in fp32 on both
sides, so the quantization kernel must equal oracle.quantize_rows bit for bit,
and the dequantized weight oracle.dequantize_rows.  A pass of an INT8 layer
must equal, bit for bit, the same pass of the bf16 layer whose working-layout
weight holds the dequantized values (same permutations and generators), and
meet the oracle bound with that weight.  A merge merges the dequantized weight
and quantizes the result: compared with the oracle's merge of the same weight,
quantized by oracle.quantize_rows, after dequantization.
"""

import numpy as np
import pytest

import oracle
import workloads as WL
from gpu_util import compare, from_dev, layer_floors, oracle_perms, to_dev, torch_mod

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _codes(lay):
    """(codes int64 [m][n], scales float32 [m]) of an INT8 layer's W0p."""
    torch_mod().cuda.synchronize()
    m, n = lay.m, lay.n
    raw = lay.W0p.cpu().numpy()
    off = (m * n + 255) // 256 * 256
    q = raw[:m * n].view(np.int8).reshape(m, n).astype(np.int64)
    s = raw[off:off + 4 * m].view(np.float32).copy()
    return q, s


@pytest.mark.parametrize("m,n", [(300, 520), (64, 77), (1100, 2048)])
def test_quantize_and_dequantize_match_oracle(m, n):
    torch = torch_mod()
    import orthogonal_reparameterized_poetx_amd as P
    _log("quantize m=%d n=%d" % (m, n))
    rng = np.random.default_rng(m + n)
    W = rng.standard_normal((m, n)) * np.exp(rng.uniform(-8, 3, (m, 1)))
    W[3] = 0.0                                     # a zero row
    W[5, :4] = [127 * 2.0 ** -7, 2.5 * 2.0 ** -7, -2.5 * 2.0 ** -7, 1.5 * 2.0 ** -7]
    W[5, 4:] = 0.0                                 # ties to even
    Wb = WL.to_bf16_bits(W)
    lay = P.PoetxLayer(m, n, 32, "bf16", "cuda:0", w0_int8=True)
    lay.pack(to_dev(Wb, "bf16"))                   # quantize, then the merge relayout
    # quantize the bf16 weight directly into a fresh buffer
    Wq = torch.zeros(P.w0_bytes(lay.layer), dtype=torch.uint8, device="cuda:0")
    P.poetx_quantize_w0(lay.layer, to_dev(Wb, "bf16"), Wq)
    lay.W0p.copy_(Wq)
    q, s = _codes(lay)
    qr, sr = oracle.quantize_rows(WL.bf16_bits_to_f64(Wb))
    assert np.array_equal(s, sr)
    assert np.array_equal(q, qr.astype(np.int64))
    assert np.array_equal(from_dev(lay.weight()), oracle.dequantize_rows(qr, sr))


# n % 16 or m % 8 nonzero: each pass dequantizes into its workspace; the
# others go through the fused GEMM (ragged tiles, K below and above the ring)
@pytest.mark.parametrize("m,n,b,N", [(600, 520, 256, 70), (2048, 2048, 256, 45), (512, 256, 64, 33),
                                     (600, 528, 128, 300), (96, 64, 32, 130)])
def test_int8_layer_equals_bf16_layer_on_dequantized_weight(m, n, b, N):
    torch = torch_mod()
    import orthogonal_reparameterized_poetx_amd as P
    from orthogonal_reparameterized_poetx_amd import build_layer_blocks
    inp = WL.small_case(90, m, n, b, N, dtype="bf16")
    _log("int8 layer m=%d n=%d b=%d N=%d" % (m, n, b, N))
    d = {k: to_dev(inp[k][0], "bf16" if k in ("W0", "X", "gY") else "f32") for k in ("W0", "thR", "thP", "X", "gY")}
    l8 = P.PoetxLayer(m, n, b, "bf16", "cuda:0", perm_seed=inp["perm_seed"], w0_int8=True)
    l8.pack(d["W0"])
    l8.thR.copy_(d["thR"])
    l8.thP.copy_(d["thP"])
    l16 = P.PoetxLayer(m, n, b, "bf16", "cuda:0", perm_seed=inp["perm_seed"])
    l16.W0p.copy_(l8.weight())
    l16.sigma.copy_(l8.sigma)
    l16.tau.copy_(l8.tau)
    l16.thR.copy_(d["thR"])
    l16.thP.copy_(d["thP"])
    l16.merges = l8.merges
    outs = []
    for lay in (l8, l16):
        Y = lay.forward(d["X"])
        dX, dR, dP = lay.backward(d["X"], d["gY"])
        build_layer_blocks([lay], "forward")
        build_layer_blocks([lay], "backward")
        Yb = lay.forward_blocks(d["X"])
        Yz, Z2 = lay.forward_blocks_z2(d["X"])
        dXq, GR, GP = (t.clone() for t in lay.backward_blocks_dq(d["X"], d["gY"]))
        dXz, GRz, GPz = (t.clone() for t in lay.backward_blocks_dq_z2(d["X"], d["gY"], Z2))
        outs.append([Y, dX, dR, dP, Yb, Yz, Z2, dXq, GR, GP, dXz, GRz, GPz])
    torch.cuda.synchronize()
    for a, c in zip(*outs):
        assert torch.equal(a, c)
    # the oracle with the dequantized weight in true coordinates
    sigma, tau = oracle_perms(inp, 0)
    assert np.array_equal(from_dev(l8.sigma), sigma) and np.array_equal(from_dev(l8.tau), tau)
    # the layer quantizes the true-coordinate weight by rows (the packing
    # relayout moves whole rows with their scales), so the weight its passes
    # use is the oracle's per-row codes of W0, dequantized
    W0d = oracle.dequantize_rows(*oracle.quantize_rows(inp["W0"][1]))
    assert np.array_equal(from_dev(l8.weight()), oracle.pack(W0d, sigma, tau))
    thR, thP, X, gY = inp["thR"][1], inp["thP"][1], inp["X"][1], inp["gY"][1]
    Y, dX, dR, dP = (from_dev(t) for t in outs[0][:4])
    dXr, dRr, dPr, it = oracle.backward(W0d, thR, thP, sigma, tau, X, gY, b, contract=True, intermediates=True)
    fl = layer_floors(W0d, it)
    compare(Y, oracle.forward(W0d, thR, thP, sigma, tau, X, b, contract=True), "bf16", "Y", floor=fl["Y"])
    compare(dX, dXr, "bf16", "dX", floor=fl["dX"])
    compare(dR, dRr, "sum", "dthR", terms=N)
    compare(dP, dPr, "sum", "dthP", terms=N)


@pytest.mark.parametrize("m,n,b", [(600, 520, 256), (512, 768, 128), (1100, 700, 512)])
def test_int8_merge_matches_oracle(m, n, b):
    torch = torch_mod()
    import orthogonal_reparameterized_poetx_amd as P
    inp = WL.small_case(95, m, n, b, 8, dtype="bf16")
    _log("int8 merge m=%d n=%d b=%d" % (m, n, b))
    l8 = P.PoetxLayer(m, n, b, "bf16", "cuda:0", perm_seed=inp["perm_seed"], w0_int8=True)
    l8.pack(to_dev(inp["W0"][0], "bf16"))
    l8.thR.copy_(to_dev(inp["thR"][0], "f32"))
    l8.thP.copy_(to_dev(inp["thP"][0], "f32"))
    sigma, tau = oracle_perms(inp, 0)
    W0d = oracle.dequantize_rows(*oracle.quantize_rows(inp["W0"][1]))
    assert np.array_equal(from_dev(l8.weight()), oracle.pack(W0d, sigma, tau))
    l8.merge()
    torch.cuda.synchronize()
    s1, t1 = oracle_perms(inp, 1)
    assert np.array_equal(from_dev(l8.sigma), s1) and np.array_equal(from_dev(l8.tau), t1)
    assert not l8.thR.any().item() and not l8.thP.any().item()
    Wn = oracle.merge(W0d, inp["thR"][1], inp["thP"][1], sigma, tau, b, contract=True)
    qr, sr = oracle.quantize_rows(oracle.pack(Wn, s1, t1))
    q, s = _codes(l8)
    got = from_dev(l8.weight())
    ref = oracle.dequantize_rows(qr, sr)
    same = float(np.mean(q == qr))
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    # the GPU's merged bf16 values match the oracle's to the merge tolerance,
    # so they differ from them by an ulp now and then; the code of such a
    # value (and the scale of its row, for the row's largest element) can
    # then land one step away.  Codes: most equal, none more than a step
    # apart; weights: within two steps of the oracle's unquantized merge
    # (half a step of code rounding, up to half a step of bf16 rounding of
    # s * q near the row's maximum, and a bf16 ulp of the merged value, at
    # most one step there), normwise like the merge.
    Wp = oracle.pack(Wn, s1, t1)
    step = np.abs(got - Wp) / np.where(sr > 0, sr, 1.0)[:, None]
    _log("  merged codes equal %.4f, max |W - merge| %.3g steps, rel_norm %.3g" % (same, step.max(), rel))
    assert same > 0.9 and np.all(np.abs(q - qr) <= 1)
    assert np.allclose(s, sr, rtol=2 ** -7, atol=0)
    assert np.all(step <= 2.0) and rel <= 4e-3
