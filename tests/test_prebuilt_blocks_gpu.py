"""GPU parity of the batched builder and the prebuilt-block entry points.

poetx_build_block_sets must give, for every set, the blocks poetx_build_blocks
gives for that set alone, bit for bit (one block never depends on another, and
both run the same kernels).  poetx_forward_blocks / poetx_backward_blocks with
blocks rebuilt from the generators must reproduce poetx_forward /
poetx_backward bit for bit, and so meet the oracle bound of those calls.
"""

import numpy as np
import pytest

import oracle
import workloads as WL
from gpu_util import compare, from_dev, layer_floors, make_layer, oracle_perms, to_dev, torch_mod

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("b,counts", [
    (32, [3, 0, 5, 1, 2, 7, 1, 4, 0, 2, 6, 1, 3, 2, 5, 1, 1, 2, 3, 4] * 3 + [2] * 10),   # 70 sets: two launches
    (64, [4, 9]),
    (128, [2, 1, 3]),
    (256, [5, 3, 1, 2]),
    (512, [2, 1]),
])
def test_block_sets_match_single_builds(b, counts):
    torch = torch_mod()
    import orthogonal_reparameterized_poetx_amd as P
    _log("block sets b=%d counts=%s" % (b, counts))
    rng = np.random.default_rng(1000 + b)
    dev = "cuda:0"
    nt = b * (b - 1) // 2
    sets, single, host = [], [], []
    for i, nb in enumerate(counts):
        th_h = (rng.standard_normal((max(nb, 1), nt)) * np.sqrt(1e-3)).astype(np.float32)[:nb]
        host.append(th_h)
        th = to_dev(th_h, "f32")
        # vary which outputs a set asks for
        want = [(True, True, True), (True, False, False), (False, True, True), (False, False, True)][i % 4]
        q32 = torch.full((nb, b, b), np.nan, dtype=torch.float32, device=dev) if want[0] else None
        qb = torch.zeros(nb, b, b, dtype=torch.bfloat16, device=dev) if want[1] else None
        qt = torch.zeros(nb, b, b, dtype=torch.bfloat16, device=dev) if want[2] else None
        sets.append((th, nb, q32, qb, qt))
        single.append(tuple(torch.empty(nb, b, b, dtype=t, device=dev)
                            for t in (torch.float32, torch.bfloat16, torch.bfloat16)))
    ws = P.make_workspace(P.build_workspace_bytes(sum(counts), b), dev)
    P.poetx_build_block_sets(sets, b, ws)
    for (th, nb, _, _, _), (q32, qb, qt) in zip(sets, single):
        ws1 = P.make_workspace(P.build_workspace_bytes(nb, b), dev)
        P.poetx_build_blocks(th, nb, b, q32, qb, qt, ws1)
    torch.cuda.synchronize()
    for (th, nb, q32, qb, qt), ref in zip(sets, single):
        for got, want in zip((q32, qb, qt), ref):
            if got is not None:
                assert torch.equal(got, want)
    # one spot check against the oracle
    i = next(i for i, s in enumerate(sets) if s[1] > 0 and s[2] is not None)
    ref = oracle.cayley(oracle.unpack_skew(host[i][0].astype(np.float64), b))
    # the solve's accuracy is absolute: see test_build_blocks
    compare(from_dev(sets[i][2])[0], ref, "f32", "Q32[0]", max_strict=1.0)


LAYER_GROUPS = [
    # (dtype, [(m, n)], b, N): several layers sharing one batched build
    ("bf16", [(600, 520), (256, 768), (512, 512)], 256, 70),
    ("bf16", [(300, 200), (130, 64), (64, 300)], 64, 45),
    ("f32", [(96, 80), (200, 96)], 32, 37),
    ("bf16", [(1100, 700), (512, 1024)], 512, 24),
]


@pytest.mark.parametrize("dtype,shapes,b,N", LAYER_GROUPS)
def test_prebuilt_blocks_match_self_building_calls(dtype, shapes, b, N):
    torch = torch_mod()
    from orthogonal_reparameterized_poetx_amd import build_layer_blocks
    layers, inps, ds = [], [], []
    for i, (m, n) in enumerate(shapes):
        inp = WL.small_case(40 + i, m, n, b, N, dtype=dtype)
        lay, d = make_layer(inp)
        layers.append(lay), inps.append(inp), ds.append(d)
    _log("prebuilt %s b=%d N=%d shapes=%s" % (dtype, b, N, shapes))
    build_layer_blocks(layers, "forward")
    build_layer_blocks(layers, "backward")
    for lay, inp, d in zip(layers, inps, ds):
        Y = lay.forward(d["X"])
        dX, dR, dP = lay.backward(d["X"], d["gY"])
        Yb = lay.forward_blocks(d["X"])
        dXb, dRb, dPb = lay.backward_blocks(d["X"], d["gY"])
        torch.cuda.synchronize()
        assert torch.equal(Y, Yb)
        assert torch.equal(dX, dXb) and torch.equal(dR, dRb) and torch.equal(dP, dPb)
        sigma, tau = oracle_perms(inp, 0)
        args = (inp["W0"][1], inp["thR"][1], inp["thP"][1], sigma, tau, inp["X"][1])
        contract = dtype == "bf16"
        dXr, dRr, dPr, it = oracle.backward(*args, inp["gY"][1], b, contract=contract, intermediates=True)
        fl = layer_floors(inp["W0"][1], it)
        bk, sk = ("bf16", "sum") if contract else ("f32", "f32")
        compare(from_dev(Yb), oracle.forward(*args, b, contract=contract), bk, "Y", floor=fl["Y"] if contract else None)
        compare(from_dev(dXb), dXr, bk, "dX", floor=fl["dX"] if contract else None)
        if dRr.size:
            compare(from_dev(dRb), dRr, sk, "dthR", terms=N)
        if dPr.size:
            compare(from_dev(dPb), dPr, sk, "dthP", terms=N)


def test_prebuilt_backward_accumulate_and_empty():
    torch = torch_mod()
    from orthogonal_reparameterized_poetx_amd import build_layer_blocks
    inp = WL.small_case(3, 256, 256, 64, 40, dtype="bf16")
    lay, d = make_layer(inp)
    build_layer_blocks([lay], "backward")
    _, dR, dP = lay.backward_blocks(d["X"], d["gY"])
    dR2, dP2 = dR.clone(), dP.clone()
    lay.backward_blocks(d["X"], d["gY"], dthR=dR2, dthP=dP2, want_dx=False, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(dR2, dR + dR) and torch.equal(dP2, dP + dP)
    build_layer_blocks([lay], "forward")
    lay.forward_blocks(d["X"][:0])
    _, z1, z2 = lay.backward_blocks(d["X"][:0], d["gY"][:0], dthR=dR2, dthP=dP2, want_dx=False)
    torch.cuda.synchronize()
    assert not z1.any().item() and not z2.any().item()


@pytest.mark.parametrize("dtype,m,n,b", [("bf16", 600, 520, 256), ("bf16", 1100, 700, 512), ("f32", 96, 80, 32),
                                         ("bf16", 300, 200, 64)])
def test_merge_blocks_matches_merge(dtype, m, n, b):
    torch = torch_mod()
    from orthogonal_reparameterized_poetx_amd import build_layer_blocks
    inp = WL.small_case(51, m, n, b, 4, dtype=dtype)
    a, _ = make_layer(inp)
    c, _ = make_layer(inp)
    _log("merge_blocks %s m=%d n=%d b=%d" % (dtype, m, n, b))
    a.merge()
    build_layer_blocks([c], "merge")
    c.merge_blocks()
    torch.cuda.synchronize()
    assert torch.equal(a.W0p, c.W0p)
    assert torch.equal(a.sigma, c.sigma) and torch.equal(a.tau, c.tau)
    assert not c.thR.any().item() and not c.thP.any().item()


def test_merge_sets_match_merge_blocks():
    # batched stages (bf16, rows of a multiple of 8 columns; 21 such sets, so
    # two launches per stage) beside sets merged one by one inside the call
    # (fp32, 90-column rows and INT8 weights); two merges in a row
    torch = torch_mod()
    from orthogonal_reparameterized_poetx_amd import build_layer_blocks, merge_layers_sets
    cases = [("bf16", 600, 520, 256), ("bf16", 300, 200, 64), ("f32", 96, 80, 32), ("bf16", 70, 90, 32),
             ("int8", 512, 256, 64), ("bf16", 256, 768, 128)] + [("bf16", 128, 64, 32)] * 18
    a, c = [], []
    for i, (dt, m, n, b) in enumerate(cases):
        inp = WL.small_case(60 + i, m, n, b, 4, dtype="bf16" if dt == "int8" else dt)
        a.append(make_layer(inp, w0_int8=dt == "int8")[0])
        c.append(make_layer(inp, w0_int8=dt == "int8")[0])
    _log("merge sets: %d layers" % len(cases))
    m0 = [lay.merges for lay in a]     # the packing merge made by make_layer
    for rnd in range(2):
        build_layer_blocks(a, "merge")
        for lay in a:
            lay.merge_blocks()
        build_layer_blocks(c, "merge")
        merge_layers_sets(c)
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(a, c)):
            assert torch.equal(x.W0p, y.W0p), (rnd, i, cases[i])
            assert torch.equal(x.sigma, y.sigma) and torch.equal(x.tau, y.tau), (rnd, i)
            assert not y.thR.any().item() and not y.thP.any().item(), (rnd, i)
            assert x.merges == y.merges == m0[i] + rnd + 1
        # new generators for the next round, the same on both sides
        for i, (x, y) in enumerate(zip(a, c)):
            g = torch.Generator(device="cuda").manual_seed(1000 * rnd + i)
            for tx, ty in ((x.thR, y.thR), (x.thP, y.thP)):
                v = torch.randn(tx.shape, generator=g, device="cuda") * 0.03
                tx.copy_(v)
                ty.copy_(v)


@pytest.mark.parametrize("shapes,b,N", [
    ([(600, 520), (256, 768), (512, 512)], 256, 70),
    ([(512, 1024)] * 40, 32, 20),                 # 80 sets, 1920 blocks: several chunks of the batched chain
    ([(1100, 700), (512, 1024)], 512, 24),
])
def test_deferred_chain_matches_backward_blocks(shapes, b, N):
    torch = torch_mod()
    from orthogonal_reparameterized_poetx_amd import build_layer_blocks, chain_rule_layers
    layers, ds = [], []
    for i, (m, n) in enumerate(shapes):
        inp = WL.small_case(60 + i, m, n, b, N, dtype="bf16")
        lay, d = make_layer(inp)
        layers.append(lay), ds.append(d)
    _log("deferred chain b=%d layers=%d" % (b, len(layers)))
    build_layer_blocks(layers, "backward")
    ref, grads, dxs = [], [], []
    for lay, d in zip(layers, ds):
        ref.append(lay.backward_blocks(d["X"], d["gY"]))
        dX, _, _ = lay.backward_blocks_dq(d["X"], d["gY"])
        dxs.append(dX)
        grads.append((torch.empty_like(lay.thR), torch.empty_like(lay.thP)))
    chain_rule_layers(layers, grads)
    torch.cuda.synchronize()
    for (dX0, dR0, dP0), dX, (dR, dP) in zip(ref, dxs, grads):
        assert torch.equal(dX0, dX)
        assert torch.equal(dR0, dR) and torch.equal(dP0, dP)
    # accumulation into existing gradients
    acc = [(dR.clone(), dP.clone()) for dR, dP in grads]
    chain_rule_layers(layers, acc, accumulate=True)
    torch.cuda.synchronize()
    for (dR, dP), (aR, aP) in zip(grads, acc):
        assert torch.equal(aR, dR + dR) and torch.equal(aP, dP + dP)


@pytest.mark.parametrize("m,n,b,N", [
    (256, 2048, 256, 300),     # one column tile (k and v of the layer set)
    (768, 2112, 256, 257),     # K = 33 * 64, a ragged token tile
    (2048, 5632, 256, 333),    # the down projection's K
    (5632, 2048, 256, 1000),   # 22 column tiles (gate and up)
    (1024, 2048, 64, 300),     # four blocks per column tile
    (1536, 2112, 128, 257),    # two blocks per column tile
    (2816, 4096, 128, 129),
])
def test_fused_block_products_match_separate_passes(m, n, b, N):
    """At b in {64, 128, 256} (no identity tail, K >= 2048) the forward GEMM
    applies the R-side blocks in its epilogue.  Y equals that of the same layer with
    POETX_SEPARATE_BLOCK_PRODUCTS (GEMM, then the block product) bit for
    bit, and so do the kept-z2' forward and both backward calls (which take
    the two passes either way); for the smaller shapes Y, dX and dL/dQ meet
    the oracle's bounds."""
    torch = torch_mod()
    from orthogonal_reparameterized_poetx_amd import build_layer_blocks
    inp = WL.small_case(81, m, n, b, N, dtype="bf16")
    lay, d = make_layer(inp)
    sep, _ = make_layer(inp, separate_block_products=True)
    _log("fused block products m=%d n=%d b=%d N=%d" % (m, n, b, N))
    build_layer_blocks([lay, sep], "forward")
    build_layer_blocks([lay, sep], "backward")
    outs = []
    for L_ in (lay, sep):
        lay_y = L_.forward_blocks(d["X"]).clone()
        Z2 = torch.empty((N, m), dtype=torch.bfloat16, device="cuda:0")
        Yz, _ = L_.forward_blocks_z2(d["X"], Z2=Z2)
        dX, GR, GP = (t.clone() for t in L_.backward_blocks_dq(d["X"], d["gY"]))
        dXz, GRz, GPz = (t.clone() for t in L_.backward_blocks_dq_z2(d["X"], d["gY"], Z2))
        outs.append((lay_y, Yz.clone(), Z2, dX, GR, GP, dXz, GRz, GPz))
    torch.cuda.synchronize()
    for got, sep_got in zip(*outs):
        assert torch.equal(got, sep_got)
    Y, dX, GR, GP = outs[0][0], outs[0][3], outs[0][4], outs[0][5]
    if m * n * N <= (1 << 29):
        sigma, tau = oracle_perms(inp, 0)
        W0, thR, thP, X, gY = inp["W0"][1], inp["thR"][1], inp["thP"][1], inp["X"][1], inp["gY"][1]
        dXr, _, _, it = oracle.backward(W0, thR, thP, sigma, tau, X, gY, b, contract=True, intermediates=True)
        fl = layer_floors(W0, it)
        compare(from_dev(Y), oracle.forward(W0, thR, thP, sigma, tau, X, b, contract=True), "bf16", "Y",
                floor=fl["Y"])
        compare(from_dev(dX), dXr, "bf16", "dX", floor=fl["dX"])
        compare(from_dev(GR), np.array(it["GR"]), "sum", "dL/dQ_R", terms=N)
        compare(from_dev(GP), np.array(it["GP"]), "sum", "dL/dQ_P", terms=N)


@pytest.mark.parametrize("m,n,b,N", [
    (600, 520, 256, 70),     # identity tails on both sides
    (2048, 2048, 256, 45),   # the 64-deep GEMM ring (K >= 2048)
    (1100, 700, 512, 24),
    (2048, 2048, 256, 4096),  # the square layer's shape and token count
])
def test_stored_z2_matches_recompute(m, n, b, N):
    """The variant that keeps z2' from the forward pass gives the results of
    the recomputing one bit for bit; its z2' is the oracle's Z2 in the working
    (sigma-gathered) layout, with a relative rms deviation below ETA (the
    bound the token-sum floors rest on); and its Y, dX, dL/dQ and (through
    the batched chain rule) dtheta meet the oracle bounds directly."""
    torch = torch_mod()
    from gpu_util import ETA_BF16
    from orthogonal_reparameterized_poetx_amd import build_layer_blocks, chain_rule_layers
    inp = WL.small_case(80, m, n, b, N, dtype="bf16") if N < 1000 else WL.matrix_inputs(2, 0)
    lay, d = make_layer(inp)
    _log("stored z2 m=%d n=%d b=%d N=%d" % (m, n, b, N))
    build_layer_blocks([lay], "forward")
    build_layer_blocks([lay], "backward")
    Y0 = lay.forward_blocks(d["X"])
    dX0, GR0, GP0 = (t.clone() for t in lay.backward_blocks_dq(d["X"], d["gY"]))
    Z2 = torch.full((N, m), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    Y1, _ = lay.forward_blocks_z2(d["X"], Z2=Z2)
    dX1, GR1, GP1 = lay.backward_blocks_dq_z2(d["X"], d["gY"], Z2)
    dR, dP = torch.empty_like(lay.thR), torch.empty_like(lay.thP)
    chain_rule_layers([lay], [(dR, dP)])
    torch.cuda.synchronize()
    assert torch.equal(Y0, Y1) and torch.equal(dX0, dX1)
    assert torch.equal(GR0, GR1) and torch.equal(GP0, GP1)
    sigma, tau = oracle_perms(inp, 0)
    W0, thR, thP, X, gY = inp["W0"][1], inp["thR"][1], inp["thP"][1], inp["X"][1], inp["gY"][1]
    dXr, dRr, dPr, it = oracle.backward(W0, thR, thP, sigma, tau, X, gY, b, contract=True, intermediates=True)
    fl = layer_floors(W0, it)
    # z2' = rnd(z1' W0p^T): one-ulp flips of z1' reach it through a sum over
    # n terms (Gaussian, relative rms deviation that of z1'), hence the
    # token-sum floor; nearly every element meets the stated bound
    st = compare(from_dev(Z2), it["Z2"][:, sigma], "sum", "Z2", max_strict=1e-3, terms=n)
    assert st["rel_norm"] <= ETA_BF16
    compare(from_dev(Y1), oracle.forward(W0, thR, thP, sigma, tau, X, b, contract=True), "bf16", "Y", floor=fl["Y"])
    compare(from_dev(dX1), dXr, "bf16", "dX", floor=fl["dX"])
    if it["GR"]:
        compare(from_dev(GR1), np.array(it["GR"]), "sum", "dL/dQ_R", terms=N)
        compare(from_dev(dR), dRr, "sum", "dthR", terms=N)
    if it["GP"]:
        compare(from_dev(GP1), np.array(it["GP"]), "sum", "dL/dQ_P", terms=N)
        compare(from_dev(dP), dPr, "sum", "dthP", terms=N)
    # N = 0: nothing is written, dL/dQ is zero
    lay.forward_blocks_z2(d["X"][:0], Z2=Z2[:0])
    _, GR, GP = lay.backward_blocks_dq_z2(d["X"][:0], d["gY"][:0], Z2[:0], want_dx=False)
    torch.cuda.synchronize()
    assert not GR.any().item() and not GP.any().item()
