"""GPU checks of layers that take the input already gathered (POETX_X_PERMUTED).

poetx_permute_input must produce x' = X[:, tau] exactly (an index operation).
Given x', every forward and backward call of such a layer runs the same
kernels on the same operands as the layer without the flag, less its own
gather, so every output must equal that layer's bit for bit (the parity tests
check that layer against the oracle; one case here checks the flagged layer
against the oracle directly).
"""

import numpy as np
import pytest

import oracle
import workloads as WL
from gpu_util import compare, from_dev, layer_floors, make_layer, oracle_perms, torch_mod

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _outputs(lay, X, gY, N, m):
    torch = torch_mod()
    Y = lay.forward_blocks(X).clone()
    Yn = torch.empty(N, m, dtype=torch.bfloat16, device="cuda:0")
    lay.forward_blocks_noalloc(X, Yn)
    Z2 = torch.empty(N, m, dtype=torch.bfloat16, device="cuda:0")
    Yz, _ = lay.forward_blocks_z2(X, Z2=Z2)
    Yz = Yz.clone()
    dXz, GRz, GPz = (x.clone() for x in lay.backward_blocks_dq_z2(X, gY, Z2))
    dX, GR, GP = (x.clone() for x in lay.backward_blocks_dq(X, gY))
    Yf = lay.forward(X).clone()
    dR, dP = torch.empty_like(lay.thR), torch.empty_like(lay.thP)
    dXf, _, _ = lay.backward(X, gY, dthR=dR, dthP=dP)
    dXb, dRb, dPb = (x.clone() for x in lay.backward_blocks(X, gY))
    return (Y, Yn, Yz, Z2, dXz, GRz, GPz, dX, GR, GP, Yf, dXf.clone(), dR, dP, dXb, dRb, dPb)


@pytest.mark.parametrize("m,n,b,N,kw", [
    (2048, 2048, 256, 300, {"w0_transposed": True}),   # 8 blocks a row: gather and block product as two passes
    (600, 520, 256, 70, {}),                          # identity tails on both sides
    (512, 768, 256, 33, {}),                          # 3 blocks a row: the fused gather without the flag
    (300, 200, 64, 50, {}),                           # b = 64, tails
    (1100, 700, 512, 24, {}),                         # b = 512, tails
    (2048, 2048, 256, 45, {"w0_int8": True}),         # INT8 base weights
    (5632, 2048, 256, 129, {"w0_transposed": True}),
])
def test_permuted_input_matches_plain_layer(m, n, b, N, kw):
    torch = torch_mod()
    from orthogonal_reparameterized_poetx_amd import build_layer_blocks
    inp = WL.small_case(91, m, n, b, N, dtype="bf16")
    a, d = make_layer(inp, **kw)
    p, _ = make_layer(inp, x_permuted=True, **kw)
    _log("permuted input m=%d n=%d b=%d N=%d %s" % (m, n, b, N, kw))
    Xp = p.permute_input(d["X"])
    torch.cuda.synchronize()
    assert torch.equal(Xp, d["X"][:, p.tau.long()])
    # a layer without the flag gathers the same way
    assert torch.equal(a.permute_input(d["X"]), Xp)
    build_layer_blocks([a, p], "forward")
    build_layer_blocks([a, p], "backward")
    ra = _outputs(a, d["X"], d["gY"], N, m)
    rp = _outputs(p, Xp, d["gY"], N, m)
    torch.cuda.synchronize()
    for k, (x, y) in enumerate(zip(ra, rp)):
        assert torch.equal(x, y), k


def test_permuted_input_against_oracle():
    torch = torch_mod()
    inp = WL.small_case(92, 600, 520, 256, 70, dtype="bf16")
    p, d = make_layer(inp, x_permuted=True)
    sigma, tau = oracle_perms(inp, 0)
    W0, thR, thP, X, gY = inp["W0"][1], inp["thR"][1], inp["thP"][1], inp["X"][1], inp["gY"][1]
    Xp = p.permute_input(d["X"])
    Y = p.forward(Xp)
    dX, dR, dP = p.backward(Xp, d["gY"])
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(Xp), X[:, tau])
    Yr = oracle.forward(W0, thR, thP, sigma, tau, X, 256, contract=True)
    dXr, dRr, dPr, it = oracle.backward(W0, thR, thP, sigma, tau, X, gY, 256, contract=True, intermediates=True)
    fl = layer_floors(W0, it)
    compare(from_dev(Y), Yr, "bf16", "Y", floor=fl["Y"])
    compare(from_dev(dX), dXr, "bf16", "dX", floor=fl["dX"])
    compare(from_dev(dR), dRr, "sum", "dthR", terms=70)
    compare(from_dev(dP), dPr, "sum", "dthP", terms=70)
