"""GPU checks of the weight format with a transposed copy (POETX_W0_TRANSPOSED).

The forward product and its recompute read W0p^T [n][m] as an NN GEMM
instead of W0p [m][n] as an NT one; both sum over k in the same order on the
same MFMA, so every output of such a layer must equal, bit for bit, that of
the same layer without the flag (which the parity tests check against the
oracle).  Every merge must leave the second half equal to the transpose of
the first.
"""

import pytest

import workloads as WL
from gpu_util import make_layer, torch_mod

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("m,n,b,N", [
    (2048, 2048, 256, 300),    # NN with the R-side blocks in the epilogue
    (600, 520, 64, 70),        # identity tails, K below the wide kernel's
    (768, 2112, 128, 257),     # the fused epilogue at b = 128, ragged tokens
    (1100, 700, 512, 24),      # b = 512 (Schur builds), tails
    (5632, 2048, 256, 129),
])
def test_transposed_weight_matches_plain_layer(m, n, b, N):
    torch = torch_mod()
    from orthogonal_reparameterized_poetx_amd import build_layer_blocks, merge_layers_sets
    inp = WL.small_case(82, m, n, b, N, dtype="bf16")
    a, d = make_layer(inp)
    t, _ = make_layer(inp, w0_transposed=True)
    _log("transposed weight m=%d n=%d b=%d N=%d" % (m, n, b, N))

    def same_weights():
        torch.cuda.synchronize()
        assert torch.equal(t.weight(), a.W0p)
        assert torch.equal(t.weight_t(), a.W0p.t().contiguous())
        assert torch.equal(t.sigma, a.sigma) and torch.equal(t.tau, a.tau)

    same_weights()
    for rnd in range(3):
        # generators of the case again (a merge zeroes them)
        for L_ in (a, t):
            L_.thR.copy_(d["thR"])
            L_.thP.copy_(d["thP"])
        build_layer_blocks([a, t], "forward")
        build_layer_blocks([a, t], "backward")
        outs = []
        for L_ in (a, t):
            Y = L_.forward_blocks(d["X"]).clone()
            Yn = torch.empty(N, m, dtype=torch.bfloat16, device="cuda:0")
            L_.forward_blocks_noalloc(d["X"], Yn)
            Z2 = torch.empty(N, m, dtype=torch.bfloat16, device="cuda:0")
            Yz, _ = L_.forward_blocks_z2(d["X"], Z2=Z2)
            dX, GR, GP = (x.clone() for x in L_.backward_blocks_dq(d["X"], d["gY"]))
            Yf = L_.forward(d["X"]).clone()
            dR, dP = torch.empty_like(L_.thR), torch.empty_like(L_.thP)
            dXf, _, _ = L_.backward(d["X"], d["gY"], dthR=dR, dthP=dP)
            outs.append((Y, Yn, Yz.clone(), Z2, dX, GR, GP, Yf, dXf.clone(), dR, dP))
        torch.cuda.synchronize()
        for k, (x, y) in enumerate(zip(*outs)):
            assert torch.equal(x, y), (rnd, k)
        # merges write both halves: the single-layer call, then the batched one
        if rnd == 0:
            build_layer_blocks([a, t], "merge")
            a.merge_blocks()
            t.merge_blocks()
        elif rnd == 1:
            build_layer_blocks([a, t], "merge")
            merge_layers_sets([a])
            merge_layers_sets([t])
        same_weights()
