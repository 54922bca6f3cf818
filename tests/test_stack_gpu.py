"""GPU parity on the 24-layer stack of layer-set shapes (168 matrices,
8192 tokens): one training step -- forward and backward of every matrix with
blocks rebuilt per pass, one Adam step over all generators, then the global
merge with re-permutation.  Two matrices (layer 0 q, layer 23 down) take the
shared seeded recipe and are checked against the float64 oracle at every
stage; every matrix is checked for the reset and the new permutations."""

import numpy as np
import pytest

import bench
import oracle
import workloads as WL
from gpu_util import compare, from_dev, oracle_perms, torch_mod

pytestmark = pytest.mark.gpu

EXACT = (0, 167)


def test_stack_training_step():
    torch = torch_mod()
    import orthogonal_reparameterized_poetx_amd as P
    print("stack: building 24 layers", flush=True)
    st = bench.Stack(P, WL, torch, "cuda:0", WL.CONFIGS[5]["N"], exact=EXACT)
    torch.cuda.synchronize()
    print("stack: fwd+bwd", flush=True)
    st.forward_backward()
    st.adam()
    torch.cuda.synchronize()
    snap = {}
    for lay, o in zip(st.layers, st.out):
        if lay.j in EXACT:
            snap[lay.j] = dict(Y=from_dev(o["Y"]), dX=from_dev(o["dX"]), dR=from_dev(lay.dR), dP=from_dev(lay.dP),
                               tR=from_dev(lay.thR), tP=from_dev(lay.thP))
    m1, v1 = st.m1.clone(), st.v1.clone()
    print("stack: merge", flush=True)
    st.merge()
    torch.cuda.synchronize()
    assert not st.theta.any().item()
    for lay in st.layers:
        assert lay.merges == 2
    for lay in st.layers:
        if lay.j not in EXACT:
            continue
        j, s = lay.j, snap[lay.j]
        print("stack: oracle for matrix %d" % j, flush=True)
        inp = WL.matrix_inputs(5, j)
        b = inp["b"]
        sigma, tau = oracle_perms(inp, 0)
        W0, th0R, th0P, X, gY = inp["W0"][1], inp["thR"][1], inp["thP"][1], inp["X"][1], inp["gY"][1]
        compare(s["Y"], oracle.forward(W0, th0R, th0P, sigma, tau, X, b, contract=True), "bf16", "Y")
        dXr, dRr, dPr = oracle.backward(W0, th0R, th0P, sigma, tau, X, gY, b, contract=True)
        compare(s["dX"], dXr, "bf16", "dX")
        compare(s["dR"], dRr, "bf16", "dthR")
        compare(s["dP"], dPr, "bf16", "dthP")
        # Adam from zero moments on the GPU's own gradients (the gradients are checked above)
        hp = {k: float(np.float32(v)) for k, v in dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8).items()}
        tR = oracle.adam_step(th0R, s["dR"], 0.0, 0.0, 1, **hp)[0]
        tP = oracle.adam_step(th0P, s["dP"], 0.0, 0.0, 1, **hp)[0]
        compare(s["tR"], tR, "f32", "theta_R after Adam")
        compare(s["tP"], tP, "f32", "theta_P after Adam")
        # merge with the post-Adam generators, relaid to the merge-1 permutations
        s1, t1 = oracle_perms(inp, 1)
        assert np.array_equal(from_dev(lay.sigma), s1) and np.array_equal(from_dev(lay.tau), t1)
        Wn = oracle.merge(W0, s["tR"], s["tP"], sigma, tau, b, contract=True)
        compare(from_dev(lay.W0p), oracle.pack(Wn, s1, t1), "bf16", "W0p merged")
    assert torch.isfinite(m1).all().item() and torch.isfinite(v1).all().item()
