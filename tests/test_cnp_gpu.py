"""GPU parity of the truncated-series (CNP) Cayley builder.

poetx_build_block_sets_cnp takes, per block, I + 2 (S + ... + S^terms) where
the dropped tail is provably below 2^-22 in spectral norm, and the exact solve
elsewhere.  Series blocks are checked against oracle.cayley_neumann (fp32
bound) and the exact oracle.cayley (the tail bound plus fp32 rounding); the
other blocks must equal poetx_build_block_sets bit for bit.  Which form a
block takes is fixed by the oracle's bound: the test scales stay far from the
threshold.
"""

import numpy as np
import pytest

import oracle
from gpu_util import compare, from_dev, to_dev, torch_mod

pytestmark = pytest.mark.gpu
TOL = 2.0 ** -22


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("b,terms", [(32, 3), (64, 4), (128, 6), (256, 8)])
def test_cnp_builder(b, terms):
    torch = torch_mod()
    import orthogonal_reparameterized_poetx_amd as P
    rng = np.random.default_rng(300 + b)
    nt = b * (b - 1) // 2
    # per block scale: zero, tiny (series), large (exact solve), mixed in one set
    scales = [[0.0, 1e-6, 0.05, 2e-6], [0.02, 1e-7], [3e-7, 3e-7, 0.1]]
    sets, ref_sets, thetas = [], [], []
    for sc in scales:
        th = rng.standard_normal((len(sc), nt)) * np.array(sc)[:, None]
        th32 = th.astype(np.float32)
        thetas.append(th32.astype(np.float64))
        dth = to_dev(th32, "f32")
        nb = len(sc)
        mk = lambda: (torch.full((nb, b, b), np.nan, dtype=torch.float32, device="cuda:0"),
                      torch.zeros(nb, b, b, dtype=torch.bfloat16, device="cuda:0"),
                      torch.zeros(nb, b, b, dtype=torch.bfloat16, device="cuda:0"))
        sets.append((dth, nb) + mk())
        ref_sets.append((dth, nb) + mk())
    total = sum(len(sc) for sc in scales)
    ws = P.make_workspace(P.build_cnp_workspace_bytes(total, b), "cuda:0")
    P.poetx_build_block_sets_cnp(sets, b, terms, ws)
    P.poetx_build_block_sets(ref_sets, b, P.make_workspace(P.build_workspace_bytes(4, b), "cuda:0"))
    torch.cuda.synchronize()
    nseries = 0
    for (_, nb, q32, qb, qt), (_, _, r32, rb, rt), th in zip(sets, ref_sets, thetas):
        for l in range(nb):
            S = oracle.unpack_skew(th[l], b)
            bound = oracle.cnp_error_bound(S, terms)
            got = from_dev(q32[l])
            if bound <= TOL * 0.5:
                nseries += 1
                st = compare(got, oracle.cayley_neumann(S, terms), "f32", "Q_series")
                err = np.abs(got - oracle.cayley(S)).max()
                assert err <= bound + 4e-7, (err, bound)
                assert torch.equal(qb[l], q32[l].to(torch.bfloat16))
                assert torch.equal(qt[l], qb[l].t().contiguous())
                _log("  b=%d block %d series: bound %.2e, |Q - cayley| %.2e, tol ratio %.3g"
                     % (b, l, bound, err, st["max_ratio"]))
            else:
                assert bound > TOL * 2, "test scale too close to the threshold"
                assert torch.equal(q32[l], r32[l]) and torch.equal(qb[l], rb[l]) and torch.equal(qt[l], rt[l])
    assert nseries == 6   # the zero and tiny blocks


def test_cnp_zero_generators_give_identity():
    torch = torch_mod()
    import orthogonal_reparameterized_poetx_amd as P
    b, nb = 256, 3
    th = torch.zeros(nb, b * (b - 1) // 2, dtype=torch.float32, device="cuda:0")
    q32 = torch.full((nb, b, b), np.nan, dtype=torch.float32, device="cuda:0")
    ws = P.make_workspace(P.build_cnp_workspace_bytes(nb, b), "cuda:0")
    P.poetx_build_block_sets_cnp([(th, nb, q32, None, None)], b, 1, ws)
    torch.cuda.synchronize()
    assert torch.equal(q32, torch.eye(b, device="cuda:0").expand(nb, b, b))
