"""GPU parity of the generator optimizer step (poetx_adam_step) against the
float64 oracle: three consecutive steps on seeded generators, gradients and
moments (fp32 bound |d| <= 1e-5 * max(|ref|, rms(ref))), the oracle carrying
its own state, stored in fp32, from step to step."""

import numpy as np
import pytest

import oracle
from gpu_util import compare, from_dev, to_dev, torch_mod

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("count", [1, 1000, 1 << 20])
def test_adam_three_steps(count):
    torch = torch_mod()
    import orthogonal_reparameterized_poetx_amd as P
    rng = np.random.default_rng([31, count])
    th = (rng.standard_normal(count) * 0.03).astype(np.float32)
    th_d = to_dev(th, "f32")
    m_d = torch.zeros(count, dtype=torch.float32, device="cuda:0")
    v_d = torch.zeros_like(m_d)
    ref_t, ref_m, ref_v = th.astype(np.float64), np.zeros(count), np.zeros(count)
    # the C ABI takes the hyperparameters as fp32: the oracle gets the values
    # the device receives (1 - fl32(0.999) differs from 1e-3 by 1.3e-5 relative)
    hp = {k: float(np.float32(v)) for k, v in dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8).items()}
    for step in (1, 2, 3):
        g = (rng.standard_normal(count) * 10.0 ** rng.uniform(-6, 0, count)).astype(np.float32)
        g[: min(count, 3)] = 0.0       # zero gradients leave the moments decaying, the update finite
        P.poetx_adam_step(th_d, to_dev(g, "f32"), m_d, v_d, count, step, **hp)
        torch.cuda.synchronize()
        ref_t, ref_m, ref_v = oracle.adam_step(ref_t, g.astype(np.float64), ref_m, ref_v, step, **hp)
        compare(from_dev(m_d), ref_m, "f32", "m")
        compare(from_dev(v_d), ref_v, "f32", "v")
        compare(from_dev(th_d), ref_t, "f32", "theta")
        # the state is stored in fp32 between steps: the oracle carries its
        # own values rounded to fp32 (round to nearest even) into the next step
        ref_t, ref_m, ref_v = (np.asarray(a, dtype=np.float32).astype(np.float64) for a in (ref_t, ref_m, ref_v))
