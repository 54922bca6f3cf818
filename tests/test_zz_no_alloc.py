"""GPU test of poetx_forward_blocks_noalloc (the forward that allocates
nothing): its output equals poetx_forward_blocks' bit for bit on two calls in
a row, the second with a smaller input (the scratch array keeps the first
call's contents), for a bf16 layer whose token count needs several chunks of
the scratch, a ragged bf16 layer, an fp32 layer and an INT8 layer whose GEMMs
read the codes directly; INT8 layers that would need a dequantized copy are
rejected."""

import numpy as np
import pytest

import workloads as WL
from gpu_util import make_layer, torch_mod

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _check_pair(inp, n_small, w0_int8=False):
    torch = torch_mod()
    from orthogonal_reparameterized_poetx_amd import build_layer_blocks
    lay, d = make_layer(inp, w0_int8=w0_int8)
    build_layer_blocks([lay], "forward")
    X = d["X"]
    N = X.shape[0]
    ref = lay.forward_blocks(X)
    torch.cuda.synchronize()
    # first call: every token; second: a smaller input, into fresh outputs
    Y1 = torch.full_like(ref, float("nan"))
    lay.forward_blocks_noalloc(X, Y1)
    Xs = X[:n_small].clone()
    ref_s = lay.forward_blocks(Xs)
    Y2 = torch.full_like(ref_s, float("nan"))
    lay.forward_blocks_noalloc(Xs, Y2)
    torch.cuda.synchronize()
    _log("  N=%d then N=%d: equal %s %s" % (N, n_small, torch.equal(Y1, ref), torch.equal(Y2, ref_s)))
    assert torch.equal(Y1, ref)
    assert torch.equal(Y2, ref_s)


def test_noalloc_forward_bf16_chunked():
    # 5632 x 2048: 26.6 KiB of intermediates per token, so 8192 tokens take
    # four chunks of the 64 MiB scratch
    inp = WL.matrix_inputs(3, 4)
    _log("noalloc gate 5632x2048 N=8192")
    _check_pair(inp, 300)


def test_noalloc_forward_ragged_and_fp32():
    _log("noalloc ragged bf16 600x520 b=256")
    _check_pair(WL.small_case(71, 600, 520, 256, 333, dtype="bf16"), 70)
    _log("noalloc fp32 96x80 b=32")
    _check_pair(WL.small_case(72, 96, 80, 32, 150, dtype="f32"), 37)


def test_noalloc_forward_int8_codes():
    # n % 16 == 0 and m % 8 == 0: the GEMM reads the codes, nothing else is needed
    _log("noalloc INT8 600x528 b=128")
    _check_pair(WL.small_case(74, 600, 528, 128, 301, dtype="bf16"), 45, w0_int8=True)
    # K = 2048 both ways: poetx_forward_blocks dequantizes into its workspace
    # and runs the wide bf16 kernel, the no-allocation call reads the codes
    _log("noalloc INT8 2048x2048 b=256")
    _check_pair(WL.small_case(75, 2048, 2048, 256, 200, dtype="bf16"), 64, w0_int8=True)


def test_noalloc_rejects_int8_layers_needing_a_copy():
    torch = torch_mod()
    import orthogonal_reparameterized_poetx_amd as P
    from orthogonal_reparameterized_poetx_amd import build_layer_blocks
    # n = 520: not a multiple of 16, so every pass would dequantize into a workspace
    inp = WL.small_case(73, 256, 520, 64, 8, dtype="bf16")
    lay = P.PoetxLayer(256, 520, 64, "bf16", "cuda:0", perm_seed=inp["perm_seed"], w0_int8=True)
    build_layer_blocks([lay], "forward")
    X = torch.zeros(8, 520, dtype=torch.bfloat16, device="cuda:0")
    Y = torch.empty(8, 256, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(P.PoetxError) as e:
        lay.forward_blocks_noalloc(X, Y)
    assert e.value.code == -1 and "INT8" in str(e.value)
