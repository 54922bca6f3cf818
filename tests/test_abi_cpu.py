"""C ABI checks that need no GPU: the library loads, exports every function
include/poetx.h declares, validates arguments on the host before anything is
enqueued, and its host permutation generator equals the oracle's bit for bit."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "poetx.h")


def _P():
    P = pytest.importorskip("orthogonal_reparameterized_poetx_amd")
    if not os.path.exists(P.LIB_PATH):
        pytest.skip("libpoetx.so not built")
    return P


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(poetx_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    P = _P()
    names = declared_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(P.lib(), name), name
    assert set(names) == set(P.EXPORTED)


@pytest.mark.parametrize("seed,k,side,n", [(0, 0, 0, 1), (1, 0, 1, 2), (123, 0, 0, 2048), (2 ** 64 - 1, 7, 1, 5632),
                                           ((3 << 32) | (6 << 8) | 6, 0, 0, 2048), (42, 3, 1, 11008)])
def test_host_permutation_matches_oracle(seed, k, side, n):
    P = _P()
    got = np.array(P.poetx_make_permutation(seed, k, side, n))
    assert np.array_equal(got, oracle.make_permutation(seed, k, side, n))


def _status(fn, *args):
    return fn(*args)


def test_argument_validation_on_host():
    P = _P()
    L = P.lib()
    fake = ctypes.c_void_p(0x1000)       # never dereferenced: validation fails first
    good = P.Layer(256, 256, 32, P.POETX_BF16)
    ws_need = P.workspace_bytes(good, 64, P.OP_FORWARD)
    assert ws_need > 0
    # bad block size, dtype, shape, flags, reserved
    for lay, code in [(P.Layer(256, 256, 48), -1), (P.Layer(256, 256, 32, 7), -3), (P.Layer(0, 256, 32), -2),
                      (P.Layer(256, 40000, 32), -2), (P.Layer(256, 256, 32, P.POETX_BF16, 32), -1),
                      (P.Layer(256, 256, 32, P.POETX_F32, P.POETX_W0_TRANSPOSED), -3),
                      (P.Layer(256, 256, 32, P.POETX_BF16, P.POETX_W0_TRANSPOSED | P.POETX_W0_INT8), -1)]:
        rc = L.poetx_forward(ctypes.byref(lay), fake, fake, fake, fake, fake, fake, 64, fake, fake, ws_need, None)
        assert rc == code, (rc, P.last_error())
        assert P.last_error()
        assert L.poetx_workspace_bytes(ctypes.byref(lay), 64, 0) == 0
    # the transposed weight format: W0p, then its transpose 256-byte aligned;
    # the transpose call wants the flag and a weight
    tl = P.Layer(600, 520, 64, P.POETX_BF16, P.POETX_W0_TRANSPOSED)
    assert P.w0_bytes(tl) == -(-600 * 520 * 2 // 256) * 256 + 600 * 520 * 2
    assert P.w0_bytes(P.Layer(600, 520, 64, P.POETX_BF16)) == 600 * 520 * 2
    assert L.poetx_transpose_w0(ctypes.byref(P.Layer(600, 520, 64, P.POETX_BF16)), fake, None) == -1
    assert "POETX_W0_TRANSPOSED" in P.last_error()
    assert L.poetx_transpose_w0(ctypes.byref(tl), None, None) == -1
    for op in range(7):
        assert L.poetx_workspace_bytes(ctypes.byref(tl), 64, op) == L.poetx_workspace_bytes(
            ctypes.byref(P.Layer(600, 520, 64, P.POETX_BF16)), 64, op) > 0
    # POETX_SEPARATE_BLOCK_PRODUCTS is a known flag and changes no workspace size
    sep = P.Layer(2048, 2048, 256, P.POETX_BF16, P.POETX_SEPARATE_BLOCK_PRODUCTS)
    plain = P.Layer(2048, 2048, 256, P.POETX_BF16)
    for op in range(7):
        assert L.poetx_workspace_bytes(ctypes.byref(sep), 64, op) == L.poetx_workspace_bytes(ctypes.byref(plain), 64, op) > 0
    bad = P.Layer(256, 256, 32)
    bad.reserved = 1
    assert L.poetx_forward(ctypes.byref(bad), fake, fake, fake, fake, fake, fake, 64, fake, fake, ws_need, None) == -1
    # NULL layer / tensors, negative N
    assert L.poetx_forward(None, fake, fake, fake, fake, fake, fake, 64, fake, fake, ws_need, None) == -1
    assert L.poetx_forward(ctypes.byref(good), None, fake, fake, fake, fake, fake, 64, fake, fake, ws_need, None) == -1
    assert L.poetx_forward(ctypes.byref(good), fake, fake, fake, fake, fake, fake, -1, fake, fake, ws_need, None) == -2
    # workspace too small / NULL / misaligned
    assert L.poetx_forward(ctypes.byref(good), fake, fake, fake, fake, fake, fake, 64, fake, fake, ws_need - 1, None) == -4
    assert L.poetx_forward(ctypes.byref(good), fake, fake, fake, fake, fake, fake, 64, fake, None, ws_need, None) == -4
    assert L.poetx_forward(ctypes.byref(good), fake, fake, fake, fake, fake, fake, 64, fake,
                           ctypes.c_void_p(0x1010), ws_need, None) == -4
    bneed = P.workspace_bytes(good, 64, P.OP_BACKWARD)
    assert L.poetx_backward(ctypes.byref(good), fake, fake, fake, fake, fake, fake, fake, 64, None, None, fake,
                            fake, bneed, None) == -1
    assert L.poetx_merge(ctypes.byref(good), None, fake, fake, fake, fake, 0, 0, fake, 1 << 30, None) == -1
    # builder and Adam
    assert L.poetx_build_blocks(fake, 4, 48, fake, None, None, None, 0, None) == -1
    assert L.poetx_build_blocks(fake, 0, 64, fake, None, None, None, 0, None) == 0
    assert L.poetx_build_blocks(None, 4, 64, fake, None, None, None, 0, None) == -1
    assert L.poetx_build_blocks(fake, 4, 64, None, None, None, None, 0, None) == -1
    assert L.poetx_build_blocks(fake, 4, 512, fake, None, None, None, 0, None) == -4
    assert L.poetx_adam_step(fake, fake, fake, fake, 10, 0, 1e-3, 0.9, 0.999, 1e-8, None) == -1
    assert L.poetx_adam_step(fake, fake, fake, fake, 0, 1, 1e-3, 0.9, 0.999, 1e-8, None) == 0
    assert L.poetx_make_permutation(0, 0, 2, 4, fake) == -1


def test_workspace_sizes_grow_with_tokens():
    P = _P()
    lay = P.Layer(2048, 5632, 256, P.POETX_BF16)
    f1, f2 = P.workspace_bytes(lay, 4096, P.OP_FORWARD), P.workspace_bytes(lay, 8192, P.OP_FORWARD)
    b1, b2 = P.workspace_bytes(lay, 4096, P.OP_BACKWARD), P.workspace_bytes(lay, 8192, P.OP_BACKWARD)
    assert f2 > f1 > 0 and b2 > b1 > f1
    # forward holds z1' (N x n) and z2' (N x m) in bf16
    assert f2 >= 8192 * (2048 + 5632) * 2
    # the merge works in place: besides the blocks it holds the rows the
    # relayout saves aside, at most 2 ceil(m / 16) + 1 of them, far below the
    # matrix itself
    saved = (2 * ((2048 + 15) // 16) + 1) * 5632 * 2
    blocks = (2048 // 256 + 5632 // 256) * 256 * 256 * 2
    mrg = P.workspace_bytes(lay, 0, P.OP_MERGE)
    assert saved + blocks <= mrg < saved + blocks + (1 << 20)
    assert mrg < 2048 * 5632 * 2 // 2
    assert P.workspace_bytes(lay, 0, P.OP_MERGE_BLOCKS) < 2048 * 5632 * 2 // 4
    assert P.build_workspace_bytes(29, 512) > 29 * 2 * 512 * 512 * 4
    assert P.build_workspace_bytes(29, 256) == 0


def test_prebuilt_block_entry_points_validate_on_host():
    P = _P()
    L = P.lib()
    fake = ctypes.c_void_p(0x1000)
    lay = P.Layer(512, 256, 64, P.POETX_BF16)
    fneed = P.workspace_bytes(lay, 64, P.OP_FORWARD_BLOCKS)
    bneed = P.workspace_bytes(lay, 64, P.OP_BACKWARD_BLOCKS)
    # the prebuilt-block calls need no block storage of their own
    assert 0 < fneed < P.workspace_bytes(lay, 64, P.OP_FORWARD)
    assert 0 < bneed < P.workspace_bytes(lay, 64, P.OP_BACKWARD)
    f = 0x2000
    fwd_ok = P.Blocks(None, None, f, f, None, None)          # bf16 forward reads QR, QP
    bwd_ok = P.Blocks(f, f, None, f, f, f)                   # bf16 backward: Q32R/P, QP, QTR, QTP
    # NULL blocks struct, or a block array the pass reads left NULL
    assert L.poetx_forward_blocks(ctypes.byref(lay), fake, None, fake, fake, fake, 64, fake, fake, fneed, None) == -1
    for blk in [P.Blocks(None, None, None, f, None, None), P.Blocks(f, f, f, None, f, f)]:
        assert L.poetx_forward_blocks(ctypes.byref(lay), fake, ctypes.byref(blk), fake, fake, fake, 64, fake, fake,
                                      fneed, None) == -1, P.last_error()
    for blk in [fwd_ok, P.Blocks(None, f, f, f, f, f), P.Blocks(f, f, f, f, None, f), P.Blocks(f, f, f, None, f, f)]:
        assert L.poetx_backward_blocks(ctypes.byref(lay), fake, ctypes.byref(blk), fake, fake, fake, fake, 64, fake,
                                       fake, fake, fake, bneed, None) == -1, P.last_error()
    # workspace checks apply with valid blocks
    assert L.poetx_forward_blocks(ctypes.byref(lay), fake, ctypes.byref(fwd_ok), fake, fake, fake, 64, fake, fake,
                                  fneed - 1, None) == -4
    assert L.poetx_backward_blocks(ctypes.byref(lay), fake, ctypes.byref(bwd_ok), fake, fake, fake, fake, 64, fake,
                                   fake, fake, fake, bneed - 1, None) == -4
    # fp32 layers read Q32R / Q32P in both passes
    l32 = P.Layer(512, 256, 64, P.POETX_F32)
    assert L.poetx_forward_blocks(ctypes.byref(l32), fake, ctypes.byref(fwd_ok), fake, fake, fake, 64, fake, fake,
                                  1 << 30, None) == -1
    # batched builder: count range, NULL sets, bad set, b=512 workspace
    S = P.BlockSet
    one = (S * 2)(S(0x1000, 4, 0x2000, None, None), S(0x3000, 3, None, 0x4000, None))
    assert L.poetx_build_block_sets(one, -1, 64, None, 0, None) == -2
    assert L.poetx_build_block_sets(None, 2, 64, None, 0, None) == -1
    assert L.poetx_build_block_sets(one, 2, 48, None, 0, None) == -1
    assert L.poetx_build_block_sets(one, 0, 64, None, 0, None) == 0
    bad = (S * 2)(S(0x1000, 4, 0x2000, None, None), S(0x3000, 3, None, None, None))
    assert L.poetx_build_block_sets(bad, 2, 64, None, 0, None) == -1
    bad = (S * 2)(S(0x1000, 4, 0x2000, None, None), S(None, 3, 0x2000, None, None))
    assert L.poetx_build_block_sets(bad, 2, 64, None, 0, None) == -1
    bad = (S * 2)(S(0x1000, -4, 0x2000, None, None), S(0x3000, 3, 0x2000, None, None))
    assert L.poetx_build_block_sets(bad, 2, 64, None, 0, None) == -2
    assert L.poetx_build_block_sets(one, 2, 512, None, 0, None) == -4
    # empty sets are skipped without a look at their pointers
    empty = (S * 1)(S(None, 0, None, None, None))
    assert L.poetx_build_block_sets(empty, 1, 64, None, 0, None) == 0


def test_merge_blocks_validates_on_host():
    P = _P()
    L = P.lib()
    fake = ctypes.c_void_p(0x1000)
    f = 0x2000
    lay = P.Layer(512, 256, 64, P.POETX_BF16)
    need = P.workspace_bytes(lay, 0, P.OP_MERGE_BLOCKS)
    assert 0 < need < P.workspace_bytes(lay, 0, P.OP_MERGE)
    ok = P.Blocks(None, None, f, None, None, f)          # bf16 merge reads QR and QTP
    args = lambda blk, nb: (ctypes.byref(lay), fake, blk, fake, fake, fake, fake, 1, 1, fake, nb, None)
    assert L.poetx_merge_blocks(*args(None, need)) == -1
    assert L.poetx_merge_blocks(*args(ctypes.byref(P.Blocks(None, None, f, f, f, None)), need)) == -1
    assert L.poetx_merge_blocks(*args(ctypes.byref(ok), need - 1)) == -4
    l32 = P.Layer(512, 256, 64, P.POETX_F32)
    assert L.poetx_merge_blocks(ctypes.byref(l32), fake, ctypes.byref(ok), fake, fake, fake, fake, 1, 1, fake,
                                1 << 30, None) == -1


def test_merge_sets_validate_on_host():
    P = _P()
    L = P.lib()
    from orthogonal_reparameterized_poetx_amd import _lib
    f = 0x2000
    a = P.Layer(512, 256, 64, P.POETX_BF16)
    c = P.Layer(600, 520, 256, P.POETX_BF16)
    ok = P.Blocks(None, None, f, None, None, f)
    sets = _lib.MergeSet * 2
    good = sets(_lib.MergeSet(ctypes.pointer(a), f, ctypes.pointer(ok), f, f, f, f, 1, 0),
                _lib.MergeSet(ctypes.pointer(c), f, ctypes.pointer(ok), f, f, f, f, 2, 0))
    need = L.poetx_merge_sets_workspace_bytes(good, 2)
    single = P.workspace_bytes(a, 0, P.OP_MERGE_BLOCKS) + P.workspace_bytes(c, 0, P.OP_MERGE_BLOCKS)
    assert need >= single
    assert L.poetx_merge_blocks_sets(good, 0, None, 0, None) == 0
    assert L.poetx_merge_blocks_sets(good, -1, None, 0, None) == -1
    assert L.poetx_merge_blocks_sets(None, 2, None, 0, None) == -1
    assert L.poetx_merge_blocks_sets(good, 2, ctypes.c_void_p(0x100000), need - 1, None) == -4
    # a set without its blocks, or with a bad block size, fails before any launch
    bad = sets(good[0], _lib.MergeSet(ctypes.pointer(c), f, None, f, f, f, f, 2, 0))
    assert L.poetx_merge_blocks_sets(bad, 2, ctypes.c_void_p(0x100000), need, None) == -1
    assert "merge set 1" in P.last_error()
    assert L.poetx_merge_sets_workspace_bytes(bad, 2) == 0
    wrong = P.Layer(512, 256, 48, P.POETX_BF16)
    bad2 = sets(good[0], _lib.MergeSet(ctypes.pointer(wrong), f, ctypes.pointer(ok), f, f, f, f, 2, 0))
    assert L.poetx_merge_blocks_sets(bad2, 2, ctypes.c_void_p(0x100000), need, None) == -1


def test_deferred_chain_entry_points_validate_on_host():
    P = _P()
    L = P.lib()
    fake = ctypes.c_void_p(0x1000)
    f = 0x2000
    lay = P.Layer(512, 256, 64, P.POETX_BF16)
    need = P.workspace_bytes(lay, 64, P.OP_BACKWARD_DQ)
    assert 0 < need < P.workspace_bytes(lay, 64, P.OP_BACKWARD_BLOCKS)
    blk = P.Blocks(f, f, None, f, f, f)
    args = lambda l, GR, GP, nb: (ctypes.byref(l), fake, ctypes.byref(blk), fake, fake, fake, fake, 64, fake, GR, GP,
                                  fake, nb, None)
    assert L.poetx_backward_blocks_dq(*args(lay, None, fake, need)) == -1
    assert L.poetx_backward_blocks_dq(*args(lay, fake, fake, need - 1)) == -4
    acc = P.Layer(512, 256, 64, P.POETX_BF16, P.POETX_ACCUMULATE_GRAD)
    assert L.poetx_backward_blocks_dq(*args(acc, fake, fake, need)) == -1
    l32 = P.Layer(512, 256, 64, P.POETX_F32)
    assert L.poetx_backward_blocks_dq(*args(l32, fake, fake, 1 << 30)) == -3
    S = P.ChainSet
    two = (S * 2)(S(0x1000, 0x2000, 3, 0x3000), S(0x1000, 0x2000, 5, 0x3000))
    wneed = P.chain_workspace_bytes(8, 64)
    assert wneed > 8 * 64 * 64 * 8
    assert L.poetx_chain_rule_sets(two, -1, 64, 0, None, 0, None) == -2
    assert L.poetx_chain_rule_sets(None, 2, 64, 0, None, 0, None) == -1
    assert L.poetx_chain_rule_sets(two, 2, 48, 0, None, 0, None) == -1
    assert L.poetx_chain_rule_sets(two, 2, 64, 4, fake, wneed, None) == -1
    assert L.poetx_chain_rule_sets(two, 2, 64, 0, fake, wneed - 1, None) == -4
    bad = (S * 1)(S(0x1000, None, 3, 0x3000))
    assert L.poetx_chain_rule_sets(bad, 1, 64, 0, fake, wneed, None) == -1
    assert L.poetx_chain_rule_sets((S * 1)(S(None, None, 0, None)), 1, 64, 0, None, 0, None) == 0
    assert L.poetx_chain_rule_sets(two, 0, 64, 0, None, 0, None) == 0


def test_stored_z2_entry_points_validate_on_host():
    P = _P()
    L = P.lib()
    fake = ctypes.c_void_p(0x1000)
    f = 0x2000
    lay = P.Layer(512, 256, 64, P.POETX_BF16)
    l32 = P.Layer(512, 256, 64, P.POETX_F32)
    fneed = P.workspace_bytes(lay, 64, P.OP_FORWARD_BLOCKS)
    bneed = P.workspace_bytes(lay, 64, P.OP_BACKWARD_DQ)
    fwd = P.Blocks(None, None, f, f, None, None)
    bwd = P.Blocks(f, f, None, f, f, f)
    fargs = lambda l, blk, z2, nb: (ctypes.byref(l), fake, blk, fake, fake, fake, 64, fake, z2, fake, nb, None)
    # NULL Z2, fp32 layer, NULL or incomplete blocks, short workspace
    assert L.poetx_forward_blocks_z2(*fargs(lay, ctypes.byref(fwd), None, fneed)) == -1
    assert L.poetx_forward_blocks_z2(*fargs(l32, ctypes.byref(fwd), fake, 1 << 30)) == -3
    assert L.poetx_forward_blocks_z2(*fargs(lay, None, fake, fneed)) == -1
    assert L.poetx_forward_blocks_z2(*fargs(lay, ctypes.byref(P.Blocks(None, None, None, f, None, None)), fake,
                                            fneed)) == -1
    assert L.poetx_forward_blocks_z2(*fargs(lay, ctypes.byref(fwd), fake, fneed - 1)) == -4
    bargs = lambda l, blk, z2, GR, nb: (ctypes.byref(l), fake, blk, fake, fake, fake, fake, z2, 64, fake, GR, fake,
                                        fake, nb, None)
    assert L.poetx_backward_blocks_dq_z2(*bargs(lay, ctypes.byref(bwd), None, fake, bneed)) == -1
    assert L.poetx_backward_blocks_dq_z2(*bargs(lay, ctypes.byref(bwd), fake, None, bneed)) == -1
    assert L.poetx_backward_blocks_dq_z2(*bargs(l32, ctypes.byref(bwd), fake, fake, 1 << 30)) == -3
    assert L.poetx_backward_blocks_dq_z2(*bargs(lay, ctypes.byref(fwd), fake, fake, bneed)) == -1
    assert L.poetx_backward_blocks_dq_z2(*bargs(lay, ctypes.byref(bwd), fake, fake, bneed - 1)) == -4
    acc = P.Layer(512, 256, 64, P.POETX_BF16, P.POETX_ACCUMULATE_GRAD)
    assert L.poetx_backward_blocks_dq_z2(*bargs(acc, ctypes.byref(bwd), fake, fake, bneed)) == -1


def test_int8_weight_format_validates_on_host():
    P = _P()
    L = P.lib()
    fake = ctypes.c_void_p(0x1000)
    lay = P.Layer(600, 520, 64, P.POETX_BF16, P.POETX_W0_INT8)
    # codes, then the scales at the next multiple of 256 bytes
    assert P.w0_bytes(lay) == (600 * 520 + 255) // 256 * 256 + 4 * 600
    assert P.w0_bytes(P.Layer(600, 520, 64, P.POETX_BF16)) == 600 * 520 * 2
    # the dequantized copy is part of every pass's workspace
    plain = P.Layer(600, 520, 64, P.POETX_BF16)
    for op in (P.OP_FORWARD, P.OP_BACKWARD, P.OP_FORWARD_BLOCKS, P.OP_BACKWARD_DQ, P.OP_MERGE):
        assert P.workspace_bytes(lay, 64, op) >= P.workspace_bytes(plain, 64, op) + 600 * 520 * 2
    # n % 16 == 0 and m % 8 == 0: the GEMMs read the codes, so the passes
    # need no copy (the merge still merges a dequantized weight)
    fused = P.Layer(600, 528, 64, P.POETX_BF16, P.POETX_W0_INT8)
    plain_f = P.Layer(600, 528, 64, P.POETX_BF16)
    for op in (P.OP_FORWARD, P.OP_BACKWARD, P.OP_FORWARD_BLOCKS, P.OP_BACKWARD_DQ):
        assert P.workspace_bytes(fused, 64, op) == P.workspace_bytes(plain_f, 64, op)
    assert P.workspace_bytes(fused, 0, P.OP_MERGE) >= P.workspace_bytes(plain_f, 0, P.OP_MERGE) + 600 * 528 * 2
    # K >= 2048 (a multiple of 64) in either GEMM: the dequantized copy feeds the wide bf16 kernel
    big = P.Layer(2048, 2048, 256, P.POETX_BF16, P.POETX_W0_INT8)
    big_plain = P.Layer(2048, 2048, 256, P.POETX_BF16)
    for op in (P.OP_FORWARD_BLOCKS, P.OP_BACKWARD_DQ):
        assert P.workspace_bytes(big, 64, op) == P.workspace_bytes(big_plain, 64, op) + 2048 * 2048 * 2
    # host-side rejections, before anything is enqueued: codes not 16-byte
    # aligned (fused shapes), and the no-allocation forward of a layer that
    # would need a copy
    blk = P.Blocks()
    odd = ctypes.c_void_p(0x1008)
    nb = ctypes.byref(blk)
    assert L.poetx_forward_blocks_noalloc(ctypes.byref(fused), odd, nb, fake, fake, fake, 64, fake, None) == -1
    assert "aligned" in P.last_error()
    assert L.poetx_forward_blocks_noalloc(ctypes.byref(lay), fake, nb, fake, fake, fake, 64, fake, None) == -1
    assert "INT8" in P.last_error()
    # fp32 layers cannot carry the flag; the conversions need it
    l32 = P.Layer(600, 520, 64, P.POETX_F32, P.POETX_W0_INT8)
    assert L.poetx_w0_bytes(ctypes.byref(l32)) == 0
    assert L.poetx_quantize_w0(ctypes.byref(l32), fake, fake, None) == -3
    assert L.poetx_quantize_w0(ctypes.byref(plain), fake, fake, None) == -1
    assert L.poetx_dequantize_w0(ctypes.byref(plain), fake, fake, None) == -1
    assert L.poetx_quantize_w0(ctypes.byref(lay), None, fake, None) == -1
    assert L.poetx_dequantize_w0(ctypes.byref(lay), fake, None, None) == -1


def test_cnp_builder_validates_on_host():
    P = _P()
    L = P.lib()
    S = P.BlockSet
    one = (S * 1)(S(0x1000, 4, 0x2000, None, None))
    need = P.build_cnp_workspace_bytes(4, 64)
    assert need > 3 * 4 * 64 * 64 * 4
    fake = ctypes.c_void_p(0x100000)
    assert L.poetx_build_cnp_workspace_bytes(4, 512) == 0          # b = 512 has no series path
    assert L.poetx_build_block_sets_cnp(one, 1, 512, 4, fake, 1 << 30, None) == -1
    assert L.poetx_build_block_sets_cnp(one, 1, 64, 0, fake, need, None) == -1
    assert L.poetx_build_block_sets_cnp(one, 1, 64, 17, fake, need, None) == -1
    assert L.poetx_build_block_sets_cnp(one, -1, 64, 4, fake, need, None) == -2
    assert L.poetx_build_block_sets_cnp(None, 1, 64, 4, fake, need, None) == -1
    assert L.poetx_build_block_sets_cnp(one, 1, 64, 4, fake, need - 1, None) == -4
    assert L.poetx_build_block_sets_cnp(one, 1, 64, 4, None, 0, None) == -4
    big = (S * 2)(S(0x1000, 40000, 0x2000, None, None), S(0x1000, 40000, 0x2000, None, None))
    assert L.poetx_build_block_sets_cnp(big, 2, 64, 4, fake, 1 << 40, None) == -2
    assert L.poetx_build_block_sets_cnp((S * 1)(S(0x1000, 70000, 0x2000, None, None)), 1, 64, 4, fake, 1 << 40,
                                        None) == -2
    assert L.poetx_build_block_sets_cnp((S * 1)(S(None, 0, None, None, None)), 1, 64, 4, None, 0, None) == 0


def test_stream_handle_normalization():
    """Every wrapper takes a torch.cuda.Stream-like object (its cuda_stream
    handle), a raw handle as an int, or None (torch's current stream)."""
    P = _P()
    from orthogonal_reparameterized_poetx_amd import _lib

    class FakeStream:
        cuda_stream = 0x1234

    assert _lib.stream_handle(FakeStream()) == 0x1234
    assert _lib.stream_handle(0x5678) == 0x5678
    assert _lib._stream(FakeStream()).value == 0x1234


def test_permuted_input_validates_on_host():
    P = _P()
    L = P.lib()
    fake = ctypes.c_void_p(0x1000)
    lay = P.Layer(512, 256, 64, P.POETX_BF16)
    l32 = P.Layer(512, 256, 64, P.POETX_F32)
    # the gather: NULL arguments, fp32 layers, N out of range; N = 0 enqueues nothing
    assert L.poetx_permute_input(ctypes.byref(lay), None, fake, 64, fake, None) == -1
    assert L.poetx_permute_input(ctypes.byref(lay), fake, None, 64, fake, None) == -1
    assert L.poetx_permute_input(ctypes.byref(lay), fake, fake, 64, None, None) == -1
    assert L.poetx_permute_input(ctypes.byref(l32), fake, fake, 64, fake, None) == -3
    assert L.poetx_permute_input(ctypes.byref(lay), fake, fake, -1, fake, None) == -2
    assert L.poetx_permute_input(ctypes.byref(lay), None, None, 0, None, None) == 0
    # the flag: bf16 layers only; workspaces as without it
    x32 = P.Layer(512, 256, 64, P.POETX_F32, P.POETX_X_PERMUTED)
    assert L.poetx_workspace_bytes(ctypes.byref(x32), 64, P.OP_FORWARD) == 0
    assert "POETX_X_PERMUTED" in P.last_error()
    xp = P.Layer(512, 256, 64, P.POETX_BF16, P.POETX_X_PERMUTED)
    for op in (P.OP_FORWARD, P.OP_BACKWARD, P.OP_FORWARD_BLOCKS, P.OP_BACKWARD_DQ):
        assert P.workspace_bytes(xp, 64, op) == P.workspace_bytes(lay, 64, op)
    assert P.POETX_X_PERMUTED == 16
