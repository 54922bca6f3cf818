"""ctypes binding of libpoetx.so (include/poetx.h).

Argument marshalling only: every step of the hot path runs in the library's
HIP kernels.  Tensors are torch tensors on a ROCm device; their data pointers
and the current HIP stream are passed through unchanged.  There is no fallback:
if the library is missing or a call fails, an exception is raised.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpoetx.so")

POETX_F32 = 0
POETX_BF16 = 1
POETX_ACCUMULATE_GRAD = 1
POETX_W0_INT8 = 2
POETX_SEPARATE_BLOCK_PRODUCTS = 4
POETX_W0_TRANSPOSED = 8
POETX_X_PERMUTED = 16
OP_FORWARD, OP_BACKWARD, OP_MERGE, OP_FORWARD_BLOCKS, OP_BACKWARD_BLOCKS, OP_MERGE_BLOCKS, OP_BACKWARD_DQ = range(7)

_STATUS = {0: "POETX_OK", -1: "POETX_EINVAL", -2: "POETX_ESHAPE", -3: "POETX_EDTYPE",
           -4: "POETX_EWORKSPACE", -5: "POETX_EHIP"}

EXPORTED = ("poetx_workspace_bytes", "poetx_build_workspace_bytes", "poetx_build_blocks",
            "poetx_build_block_sets", "poetx_build_cnp_workspace_bytes", "poetx_build_block_sets_cnp",
            "poetx_forward", "poetx_forward_blocks", "poetx_forward_blocks_noalloc", "poetx_permute_input",
            "poetx_backward",
            "poetx_backward_blocks", "poetx_backward_blocks_dq", "poetx_forward_blocks_z2",
            "poetx_backward_blocks_dq_z2", "poetx_chain_rule_sets",
            "poetx_chain_workspace_bytes", "poetx_merge", "poetx_merge_blocks", "poetx_merge_blocks_sets",
            "poetx_merge_sets_workspace_bytes", "poetx_make_permutation",
            "poetx_adam_step", "poetx_w0_bytes", "poetx_quantize_w0", "poetx_dequantize_w0", "poetx_transpose_w0",
            "poetx_last_error", "poetx_timing_enable", "poetx_timing_summary")


class Layer(ctypes.Structure):
    """poetx_layer: W0 is m x n (out x in), block size b, dtype of W0/X/Y."""
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("b", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]

    def __init__(self, m, n, b, dtype=POETX_BF16, flags=0):
        super().__init__(int(m), int(n), int(b), int(dtype), int(flags), 0)

    @property
    def kR(self):
        return self.m // self.b

    @property
    def kP(self):
        return self.n // self.b

    @property
    def ntheta(self):
        return self.b * (self.b - 1) // 2


class BlockSet(ctypes.Structure):
    """poetx_block_set: one batch of generators and where its Q goes."""
    _fields_ = [("theta", ctypes.c_void_p), ("nblocks", ctypes.c_int64), ("Q32", ctypes.c_void_p),
                ("Qbf16", ctypes.c_void_p), ("QTbf16", ctypes.c_void_p)]


class Blocks(ctypes.Structure):
    """poetx_blocks: prebuilt Cayley blocks of one layer."""
    _fields_ = [("Q32R", ctypes.c_void_p), ("Q32P", ctypes.c_void_p), ("QR", ctypes.c_void_p),
                ("QP", ctypes.c_void_p), ("QTR", ctypes.c_void_p), ("QTP", ctypes.c_void_p)]


def _addr(t):
    return None if t is None else t.data_ptr()


def make_blocks(Q32R=None, Q32P=None, QR=None, QP=None, QTR=None, QTP=None):
    return Blocks(_addr(Q32R), _addr(Q32P), _addr(QR), _addr(QP), _addr(QTR), _addr(QTP))


class ChainSet(ctypes.Structure):
    """poetx_chain_set: blocks, their dL/dQ and the generator gradient."""
    _fields_ = [("Q32", ctypes.c_void_p), ("G", ctypes.c_void_p), ("nblocks", ctypes.c_int64),
                ("dtheta", ctypes.c_void_p)]


class MergeSet(ctypes.Structure):
    """poetx_merge_set: one layer's arguments of poetx_merge_blocks."""
    _fields_ = [("layer", ctypes.POINTER(Layer)), ("W0p", ctypes.c_void_p), ("blocks", ctypes.POINTER(Blocks)),
                ("thR", ctypes.c_void_p), ("thP", ctypes.c_void_p), ("sigma", ctypes.c_void_p),
                ("tau", ctypes.c_void_p), ("perm_seed", ctypes.c_uint64), ("merge_index", ctypes.c_uint64)]


class PoetxError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__("%s failed: %s (%d): %s" % (fn, _STATUS.get(code, "?"), code, msg))
        self.code = code


_lib = None


def lib():
    """Load libpoetx.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libpoetx.so not found at %s; build it with __graft_entry__.build()" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, u64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
    LP = ctypes.POINTER(Layer)
    BP = ctypes.POINTER(Blocks)
    sig = {
        "poetx_workspace_bytes": (sz, [LP, i64, ctypes.c_int]),
        "poetx_build_workspace_bytes": (sz, [i64, i32]),
        "poetx_build_blocks": (ctypes.c_int, [vp, i64, i32, vp, vp, vp, vp, sz, vp]),
        "poetx_build_block_sets": (ctypes.c_int, [ctypes.POINTER(BlockSet), i32, i32, vp, sz, vp]),
        "poetx_build_cnp_workspace_bytes": (sz, [i64, i32]),
        "poetx_build_block_sets_cnp": (ctypes.c_int, [ctypes.POINTER(BlockSet), i32, i32, i32, vp, sz, vp]),
        "poetx_forward": (ctypes.c_int, [LP, vp, vp, vp, vp, vp, vp, i64, vp, vp, sz, vp]),
        "poetx_forward_blocks": (ctypes.c_int, [LP, vp, BP, vp, vp, vp, i64, vp, vp, sz, vp]),
        "poetx_forward_blocks_noalloc": (ctypes.c_int, [LP, vp, BP, vp, vp, vp, i64, vp, vp]),
        "poetx_permute_input": (ctypes.c_int, [LP, vp, vp, i64, vp, vp]),
        "poetx_backward": (ctypes.c_int, [LP, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp]),
        "poetx_backward_blocks": (ctypes.c_int, [LP, vp, BP, vp, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp]),
        "poetx_backward_blocks_dq": (ctypes.c_int, [LP, vp, BP, vp, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp]),
        "poetx_forward_blocks_z2": (ctypes.c_int, [LP, vp, BP, vp, vp, vp, i64, vp, vp, vp, sz, vp]),
        "poetx_backward_blocks_dq_z2": (ctypes.c_int, [LP, vp, BP, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, sz,
                                                        vp]),
        "poetx_chain_rule_sets": (ctypes.c_int, [ctypes.POINTER(ChainSet), i32, i32, ctypes.c_uint32, vp, sz, vp]),
        "poetx_chain_workspace_bytes": (sz, [i64, i32]),
        "poetx_merge": (ctypes.c_int, [LP, vp, vp, vp, vp, vp, u64, u64, vp, sz, vp]),
        "poetx_merge_blocks": (ctypes.c_int, [LP, vp, BP, vp, vp, vp, vp, u64, u64, vp, sz, vp]),
        "poetx_merge_blocks_sets": (ctypes.c_int, [ctypes.POINTER(MergeSet), i32, vp, sz, vp]),
        "poetx_merge_sets_workspace_bytes": (sz, [ctypes.POINTER(MergeSet), i32]),
        "poetx_make_permutation": (ctypes.c_int, [u64, u64, i32, i64, vp]),
        "poetx_adam_step": (ctypes.c_int, [vp, vp, vp, vp, i64, i64, ctypes.c_float, ctypes.c_float,
                                           ctypes.c_float, ctypes.c_float, vp]),
        "poetx_w0_bytes": (sz, [LP]),
        "poetx_quantize_w0": (ctypes.c_int, [LP, vp, vp, vp]),
        "poetx_dequantize_w0": (ctypes.c_int, [LP, vp, vp, vp]),
        "poetx_transpose_w0": (ctypes.c_int, [LP, vp, vp]),
        "poetx_last_error": (ctypes.c_char_p, []),
        "poetx_timing_enable": (ctypes.c_int, [ctypes.c_int]),
        "poetx_timing_summary": (ctypes.c_int, [ctypes.c_char_p, sz]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def last_error():
    return lib().poetx_last_error().decode()


def _check(fn, code):
    if code != 0:
        raise PoetxError(fn, code, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def stream_handle(stream):
    """The raw hipStream_t (an int) of a torch.cuda.Stream, a raw handle
    given as an int, or None (torch's current stream)."""
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if hasattr(stream, "cuda_stream"):
        return int(stream.cuda_stream)
    return int(stream)


def _stream(stream):
    return ctypes.c_void_p(stream_handle(stream))


def workspace_bytes(layer, N, op):
    n = lib().poetx_workspace_bytes(ctypes.byref(layer), int(N), int(op))
    if n == 0:
        msg = last_error()
        if msg:
            raise PoetxError("poetx_workspace_bytes", -1, msg)
    return n


def build_workspace_bytes(nblocks, b):
    return lib().poetx_build_workspace_bytes(int(nblocks), int(b))


def w0_bytes(layer):
    n = lib().poetx_w0_bytes(ctypes.byref(layer))
    if n == 0:
        raise PoetxError("poetx_w0_bytes", -1, last_error())
    return n


def poetx_quantize_w0(layer, W0bf16, W0q, stream=None):
    _check("poetx_quantize_w0", lib().poetx_quantize_w0(ctypes.byref(layer), _ptr(W0bf16), _ptr(W0q),
                                                        _stream(stream)))


def poetx_dequantize_w0(layer, W0q, W0bf16, stream=None):
    _check("poetx_dequantize_w0", lib().poetx_dequantize_w0(ctypes.byref(layer), _ptr(W0q), _ptr(W0bf16),
                                                            _stream(stream)))


def poetx_transpose_w0(layer, W0p, stream=None):
    _check("poetx_transpose_w0", lib().poetx_transpose_w0(ctypes.byref(layer), _ptr(W0p), _stream(stream)))


def make_workspace(nbytes, device):
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def poetx_build_blocks(theta, nblocks, b, Q32=None, Qbf16=None, QTbf16=None, ws=None, stream=None):
    nb = ws.numel() if ws is not None else 0
    _check("poetx_build_blocks", lib().poetx_build_blocks(_ptr(theta), int(nblocks), int(b), _ptr(Q32), _ptr(Qbf16),
                                                          _ptr(QTbf16), _ptr(ws), nb, _stream(stream)))


def poetx_build_block_sets(sets, b, ws=None, stream=None):
    """sets: sequence of (theta, nblocks, Q32, Qbf16, QTbf16) with tensors or None."""
    arr = (BlockSet * max(len(sets), 1))()
    for i, (th, nb, q32, qbf, qt) in enumerate(sets):
        arr[i] = BlockSet(_addr(th), int(nb), _addr(q32), _addr(qbf), _addr(qt))
    nbytes = ws.numel() if ws is not None else 0
    _check("poetx_build_block_sets", lib().poetx_build_block_sets(arr, len(sets), int(b), _ptr(ws), nbytes,
                                                                  _stream(stream)))


def build_cnp_workspace_bytes(total_blocks, b):
    n = lib().poetx_build_cnp_workspace_bytes(int(total_blocks), int(b))
    if n == 0:
        raise PoetxError("poetx_build_cnp_workspace_bytes", -1, last_error())
    return n


def poetx_build_block_sets_cnp(sets, b, terms, ws=None, stream=None):
    """poetx_build_block_sets with the truncated Cayley series where its bound allows."""
    arr = (BlockSet * max(len(sets), 1))()
    for i, (th, nb, q32, qbf, qt) in enumerate(sets):
        arr[i] = BlockSet(_addr(th), int(nb), _addr(q32), _addr(qbf), _addr(qt))
    nbytes = ws.numel() if ws is not None else 0
    _check("poetx_build_block_sets_cnp", lib().poetx_build_block_sets_cnp(arr, len(sets), int(b), int(terms),
                                                                          _ptr(ws), nbytes, _stream(stream)))


def poetx_forward_blocks(layer, W0p, blocks, sigma, tau, X, N, Y, ws, stream=None):
    _check("poetx_forward_blocks", lib().poetx_forward_blocks(
        ctypes.byref(layer), _ptr(W0p), None if blocks is None else ctypes.byref(blocks), _ptr(sigma), _ptr(tau),
        _ptr(X), int(N), _ptr(Y), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))


def poetx_forward_blocks_noalloc(layer, W0p, blocks, sigma, tau, X, N, Y, stream=None):
    _check("poetx_forward_blocks_noalloc", lib().poetx_forward_blocks_noalloc(
        ctypes.byref(layer), _ptr(W0p), None if blocks is None else ctypes.byref(blocks), _ptr(sigma), _ptr(tau),
        _ptr(X), int(N), _ptr(Y), _stream(stream)))


def poetx_permute_input(layer, tau, X, N, Xp, stream=None):
    _check("poetx_permute_input", lib().poetx_permute_input(ctypes.byref(layer), _ptr(tau), _ptr(X), int(N), _ptr(Xp),
                                                            _stream(stream)))


def poetx_backward_blocks(layer, W0p, blocks, sigma, tau, X, dY, N, dX, dthR, dthP, ws, stream=None):
    _check("poetx_backward_blocks", lib().poetx_backward_blocks(
        ctypes.byref(layer), _ptr(W0p), None if blocks is None else ctypes.byref(blocks), _ptr(sigma), _ptr(tau),
        _ptr(X), _ptr(dY), int(N), _ptr(dX), _ptr(dthR), _ptr(dthP), _ptr(ws), ws.numel() if ws is not None else 0,
        _stream(stream)))


def poetx_backward_blocks_dq(layer, W0p, blocks, sigma, tau, X, dY, N, dX, GR, GP, ws, stream=None):
    _check("poetx_backward_blocks_dq", lib().poetx_backward_blocks_dq(
        ctypes.byref(layer), _ptr(W0p), None if blocks is None else ctypes.byref(blocks), _ptr(sigma), _ptr(tau),
        _ptr(X), _ptr(dY), int(N), _ptr(dX), _ptr(GR), _ptr(GP), _ptr(ws), ws.numel() if ws is not None else 0,
        _stream(stream)))


def poetx_forward_blocks_z2(layer, W0p, blocks, sigma, tau, X, N, Y, Z2, ws, stream=None):
    _check("poetx_forward_blocks_z2", lib().poetx_forward_blocks_z2(
        ctypes.byref(layer), _ptr(W0p), None if blocks is None else ctypes.byref(blocks), _ptr(sigma), _ptr(tau),
        _ptr(X), int(N), _ptr(Y), _ptr(Z2), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))


def poetx_backward_blocks_dq_z2(layer, W0p, blocks, sigma, tau, X, dY, Z2, N, dX, GR, GP, ws, stream=None):
    _check("poetx_backward_blocks_dq_z2", lib().poetx_backward_blocks_dq_z2(
        ctypes.byref(layer), _ptr(W0p), None if blocks is None else ctypes.byref(blocks), _ptr(sigma), _ptr(tau),
        _ptr(X), _ptr(dY), _ptr(Z2), int(N), _ptr(dX), _ptr(GR), _ptr(GP), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(stream)))


def chain_workspace_bytes(total_blocks, b):
    return lib().poetx_chain_workspace_bytes(int(total_blocks), int(b))


def poetx_chain_rule_sets(sets, b, accumulate=False, ws=None, stream=None):
    """sets: sequence of (Q32, G, nblocks, dtheta) tensors."""
    arr = (ChainSet * max(len(sets), 1))()
    for i, (q, g, nb, d) in enumerate(sets):
        arr[i] = ChainSet(_addr(q), _addr(g), int(nb), _addr(d))
    nbytes = ws.numel() if ws is not None else 0
    _check("poetx_chain_rule_sets", lib().poetx_chain_rule_sets(arr, len(sets), int(b),
                                                                POETX_ACCUMULATE_GRAD if accumulate else 0,
                                                                _ptr(ws), nbytes, _stream(stream)))


def poetx_forward(layer, W0p, thR, thP, sigma, tau, X, N, Y, ws, stream=None):
    _check("poetx_forward", lib().poetx_forward(ctypes.byref(layer), _ptr(W0p), _ptr(thR), _ptr(thP), _ptr(sigma),
                                                _ptr(tau), _ptr(X), int(N), _ptr(Y), _ptr(ws),
                                                ws.numel() if ws is not None else 0, _stream(stream)))


def poetx_backward(layer, W0p, thR, thP, sigma, tau, X, dY, N, dX, dthR, dthP, ws, stream=None):
    _check("poetx_backward", lib().poetx_backward(ctypes.byref(layer), _ptr(W0p), _ptr(thR), _ptr(thP), _ptr(sigma),
                                                  _ptr(tau), _ptr(X), _ptr(dY), int(N), _ptr(dX), _ptr(dthR),
                                                  _ptr(dthP), _ptr(ws), ws.numel() if ws is not None else 0,
                                                  _stream(stream)))


def poetx_merge(layer, W0p, thR, thP, sigma, tau, perm_seed, merge_index, ws, stream=None):
    _check("poetx_merge", lib().poetx_merge(ctypes.byref(layer), _ptr(W0p), _ptr(thR), _ptr(thP), _ptr(sigma),
                                            _ptr(tau), int(perm_seed) & (2 ** 64 - 1), int(merge_index),
                                            _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))


def poetx_merge_blocks(layer, W0p, blocks, thR, thP, sigma, tau, perm_seed, merge_index, ws, stream=None):
    _check("poetx_merge_blocks", lib().poetx_merge_blocks(
        ctypes.byref(layer), _ptr(W0p), None if blocks is None else ctypes.byref(blocks), _ptr(thR), _ptr(thP),
        _ptr(sigma), _ptr(tau), int(perm_seed) & (2 ** 64 - 1), int(merge_index), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(stream)))


def merge_sets(entries):
    """poetx_merge_set array from (layer, W0p, blocks, thR, thP, sigma, tau,
    perm_seed, merge_index) tuples; the Layer and Blocks objects must outlive
    the call (the array points at them)."""
    arr = (MergeSet * max(len(entries), 1))()
    for i, (layer, W0p, blocks, thR, thP, sigma, tau, seed, index) in enumerate(entries):
        arr[i] = MergeSet(ctypes.pointer(layer), _addr(W0p), ctypes.pointer(blocks), _addr(thR), _addr(thP),
                          _addr(sigma), _addr(tau), int(seed) & (2 ** 64 - 1), int(index))
    return arr


def merge_sets_workspace_bytes(sets, count):
    n = lib().poetx_merge_sets_workspace_bytes(sets, int(count))
    if n == 0 and count > 0:
        raise PoetxError("poetx_merge_sets_workspace_bytes", -1, last_error())
    return n


def poetx_merge_blocks_sets(sets, count, ws, stream=None):
    _check("poetx_merge_blocks_sets", lib().poetx_merge_blocks_sets(
        sets, int(count), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))


def poetx_make_permutation(seed, merge_index, side, n):
    """Host generator; returns a list of n ints."""
    buf = (ctypes.c_int32 * max(int(n), 1))()
    _check("poetx_make_permutation", lib().poetx_make_permutation(int(seed) & (2 ** 64 - 1), int(merge_index),
                                                                  int(side), int(n), ctypes.cast(buf, ctypes.c_void_p)))
    return list(buf)[: int(n)]


def poetx_adam_step(theta, grad, m, v, count, step, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, stream=None):
    _check("poetx_adam_step", lib().poetx_adam_step(_ptr(theta), _ptr(grad), _ptr(m), _ptr(v), int(count), int(step),
                                                    float(lr), float(beta1), float(beta2), float(eps),
                                                    _stream(stream)))


def timing_enable(on):
    _check("poetx_timing_enable", lib().poetx_timing_enable(1 if on else 0))


def timing_summary():
    """{kernel class: dict(launches, ms, flops, bytes)} of the recorded launches."""
    buf = ctypes.create_string_buffer(1 << 16)
    n = lib().poetx_timing_summary(buf, len(buf))
    if n < 0:
        raise PoetxError("poetx_timing_summary", n, last_error())
    out = {}
    for line in buf.value.decode().splitlines():
        name, cnt, ms, fl, by = line.split()
        out[name] = dict(launches=int(cnt), ms=float(ms), flops=float(fl), bytes=float(by))
    return out
