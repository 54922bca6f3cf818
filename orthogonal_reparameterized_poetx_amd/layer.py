"""Device state of one POET-X linear layer, driven through the C ABI.

Holds the working-layout weight W0p (W0 with rows gathered by sigma and columns
by tau), the fp32 generators, the int32 permutations and cached workspaces,
all as torch tensors on one ROCm device.  Every computation is a call into
libpoetx.so; this class only owns memory and counts merges.
"""

import torch

from . import _lib as L


class PoetxLayer:
    def __init__(self, m, n, b, dtype="bf16", device="cuda:0", perm_seed=0, ws_pool=None, w0_int8=False,
                 separate_block_products=False, w0_transposed=False, x_permuted=False):
        """w0_int8: keep W0p in the INT8 weight format (per-row codes and
        scales, POETX_W0_INT8; bf16 layers), turned into bf16 inside the
        passes' GEMMs or dequantized by each pass (include/poetx.h says which).
        separate_block_products: at b in {64, 128, 256}, run the forward's R-side block
        product as a pass of its own rather than in the epilogue of the GEMM
        before it (POETX_SEPARATE_BLOCK_PRODUCTS; bit-identical results).
        w0_transposed: W0p also holds its transpose, which the forward
        products read (POETX_W0_TRANSPOSED; bf16 layers; 2 more bytes per
        weight; bit-identical results).
        x_permuted: the forward and backward calls take x' = X[:, tau]
        (permute_input) instead of X (POETX_X_PERMUTED; bf16 layers;
        bit-identical results).  x' follows tau, so it must be gathered
        again after a merge."""
        self.device = torch.device(device)
        self.dt = L.POETX_BF16 if dtype == "bf16" else L.POETX_F32
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.flags = (L.POETX_W0_INT8 if w0_int8 else 0) | \
            (L.POETX_SEPARATE_BLOCK_PRODUCTS if separate_block_products else 0) | \
            (L.POETX_W0_TRANSPOSED if w0_transposed else 0) | \
            (L.POETX_X_PERMUTED if x_permuted else 0)
        self.layer = L.Layer(m, n, b, self.dt, self.flags)
        self.m, self.n, self.b = m, n, b
        nt = b * (b - 1) // 2
        if w0_int8:
            self.W0p = torch.zeros(L.w0_bytes(self.layer), dtype=torch.uint8, device=self.device)
        elif w0_transposed:
            self.W0p = torch.zeros(L.w0_bytes(self.layer) // 2, dtype=self.tdtype, device=self.device)
        else:
            self.W0p = torch.zeros(m, n, dtype=self.tdtype, device=self.device)
        self.thR = torch.zeros(m // b, nt, dtype=torch.float32, device=self.device)
        self.thP = torch.zeros(n // b, nt, dtype=torch.float32, device=self.device)
        self.sigma = torch.arange(m, dtype=torch.int32, device=self.device)
        self.tau = torch.arange(n, dtype=torch.int32, device=self.device)
        self.perm_seed = int(perm_seed)
        self.merges = 0
        # workspaces by op; layers that run one after another on one stream
        # may share a pool (each op's buffer grows to the largest request)
        self._ws = {} if ws_pool is None else ws_pool
        self._blk = {}

    # -- workspaces (grown on demand, reused across calls)
    def workspace(self, op, N=0):
        need = L.workspace_bytes(self.layer, N, op)
        ws = self._ws.get(op)
        if ws is None or ws.numel() < need:
            ws = L.make_workspace(need, self.device)
            self._ws[op] = ws
        return ws

    def workspace_need(self, op, N=0):
        """Bytes of workspace that op needs for N tokens."""
        return L.workspace_bytes(self.layer, N, op)

    def pack(self, W0):
        """Load a true-coordinate weight: identity permutations, zero
        generators, then a merge (an exact relayout) into the first random
        layout (merge index 0).  INT8 layers quantize W0 first."""
        if self.flags & L.POETX_W0_INT8:
            L.poetx_quantize_w0(self.layer, W0.to(self.tdtype).contiguous(), self.W0p)
        else:
            # (the merge below also writes the transposed copy)
            self.weight().copy_(W0.to(self.tdtype))
        self.thR.zero_()
        self.thP.zero_()
        self.sigma.copy_(torch.arange(self.m, dtype=torch.int32, device=self.device))
        self.tau.copy_(torch.arange(self.n, dtype=torch.int32, device=self.device))
        self.merges = 0
        self.merge()

    def forward(self, X, Y=None, stream=None):
        N = X.shape[0]
        if Y is None:
            Y = torch.empty(N, self.m, dtype=self.tdtype, device=self.device)
        ws = self.workspace(L.OP_FORWARD, N)
        L.poetx_forward(self.layer, self.W0p, self.thR, self.thP, self.sigma, self.tau, X, N, Y, ws, stream)
        return Y

    def backward(self, X, dY, dX=None, dthR=None, dthP=None, want_dx=True, accumulate=False, stream=None):
        N = X.shape[0]
        if dX is None and want_dx:
            dX = torch.empty(N, self.n, dtype=self.tdtype, device=self.device)
        if dthR is None:
            dthR = torch.empty_like(self.thR)
        if dthP is None:
            dthP = torch.empty_like(self.thP)
        self.layer.flags = self.flags | (L.POETX_ACCUMULATE_GRAD if accumulate else 0)
        ws = self.workspace(L.OP_BACKWARD, N)
        try:
            L.poetx_backward(self.layer, self.W0p, self.thR, self.thP, self.sigma, self.tau, X, dY, N,
                             dX if want_dx else None, dthR, dthP, ws, stream)
        finally:
            self.layer.flags = self.flags
        return dX, dthR, dthP

    # -- prebuilt blocks: built for many layers at once (build_layer_blocks),
    #    then consumed by forward_blocks / backward_blocks
    def block_buffers(self, kind):
        """Device buffers of this layer's Cayley blocks for kind "forward",
        "backward" or "merge" (the arrays each call reads; see poetx_blocks)."""
        if kind in self._blk:
            return self._blk[kind]
        kR, kP, b, dev = self.m // self.b, self.n // self.b, self.b, self.device

        def t(k, dt):
            return torch.empty(k, b, b, dtype=dt, device=dev)
        f32, bf = torch.float32, torch.bfloat16
        if self.dt == L.POETX_F32:
            q = dict(Q32R=t(kR, f32), Q32P=t(kP, f32))
        elif kind == "forward":
            q = dict(QR=t(kR, bf), QP=t(kP, bf))
        elif kind == "merge":
            q = dict(QR=t(kR, bf), QTP=t(kP, bf))
        else:
            q = dict(Q32R=t(kR, f32), Q32P=t(kP, f32), QP=t(kP, bf), QTR=t(kR, bf), QTP=t(kP, bf))
        self._blk[kind] = (q, L.make_blocks(**q))
        return self._blk[kind]

    def block_sets(self, kind):
        """poetx_block_set entries (R side, P side) filling block_buffers(kind)."""
        q, _ = self.block_buffers(kind)
        kR, kP = self.m // self.b, self.n // self.b
        return [(self.thR, kR, q.get("Q32R"), q.get("QR"), q.get("QTR")),
                (self.thP, kP, q.get("Q32P"), q.get("QP"), q.get("QTP"))]

    def permute_input(self, X, Xp=None, stream=None):
        """x' = X[:, tau], the input in the working layout (poetx_permute_input)."""
        N = X.shape[0]
        if Xp is None:
            Xp = torch.empty(N, self.n, dtype=self.tdtype, device=self.device)
        L.poetx_permute_input(self.layer, self.tau, X, N, Xp, stream)
        return Xp

    def forward_blocks(self, X, Y=None, stream=None):
        N = X.shape[0]
        if Y is None:
            Y = torch.empty(N, self.m, dtype=self.tdtype, device=self.device)
        ws = self.workspace(L.OP_FORWARD_BLOCKS, N)
        L.poetx_forward_blocks(self.layer, self.W0p, self.block_buffers("forward")[1], self.sigma, self.tau, X, N,
                               Y, ws, stream)
        return Y

    def forward_blocks_noalloc(self, X, Y, stream=None):
        """forward_blocks without a workspace (poetx_forward_blocks_noalloc):
        Y must be given, nothing is allocated."""
        L.poetx_forward_blocks_noalloc(self.layer, self.W0p, self.block_buffers("forward")[1], self.sigma, self.tau,
                                       X, X.shape[0], Y, stream)
        return Y

    def forward_blocks_z2(self, X, Y=None, Z2=None, stream=None):
        """forward_blocks that also returns z2' (working layout) for backward_blocks_dq_z2."""
        N = X.shape[0]
        if Y is None:
            Y = torch.empty(N, self.m, dtype=self.tdtype, device=self.device)
        if Z2 is None:
            Z2 = torch.empty(N, self.m, dtype=self.tdtype, device=self.device)
        ws = self.workspace(L.OP_FORWARD_BLOCKS, N)
        L.poetx_forward_blocks_z2(self.layer, self.W0p, self.block_buffers("forward")[1], self.sigma, self.tau, X,
                                  N, Y, Z2, ws, stream)
        return Y, Z2

    def backward_blocks(self, X, dY, dX=None, dthR=None, dthP=None, want_dx=True, accumulate=False, stream=None):
        N = X.shape[0]
        if dX is None and want_dx:
            dX = torch.empty(N, self.n, dtype=self.tdtype, device=self.device)
        if dthR is None:
            dthR = torch.empty_like(self.thR)
        if dthP is None:
            dthP = torch.empty_like(self.thP)
        self.layer.flags = self.flags | (L.POETX_ACCUMULATE_GRAD if accumulate else 0)
        ws = self.workspace(L.OP_BACKWARD_BLOCKS, N)
        try:
            L.poetx_backward_blocks(self.layer, self.W0p, self.block_buffers("backward")[1], self.sigma, self.tau,
                                    X, dY, N, dX if want_dx else None, dthR, dthP, ws, stream)
        finally:
            self.layer.flags = self.flags
        return dX, dthR, dthP

    def dq_buffers(self):
        """fp32 dL/dQ of this layer's R and P blocks ([k][b][b] each)."""
        if "dq" not in self._blk:
            kR, kP, b = self.m // self.b, self.n // self.b, self.b
            self._blk["dq"] = (torch.empty(kR, b, b, dtype=torch.float32, device=self.device),
                               torch.empty(kP, b, b, dtype=torch.float32, device=self.device))
        return self._blk["dq"]

    def backward_blocks_dq(self, X, dY, dX=None, want_dx=True, stream=None):
        """Backward up to dL/dQ (see chain_rule_layers); returns (dX, GR, GP)."""
        N = X.shape[0]
        if dX is None and want_dx:
            dX = torch.empty(N, self.n, dtype=self.tdtype, device=self.device)
        GR, GP = self.dq_buffers()
        ws = self.workspace(L.OP_BACKWARD_DQ, N)
        L.poetx_backward_blocks_dq(self.layer, self.W0p, self.block_buffers("backward")[1], self.sigma, self.tau,
                                   X, dY, N, dX if want_dx else None, GR, GP, ws, stream)
        return dX, GR, GP

    def backward_blocks_dq_z2(self, X, dY, Z2, dX=None, want_dx=True, stream=None):
        """backward_blocks_dq with z2' from forward_blocks_z2 instead of recomputed; returns (dX, GR, GP)."""
        N = X.shape[0]
        if dX is None and want_dx:
            dX = torch.empty(N, self.n, dtype=self.tdtype, device=self.device)
        GR, GP = self.dq_buffers()
        ws = self.workspace(L.OP_BACKWARD_DQ, N)
        L.poetx_backward_blocks_dq_z2(self.layer, self.W0p, self.block_buffers("backward")[1], self.sigma,
                                      self.tau, X, dY, Z2, N, dX if want_dx else None, GR, GP, ws, stream)
        return dX, GR, GP

    def weight(self):
        """The bf16 working-layout weight the passes use ([m][n])."""
        if self.flags & L.POETX_W0_TRANSPOSED:
            return self.W0p[:self.m * self.n].view(self.m, self.n)
        if not self.flags & L.POETX_W0_INT8:
            return self.W0p
        W = torch.empty(self.m, self.n, dtype=torch.bfloat16, device=self.device)
        L.poetx_dequantize_w0(self.layer, self.W0p, W)
        return W

    def weight_t(self):
        """The transposed copy [n][m] of a POETX_W0_TRANSPOSED layer."""
        off = L.w0_bytes(self.layer) // 2 - self.m * self.n
        return self.W0p[off:off + self.m * self.n].view(self.n, self.m)

    def merge_blocks(self, stream=None, ws=None):
        """Merge with blocks from build_layer_blocks(..., "merge"); ws: a merge
        workspace of the caller's (at least workspace_bytes(layer, 0,
        OP_MERGE_BLOCKS) bytes), else this layer's own."""
        if ws is None:
            ws = self.workspace(L.OP_MERGE_BLOCKS)
        elif ws.numel() < L.workspace_bytes(self.layer, 0, L.OP_MERGE_BLOCKS):
            raise ValueError("merge workspace too small")
        L.poetx_merge_blocks(self.layer, self.W0p, self.block_buffers("merge")[1], self.thR, self.thP, self.sigma,
                             self.tau, self.perm_seed, self.merges, ws, stream)
        self.merges += 1

    def merge(self, stream=None):
        ws = self.workspace(L.OP_MERGE)
        L.poetx_merge(self.layer, self.W0p, self.thR, self.thP, self.sigma, self.tau, self.perm_seed,
                      self.merges, ws, stream)
        self.merges += 1


_build_ws = {}


def merge_layers_sets(layers, ws=None, stream=None):
    """poetx_merge_blocks_sets over the layers (blocks from
    build_layer_blocks(layers, "merge")): the same results as each layer's
    merge_blocks, with the launches after the block products shared.  ws: a
    workspace of at least merge_sets_workspace_need(layers) bytes, else one is
    allocated."""
    if not layers:
        return
    sets = L.merge_sets([(lay.layer, lay.W0p, lay.block_buffers("merge")[1], lay.thR, lay.thP, lay.sigma, lay.tau,
                          lay.perm_seed, lay.merges) for lay in layers])
    need = L.merge_sets_workspace_bytes(sets, len(layers))
    if ws is None:
        ws = L.make_workspace(need, layers[0].device)
    elif ws.numel() < need:
        raise ValueError("merge workspace too small")
    L.poetx_merge_blocks_sets(sets, len(layers), ws, stream)
    for lay in layers:
        lay.merges += 1


def merge_sets_workspace_need(layers):
    """Bytes of workspace merge_layers_sets needs for these layers."""
    if not layers:
        return 0
    sets = L.merge_sets([(lay.layer, lay.W0p, lay.block_buffers("merge")[1], lay.thR, lay.thP, lay.sigma, lay.tau,
                          lay.perm_seed, lay.merges) for lay in layers])
    return L.merge_sets_workspace_bytes(sets, len(layers))


def build_layer_blocks(layers, kind, stream=None, cnp_terms=0):
    """Build the Cayley blocks of every layer for kind ("forward",
    "backward" or "merge") with one poetx_build_block_sets call per block
    size, so the builder's grid spans the blocks of all the layers.
    cnp_terms > 0 (b <= 256): poetx_build_block_sets_cnp with that many
    series terms (the truncated series where its bound allows)."""
    by_b = {}
    for lay in layers:
        by_b.setdefault(lay.b, []).extend(lay.block_sets(kind))
    for b, sets in by_b.items():
        dev = layers[0].device
        if cnp_terms and b <= 256:
            need = L.build_cnp_workspace_bytes(sum(s[1] for s in sets), b)
            ws = _build_ws.get((dev, b, kind, "cnp"))
            if ws is None or ws.numel() < need:
                ws = L.make_workspace(need, dev)
                _build_ws[(dev, b, kind, "cnp")] = ws
            L.poetx_build_block_sets_cnp(sets, b, cnp_terms, ws, stream)
            continue
        need = L.build_workspace_bytes(sum(s[1] for s in sets), b)
        # one workspace per kind: builds of different kinds may run
        # concurrently on different streams
        ws = _build_ws.get((dev, b, kind))
        if need and (ws is None or ws.numel() < need):
            ws = L.make_workspace(need, dev)
            _build_ws[(dev, b, kind)] = ws
        L.poetx_build_block_sets(sets, b, ws if need else None, stream)


_chain_ws = {}


def chain_rule_layers(layers, grads, accumulate=False, stream=None):
    """Generator gradients of many layers from their dL/dQ (backward_blocks_dq)
    and backward blocks, in one poetx_chain_rule_sets call per block size.
    grads: one (dthR, dthP) pair per layer."""
    by_b = {}
    for lay, (dR, dP) in zip(layers, grads):
        q, _ = lay.block_buffers("backward")
        GR, GP = lay.dq_buffers()
        kR, kP = lay.m // lay.b, lay.n // lay.b
        by_b.setdefault(lay.b, []).extend([(q["Q32R"], GR, kR, dR), (q["Q32P"], GP, kP, dP)])
    for b, sets in by_b.items():
        dev = layers[0].device
        need = L.chain_workspace_bytes(sum(s[2] for s in sets), b)
        # one workspace per stream: chain rules of different layers may run
        # concurrently on different streams
        sid = L.stream_handle(stream)
        ws = _chain_ws.get((dev, b, sid))
        if need and (ws is None or ws.numel() < need):
            ws = L.make_workspace(need, dev)
            _chain_ws[(dev, b, sid)] = ws
        L.poetx_chain_rule_sets(sets, b, accumulate, ws if need else None, stream)
