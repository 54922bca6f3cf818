"""Device state of one POET-X linear layer, driven through the C ABI.

Holds the working-layout weight W0p (W0 with rows gathered by sigma and columns
by tau), the fp32 generators, the int32 permutations and cached workspaces,
all as torch tensors on one ROCm device.  Every computation is a call into
libpoetx.so; this class only owns memory and counts merges.
"""

import torch

from . import _lib as L


class PoetxLayer:
    def __init__(self, m, n, b, dtype="bf16", device="cuda:0", perm_seed=0):
        self.device = torch.device(device)
        self.dt = L.POETX_BF16 if dtype == "bf16" else L.POETX_F32
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.layer = L.Layer(m, n, b, self.dt)
        self.m, self.n, self.b = m, n, b
        nt = b * (b - 1) // 2
        self.W0p = torch.zeros(m, n, dtype=self.tdtype, device=self.device)
        self.thR = torch.zeros(m // b, nt, dtype=torch.float32, device=self.device)
        self.thP = torch.zeros(n // b, nt, dtype=torch.float32, device=self.device)
        self.sigma = torch.arange(m, dtype=torch.int32, device=self.device)
        self.tau = torch.arange(n, dtype=torch.int32, device=self.device)
        self.perm_seed = int(perm_seed)
        self.merges = 0
        self._ws = {}

    # -- workspaces (grown on demand, reused across calls)
    def workspace(self, op, N=0):
        need = L.workspace_bytes(self.layer, N, op)
        ws = self._ws.get(op)
        if ws is None or ws.numel() < need:
            ws = L.make_workspace(need, self.device)
            self._ws[op] = ws
        return ws

    def pack(self, W0):
        """Load a true-coordinate weight: identity permutations, zero
        generators, then a merge (an exact relayout) into the first random
        layout (merge index 0)."""
        self.W0p.copy_(W0.to(self.tdtype))
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
        self.layer.flags = L.POETX_ACCUMULATE_GRAD if accumulate else 0
        ws = self.workspace(L.OP_BACKWARD, N)
        L.poetx_backward(self.layer, self.W0p, self.thR, self.thP, self.sigma, self.tau, X, dY, N,
                         dX if want_dx else None, dthR, dthP, ws, stream)
        self.layer.flags = 0
        return dX, dthR, dthP

    def merge(self, stream=None):
        ws = self.workspace(L.OP_MERGE)
        L.poetx_merge(self.layer, self.W0p, self.thR, self.thP, self.sigma, self.tau, self.perm_seed,
                      self.merges, ws, stream)
        self.merges += 1
