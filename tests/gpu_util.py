"""Helpers shared by the GPU parity tests (not collected by pytest).

Inputs come from ``workloads`` (seeded, shared with the oracle); expected
values come only from ``oracle``; the product path is exercised through the
C ABI via ``orthogonal_reparameterized_poetx_amd``.
"""

import numpy as np

import oracle
import workloads as WL


def torch_mod():
    import torch
    return torch


def to_dev(storage, dtype, device="cuda:0"):
    torch = torch_mod()
    a = np.ascontiguousarray(storage)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == "f32":
        return torch.from_numpy(a.astype(np.float32)).to(device)
    if dtype == "i32":
        return torch.from_numpy(a.astype(np.int32)).to(device)
    raise ValueError(dtype)


def from_dev(t):
    """Exact float64 (or int64) numpy copy of a device tensor."""
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return WL.bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    if t.dtype == torch.float32:
        return t.cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.int64)


def compare(got, ref, dtype, name, rms_floor=True, max_fail_frac=0.0):
    """Elementwise parity with the oracle.

    bf16: |d| <= 1e-3 + 2e-2 * s, fp32: |d| <= 1e-5 * s, with
    s = max(|ref|, rms(ref)) (rms_floor) or s = |ref|.  For bf16 tensors the
    normwise error ||d|| / ||ref|| must also stay below 4e-3 (about one bf16
    half-ulp, 2^-8).  The floor: an fp32-accumulating pipeline and the float64
    oracle round an intermediate (Q, z1, z2, ...) to different sides of a
    bf16 tie now and then; the one-ulp step of that intermediate reaches every
    output it feeds, with a size set by the intermediate's scale (rms of the
    tensor), not by the output element.  "strict" counts the elements outside
    the bound with s = |ref|; it is reported, not asserted.
    Returns a dict of statistics; asserts the failure fraction is at most
    max_fail_frac.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % name
    d = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    s = np.maximum(np.abs(ref), rms) if rms_floor else np.abs(ref)
    rel, ab = (1e-5, 0.0) if dtype == "f32" else (2e-2, 1e-3)
    tol = ab + rel * s
    bad = d > tol
    strict = d > ab + rel * np.abs(ref)
    stats = dict(name=name, n=int(ref.size), fail=int(bad.sum()), strict=float(strict.mean()) if d.size else 0.0,
                 max_abs=float(d.max()) if d.size else 0.0,
                 max_ratio=float(np.max(np.where(tol > 0, d / np.where(tol > 0, tol, 1.0),
                                                 np.where(d > 0, np.inf, 0.0)))) if d.size else 0.0,
                 rel_norm=float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)))
    assert stats["fail"] <= max_fail_frac * max(ref.size, 1), stats
    if dtype == "bf16":
        assert stats["rel_norm"] <= 4e-3, stats
    return stats


def inputs_to_device(inp):
    dt = inp["dtype"]
    return dict(W0=to_dev(inp["W0"][0], dt), thR=to_dev(inp["thR"][0], "f32"), thP=to_dev(inp["thP"][0], "f32"),
                X=to_dev(inp["X"][0], dt), gY=to_dev(inp["gY"][0], dt))


def make_layer(inp, device="cuda:0"):
    """PoetxLayer packed from the true-coordinate W0, generators loaded."""
    from orthogonal_reparameterized_poetx_amd import PoetxLayer
    d = inputs_to_device(inp)
    lay = PoetxLayer(inp["m"], inp["n"], inp["b"], inp["dtype"], device, perm_seed=inp["perm_seed"])
    lay.pack(d["W0"])
    lay.thR.copy_(d["thR"])
    lay.thP.copy_(d["thP"])
    return lay, d


def oracle_perms(inp, merge_index=0):
    return (oracle.make_permutation(inp["perm_seed"], merge_index, 0, inp["m"]),
            oracle.make_permutation(inp["perm_seed"], merge_index, 1, inp["n"]))
