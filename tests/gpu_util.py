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


# ---- tolerances ---------------------------------------------------------
# The stated bounds: bf16 outputs |d| <= 1e-3 + 2e-2 |ref|, fp32 1e-5 relative.
# A bf16 pipeline with fp32 accumulation and the float64 oracle with the same
# bf16 storage points round a stored value (a bf16 copy of Q, z1', z2', gZ2',
# gZ1') to different neighbours whenever the two pre-rounding values straddle
# a rounding boundary: then the two stored values are one ulp apart.  The
# fp32 Cayley solve is accurate to ~1e-6 absolute, so about 1% of the bf16 Q
# entries differ, and the differences cascade to 2-8% of the one-ulp flips
# in z2'.  Such a flip is a deviation of the intermediate's size, not of the
# output element's, so near-zero outputs cannot meet the stated bound; each
# output kind gets a floor derived from how the flips reach it:
#
# * bf16 outputs behind an orthogonal block (Y behind z2', dX behind gZ1',
#   the merged weight behind W Q_P): a flip of v_j moves output i by
#   Q_ij ulp(v_j), |Q_ij| <= 1, and ulp(v) <= 2u|v| with u = 2^-8; the largest
#   of a block's entries sit near 3 rms(v), so one flip there moves an output
#   by up to 6u rms(v): floor = 6 u rms(v).
# * fp32 sums over T terms (dL/dQ over tokens, dtheta through the linear
#   chain rule; z2' over input features): dG = sum_t a_t dv_t.  Its relative
#   rms deviation equals that of the intermediate v, at most ETA (asserted on
#   z2' where the kept-z2 call returns it), and over many flipped terms it is
#   Gaussian: 6 ETA rms(ref).  With few terms one flip dominates: a_t dv_t
#   with both factors at 3 rms and dv_t <= 2u|v_t| is 18u rms(a) rms(v) =
#   18u rms(G)/sqrt(T); a few flips per sum and the chain rule's spread
#   (entries of I + Q^T up to 2, on both sides, and dtheta = G_S - G_S^T)
#   give at most 4 times that.  floor = (6 ETA + 72u / sqrt(T)) rms(ref).
# * fp32 layers and fp32 optimizer state: the error of a K-term fp32 sum is
#   ~sqrt(K) 2^-24 times the rms of its terms, independent of the element's
#   own size: floor = 1e-5 rms(ref) (the stated relative bound at the rms).
#
# Each comparison also asserts a ceiling on the fraction of elements outside
# the stated bound (strict fraction) and a normwise bound, so that a
# regression that moves many elements cannot hide under the floor.  For fp32
# the strict fraction is the share of entries too close to zero for a
# relative 1e-5 (measured up to 9% on the fp32 layers); its ceiling is a
# regression guard, the normwise bound the sharper check.
U_BF16 = 2.0 ** -8
ETA_BF16 = 1e-3
K_FLOOR = 6.0
MAX_STRICT = {"bf16": 0.02, "sum": 0.04, "f32": 0.25}
MAX_REL_NORM = {"bf16": 4e-3, "sum": 2 * ETA_BF16, "f32": 5e-6}


def rms(a):
    a = np.asarray(a, dtype=np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def bf16_floor(v):
    """Floor of a bf16 output fed through an orthogonal block by the bf16
    intermediate v: K_FLOOR * u * rms(v)."""
    return K_FLOOR * U_BF16 * rms(v)


def layer_floors(W0, it):
    """Floors of a bf16 layer's outputs from the oracle's intermediates
    (oracle.backward(..., intermediates=True))."""
    return dict(Y=bf16_floor(it["Z2"]), dX=bf16_floor(it["gZ1"]), W=bf16_floor(W0))


def sum_floor(ref, terms):
    """Floor of an fp32 sum over `terms` terms of a bf16 layer:
    (K_FLOOR * ETA + 72u / sqrt(terms)) * rms(ref)."""
    return (K_FLOOR * ETA_BF16 + 72.0 * U_BF16 / np.sqrt(max(int(terms), 1))) * rms(ref)


def compare(got, ref, kind, name, floor=None, max_strict=None, terms=None):
    """Elementwise parity with the oracle.

    kind "bf16": bf16 outputs, |d| <= 1e-3 + 2e-2 |ref| + floor (floor given
    by the caller, see bf16_floor), normwise ||d|| / ||ref|| <= 4e-3;
    kind "sum": fp32 sums over `terms` terms of bf16 layers (dL/dQ, dtheta
    over tokens), |d| <= 1e-3 + 2e-2 |ref| + sum_floor(ref, terms), normwise
    <= 2 ETA;
    kind "f32": |d| <= 1e-5 max(|ref|, rms(ref)), normwise <= 1e-5.
    The fraction of elements outside the stated bound (1e-3 + 2e-2|ref|, or
    1e-5|ref| for fp32) must not exceed MAX_STRICT[kind] (or max_strict).
    Returns a dict of statistics.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % name
    d = np.abs(got - ref)
    r = rms(ref)
    if kind == "f32":
        strict_tol = 1e-5 * np.abs(ref)
        fl = 1e-5 * r if floor is None else floor
        tol = np.maximum(strict_tol, fl)
    else:
        strict_tol = 1e-3 + 2e-2 * np.abs(ref)
        if kind == "sum":
            assert terms is not None or floor is not None, "sum comparisons take the number of summed terms"
            fl = sum_floor(ref, terms) if floor is None else floor
        elif kind == "bf16":
            assert floor is not None, "bf16 comparisons take the floor of the intermediate feeding the output"
            fl = floor
        else:
            raise ValueError(kind)
        tol = strict_tol + fl
    bad = d > tol
    strict = d > strict_tol
    ceiling = MAX_STRICT[kind] if max_strict is None else max_strict
    stats = dict(name=name, kind=kind, n=int(ref.size), fail=int(bad.sum()),
                 strict=float(strict.mean()) if d.size else 0.0, floor=float(fl),
                 max_abs=float(d.max()) if d.size else 0.0,
                 max_ratio=float(np.max(d / tol)) if d.size and np.all(tol > 0) else
                 (float(np.max(np.where(tol > 0, d / np.where(tol > 0, tol, 1.0), np.where(d > 0, np.inf, 0.0))))
                  if d.size else 0.0),
                 rel_norm=float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)))
    print("  %-12s %-4s fail=%d/%d strict=%.4f (<= %.3f) floor=%.3g max_abs=%.3g max_tol_ratio=%.3f rel_norm=%.3g"
          % (name, kind, stats["fail"], stats["n"], stats["strict"], ceiling, fl, stats["max_abs"],
             stats["max_ratio"], stats["rel_norm"]), flush=True)
    assert stats["fail"] == 0, stats
    assert stats["strict"] <= ceiling, stats
    if ref.size and np.linalg.norm(ref) > 0:
        assert stats["rel_norm"] <= MAX_REL_NORM[kind], stats
    return stats


def inputs_to_device(inp):
    dt = inp["dtype"]
    return dict(W0=to_dev(inp["W0"][0], dt), thR=to_dev(inp["thR"][0], "f32"), thP=to_dev(inp["thP"][0], "f32"),
                X=to_dev(inp["X"][0], dt), gY=to_dev(inp["gY"][0], dt))


def make_layer(inp, device="cuda:0", w0_int8=False, **kw):
    """PoetxLayer packed from the true-coordinate W0 (w0_int8: quantized to
    the INT8 weight format), generators loaded; kw go to PoetxLayer."""
    from orthogonal_reparameterized_poetx_amd import PoetxLayer
    d = inputs_to_device(inp)
    lay = PoetxLayer(inp["m"], inp["n"], inp["b"], inp["dtype"], device, perm_seed=inp["perm_seed"],
                     w0_int8=w0_int8, **kw)
    lay.pack(d["W0"])
    lay.thR.copy_(d["thR"])
    lay.thP.copy_(d["thP"])
    return lay, d


def oracle_perms(inp, merge_index=0):
    return (oracle.make_permutation(inp["perm_seed"], merge_index, 0, inp["m"]),
            oracle.make_permutation(inp["perm_seed"], merge_index, 1, inp["n"]))
