"""Shared helpers for the GPU parity tests."""
import sys

import numpy as np

import mpb_synth as S
import oracle as O

ATOL, RTOL = 1e-3, 1e-2  # |gpu - ref| <= 1e-3 + 1e-2 |ref|, every element


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tol_ratio(gpu, ref):
    """max over elements of |gpu - ref| / (ATOL + RTOL |ref|); <= 1 passes."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape
    if gpu.size == 0:
        return 0.0
    assert np.isfinite(gpu).all()
    return float((np.abs(gpu - ref) / (ATOL + RTOL * np.abs(ref))).max())


def rel_to_max(gpu, ref):
    """max |gpu - ref| / max |ref| (a scale-free precision figure)."""
    ref = np.asarray(ref, np.float64)
    m = np.abs(ref).max() if ref.size else 0.0
    return float(np.abs(np.asarray(gpu, np.float64) - ref).max() / m) if m > 0 else 0.0


# Regression guard on top of the stated tolerance: the HIP path forms exact
# fp16 products, accumulates in fp32 and carries h as an fp16 hi/lo pair
# (~2^-22 relative), so on these layers its error measured relative to max|ref|
# stays near 1e-6; an error ten times that level means precision was lost
# somewhere (e.g. h rounded to a single fp16) even when the tolerance holds.
PREC_GUARD = 2e-5


def assert_close(gpu, ref, what="", guard=PREC_GUARD):
    r = tol_ratio(gpu, ref)
    rm = rel_to_max(gpu, ref)
    say(f"  {what}: max |err|/tol = {r:.4f}, max|err|/max|ref| = {rm:.2e}")
    assert r <= 1.0, f"{what}: max |err|/tol = {r}"
    if guard is not None:
        assert rm <= guard, f"{what}: max|err|/max|ref| = {rm:.2e} above the precision guard {guard}"


def to_dev_x(Xbits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(Xbits).view(np.int16)).cuda()


def oracle_route(L, Xbits):
    X = S.x_bits_to_f64(Xbits, L.cfg["xdtype"])
    z, r, _ = O.route(X, L.W_r, L.bias, L.K)
    return X, z, r
