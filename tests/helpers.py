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


def assert_close(gpu, ref, what=""):
    r = tol_ratio(gpu, ref)
    say(f"  {what}: max |err|/tol = {r:.4f}")
    assert r <= 1.0, f"{what}: max |err|/tol = {r}"


def to_dev_x(Xbits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(Xbits).view(np.int16)).cuda()


def oracle_route(L, Xbits):
    X = S.x_bits_to_f64(Xbits, L.cfg["xdtype"])
    z, r, _ = O.route(X, L.W_r, L.bias, L.K)
    return X, z, r
