"""Shared helpers for the GPU parity tests (tolerances and marshalling)."""

import sys

import numpy as np

# Tolerances stated for the hot path: attention max |err| <= 1e-2 and mean
# |err| <= 1e-3 on fp16 outputs; DDIM max-norm relative error <= 1e-5.
ATTN_MAX_ABS = 1e-2
ATTN_MEAN_ABS = 1e-3
DDIM_REL = 1e-5
# Window noise in fp32: u is exact; ln u, the square root and sin/cos(2 pi u)
# are each within a few ulp, so |z - z_fp64| <= ~2e-6 for |z| <= 5.8 (the
# largest normal a 24-bit uniform can give); the bound leaves a 5x margin.
NOISE_ABS = 1e-5


def say(*msg):
    """Print a case name and flush, so a failing GPU step names its case."""
    print("[case]", *msg, flush=True)
    sys.stdout.flush()


def attn_errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    return {
        "max_abs": float(err.max()),
        "mean_abs": float(err.mean()),
        "norm_rel": float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)),
    }


def assert_attn_close(got, ref, what=""):
    e = attn_errors(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert e["max_abs"] <= ATTN_MAX_ABS, f"{what}: {e}"
    assert e["mean_abs"] <= ATTN_MEAN_ABS, f"{what}: {e}"
    return e


def maxnorm_rel(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - ref)) / np.max(np.abs(ref)))
