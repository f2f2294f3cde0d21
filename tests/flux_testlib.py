"""Helpers shared by the tests: locating/building libflux and the attention
tolerance check.  Holds none of the method's arithmetic."""

import importlib.util
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "block_sparse_attention_flux_amd", "lib", "libflux.so")
HEADER = os.path.join(ROOT, "include", "flux.h")

# bf16-in / fp32-accumulate attention against the float64 oracle
ATOL = 2e-2
RTOL = 1e-2
FROB_RTOL = 1e-2


def ensure_built():
    """Build libflux.so unless it is built from exactly the current sources
    (the build's stamp: sha256 of sources, headers and flags)."""
    spec = importlib.util.spec_from_file_location(
        "flux_build", os.path.join(ROOT, "block_sparse_attention_flux_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.ensure_built()


def attn_errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    excess = np.abs(got - ref) - (ATOL + RTOL * np.abs(ref))
    frob = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    return float(excess.max()), float(frob), float(np.abs(got - ref).max())


def assert_attn_close(got, ref, what=""):
    """Elementwise allclose(atol=2e-2, rtol=1e-2) AND relative Frobenius
    error <= 1e-2 (the second check rejects near-zero outputs that the
    first alone would accept at long context)."""
    excess, frob, maxabs = attn_errors(got, ref)
    assert excess <= 0.0, f"{what}: elementwise tolerance exceeded (max |err| {maxabs:.3e})"
    assert frob <= FROB_RTOL, f"{what}: relative Frobenius error {frob:.3e} > {FROB_RTOL}"
    return frob, maxabs
