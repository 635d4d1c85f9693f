"""Shared helpers for the GPU tests (not collected by pytest)."""
import os
import sys

import numpy as np

import jev_synth as S

# Parity bars (from the build target): max |Δ log-prob| <= 1e-4 for float32
# models and <= 2e-2 for bfloat16 models; identical argmax wherever the
# oracle's top-1/top-2 margin is >= 0.05.
TOL = {"f32": 1e-4, "bf16": 2e-2}
MARGIN = 0.05


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def resolve_precision(precision):
    """"default" -> the library's default GEMM precision mode."""
    if precision == "default":
        from vlm_shared_prefix_amd.session import DEFAULT_PRECISION
        return DEFAULT_PRECISION
    return precision


def gpu_session(cfg, seed, src=None, precision="default"):
    """precision (bf16 models): "default" = the library default; "split" = two-term bfloat16
    GEMMs; "f16_down" / "f16" = single-pass float16 GEMMs on a float16 weight mirror for the
    down projection / every decoder matrix."""
    from vlm_shared_prefix_amd.session import Session
    src = src or S.WeightSource(cfg, seed)
    return Session(cfg, src.glob, src.layer, precision=resolve_precision(precision)), src


def check_suffix_out(got, ref, n_cands, dtype, label=""):
    """Element-wise |Δ| bar plus argmax agreement where the oracle margin >= 0.05."""
    from oracle import jev_oracle as O
    tol = TOL[dtype]
    B = ref.shape[0]
    for b in range(B):
        n = int(n_cands[b])
        assert np.all(np.isneginf(got[b, n:])), f"{label} pad slots of row {b} not -inf"
    valid = np.isfinite(ref)
    err = float(np.max(np.abs(got[valid] - ref[valid]))) if valid.any() else 0.0
    say(f"  {label}: max |dlogp| = {err:.3e} (bar {tol:g})")
    assert np.all(np.isfinite(got[valid])), f"{label}: non-finite outputs"
    assert err <= tol, f"{label}: max |dlogp| {err:.3e} > {tol:g}"
    m = O.margins(ref, n_cands)
    a_ref = O.argmax_first(ref, n_cands)
    a_got = O.argmax_first(got, n_cands)
    sel = m >= MARGIN
    assert np.array_equal(a_ref[sel], a_got[sel]), f"{label}: argmax differs where margin >= {MARGIN}"
    return err
