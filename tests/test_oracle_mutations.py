"""Plant plausible mistakes in the oracle (CPU only) and check that a pin catches each.

The fp64 brute force is the pin used here; each mutation is applied with
monkeypatch to the float32 oracle only.
"""
import numpy as np
import pytest

import jev_synth as S
from oracle import brute
from oracle import jev_oracle as O

CFG = S.with_overrides(S.CONFIGS["c1"], n_layers=1, n_vis=6, n_text=2, s_max=4,
                       fixed_lens=(4, 2), n_suffix=2, n_cands=3, hidden=32, mlp=40,
                       vocab=64, n_q_heads=4, n_kv_heads=2, head_dim=8)


@pytest.fixture(scope="module")
def setup():
    ws = S.WeightSource(CFG, 11)
    pre, suf = S.prefix_inputs(CFG, 11), S.suffix_inputs(CFG, 11)
    return ws, pre, suf, brute.score_suffixes(CFG, ws, pre, suf)


def _err(ws, pre, suf, ref):
    return float(np.max(np.abs(O.score_suffixes(ws, CFG, pre, suf) - ref)))


def test_unmutated_passes(setup):
    ws, pre, suf, ref = setup
    assert _err(ws, pre, suf, ref) < 1e-5


def _rope_wrong_sign(u, cos, sin):
    half = u.shape[-1] // 2
    a, b = u[..., :half], u[..., half:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([a * c + b * s, b * c - a * s], axis=-1).astype(np.float32)


def _attention_wrong_group(q, k, v, visible):
    Nq, Hq, D = q.shape
    Hkv = k.shape[1]
    out = np.empty_like(q)
    neg = np.where(visible, 0.0, -np.inf).astype(np.float32)
    for h in range(Hq):
        kv = h % Hkv                     # wrong grouping
        s = q[:, h] @ k[:, kv].T / np.sqrt(D) + neg
        p = np.exp(s - s.max(1, keepdims=True))
        out[:, h] = (p / p.sum(1, keepdims=True)) @ v[:, kv]
    return out


def _attention_no_scale(q, k, v, visible):
    return O_attention_orig(q * np.float32(np.sqrt(q.shape[-1])), k, v, visible)


O_attention_orig = O.attention


def _rmsnorm_no_gain(x, g, eps):
    return O_rmsnorm_orig(x, np.ones_like(g), eps)


O_rmsnorm_orig = O.rmsnorm


@pytest.mark.parametrize("name,attr,fn", [
    ("rope sign", "apply_rope", _rope_wrong_sign),
    ("gqa grouping", "attention", _attention_wrong_group),
    ("softmax scale", "attention", _attention_no_scale),
    ("dropped norm gain", "rmsnorm", _rmsnorm_no_gain),
    ("silu -> relu", "silu", lambda y: np.maximum(y, 0).astype(np.float32)),
])
def test_mutation_is_caught(setup, monkeypatch, name, attr, fn):
    ws, pre, suf, ref = setup
    monkeypatch.setattr(O, attr, fn)
    assert _err(ws, pre, suf, ref) > 1e-4, name
