"""GPU invariance checks of the HIP path (the pages' claims about shared-prefix batching).

Pads and their content are never read, so re-padding is bit-identical; permuting the
suffixes permutes the outputs; duplicated suffixes score alike; a single candidate scores
log 1 = 0; an empty prefix is plain causal scoring; and a workspace or KV store filled with
NaN before the calls changes nothing (no uninitialised memory is read).
"""
import numpy as np
import pytest
import torch

import jev_synth as S
from oracle import jev_oracle as O
from tests.gpu_common import TOL, check_suffix_out, gpu_session, say
from vlm_shared_prefix_amd import jev as J

pytestmark = pytest.mark.gpu


def _repad(suf, s_max, seed):
    rng = np.random.default_rng(seed)
    B = suf["ids"].shape[0]
    ids = rng.integers(0, 2**20, size=(B, s_max)).astype(np.int32) % 997   # junk in every pad slot
    L = suf["ids"].shape[1]
    ids[:, :L] = np.where(np.arange(L)[None, :] < suf["lens"][:, None], suf["ids"], ids[:, :L])
    out = dict(suf)
    out["ids"] = np.ascontiguousarray(ids)
    return out


@pytest.mark.parametrize("name,seed", [("c1", 0), ("m7", 0)])
def test_padding_and_permutation(name, seed):
    cfg = S.CONFIGS[name]
    say(f"[invariance] padding / permutation {name} seed {seed}")
    sess, src = gpu_session(cfg, seed, precision="split" if cfg.dtype == "f32" else "default")
    pre, suf = S.prefix_inputs(cfg, seed), S.suffix_inputs(cfg, seed)
    sess.prefill(pre["vis"], pre["text_ids"])
    base = sess.score_suffixes(suf).cpu().numpy()
    wide = sess.score_suffixes(_repad(suf, suf["ids"].shape[1] + 24, seed)).cpu().numpy()
    assert np.array_equal(base, wide), "re-padding with junk ids changed the scores"
    perm = np.random.default_rng(seed + 1).permutation(len(suf["lens"]))
    sp = {k: np.ascontiguousarray(v[perm]) for k, v in suf.items()}
    got = sess.score_suffixes(sp).cpu().numpy()
    err = float(np.max(np.abs(got - base[perm])[np.isfinite(base[perm])]))
    say(f"  permuted suffixes: max |d| = {err:.3e}")
    assert err <= (1e-6 if cfg.dtype == "f32" else 2e-3), err
    sess.close()


@pytest.mark.parametrize("name,seed", [("c1", 1), ("m2", 0)])
def test_duplicates_single_candidate_length_one(name, seed):
    cfg = S.CONFIGS[name]
    say(f"[invariance] duplicates / C = 1 / L = 1 {name} seed {seed}")
    sess, src = gpu_session(cfg, seed, precision="split" if cfg.dtype == "f32" else "default")
    pre, suf = S.prefix_inputs(cfg, seed), S.suffix_inputs(cfg, seed)
    sess.prefill(pre["vis"], pre["text_ids"])
    B = len(suf["lens"])
    idx = np.array([0, 1, 0, 1 % B, 0])                  # suffix 0 three times
    sd = {k: np.ascontiguousarray(v[idx]) for k, v in suf.items()}
    sd["lens"][4] = 1                                    # a one-token suffix
    sd["n_cands"][3] = 1                                 # a single candidate
    sd["cands"][1, 1] = sd["cands"][1, 0]                # a duplicated candidate id
    ref = O.score_suffixes(src, cfg, pre, sd)
    got = sess.score_suffixes(sd).cpu().numpy()
    check_suffix_out(got, ref, sd["n_cands"], cfg.dtype, f"{name}/s{seed}/dup")
    assert got[3, 0] == 0.0, "a single candidate must score log 1 = 0"
    assert abs(got[1, 0] - got[1, 1]) <= 1e-6, "duplicate candidate ids must score alike"
    tol = 1e-6 if cfg.dtype == "f32" else 2e-3
    assert np.max(np.abs(got[0] - got[2])) <= tol, "the same suffix twice must score alike"
    sess.close()


@pytest.mark.parametrize("name", ["c1", "m7"])
def test_empty_prefix(name):
    """P = 0: plain causal scoring of the suffixes alone."""
    cfg = S.with_overrides(S.CONFIGS[name], n_vis=0, n_text=0)
    say(f"[invariance] empty prefix {name}")
    sess, src = gpu_session(cfg, 0, precision="split" if cfg.dtype == "f32" else "default")
    pre, suf = S.prefix_inputs(cfg, 0), S.suffix_inputs(cfg, 0)
    assert pre["vis"].shape[0] == 0 and len(pre["text_ids"]) == 0
    sess.prefill(pre["vis"], pre["text_ids"])
    ref = O.score_suffixes(src, cfg, pre, suf)
    got = sess.score_suffixes(suf).cpu().numpy()
    check_suffix_out(got, ref, suf["n_cands"], cfg.dtype, f"{name}/P=0")
    sess.close()


@pytest.mark.parametrize("name,seed", [("c1", 2), ("m7", 1), ("m5", 0)])
def test_poisoned_workspace_and_store(name, seed):
    """The same calls on buffers filled with NaN (0xFF bytes) beforehand give bit-identical
    results: no kernel reads workspace or KV-store memory it has not written."""
    cfg = S.CONFIGS[name]
    say(f"[invariance] NaN-poisoned workspace and KV store {name} seed {seed}")
    sess, src = gpu_session(cfg, seed, precision="split" if cfg.dtype == "f32" else "default")
    pre = S.prefix_inputs(cfg, seed)
    tree = cfg.n_questions > 0
    req = S.tree_inputs(cfg, seed) if tree else S.suffix_inputs(cfg, seed)

    def run(poison):
        sess.prefill(pre["vis"], pre["text_ids"])   # fresh KV store (torch.empty) per prefill
        if poison:
            sess.kv.fill_(255)
            ws = sess.workspace(1)
            ws.fill_(255)
            torch.cuda.synchronize()
            J.jev_prefill_prefix(sess.prefix, sess.vis, int(pre["vis"].shape[0]), pre["text_ids"], sess.ws)
            torch.cuda.synchronize()
            sess.ws.fill_(255)
        if tree:
            nbytes = sess.tree_ws_bytes(req, 0)
            sess.workspace(nbytes).fill_(255 if poison else 0)
            return [t.cpu().numpy() for t in sess.score_tree(req, 0)]
        sess.workspace(sess.suffix_ws_bytes(req)).fill_(255 if poison else 0)
        return [sess.score_suffixes(req).cpu().numpy()]

    clean = run(False)
    dirty = run(True)
    for a, b in zip(clean, dirty):
        assert np.array_equal(a, b), "results depend on uninitialised memory"
        assert np.all(np.isfinite(a) | np.isneginf(a))
    sess.close()
