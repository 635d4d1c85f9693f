"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by element.

Sizes here are small enough for the oracle to run live, yet span several
attention row blocks (128 rows), several 64-key tiles with ragged tails,
several GEMM tiles, suffix length 1 and candidate overlap in trees.
"""
import numpy as np
import pytest

import jev_synth as S
from oracle import jev_oracle as O
from tests.gpu_common import TOL, check_suffix_out, gpu_session, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,seed,precision", [("c1", 0, "f32"), ("c1", 1, "f32"), ("c1", 2, "f32"),
                                                 ("m2", 0, "default"), ("m7", 0, "default"), ("m2", 3, "default"),
                                                 ("m7l", 0, "default"), ("m7", 0, "f16_down"), ("m2", 0, "split"), ("m7", 0, "split"),
                                                 ("m7l", 0, "split"), ("m7", 0, "f16"), ("m7l", 0, "f16"),
                                                 ("m7", 0, "f16_prefill"), ("m2", 1, "f16_prefill"),
                                                 ("m64", 0, "default"), ("m64", 1, "split"),
                                                 ("mb", 0, "default"), ("mb", 1, "split")])
def test_score_suffixes_vs_oracle(name, seed, precision):
    cfg = S.CONFIGS[name]
    say(f"[parity] score_suffixes {name} seed {seed} ({precision})")
    sess, src = gpu_session(cfg, seed, precision="split" if precision == "f32" else precision)
    pre, suf = S.prefix_inputs(cfg, seed), S.suffix_inputs(cfg, seed)
    ref = O.score_suffixes(src, cfg, pre, suf)
    sess.prefill(pre["vis"], pre["text_ids"])
    got = sess.score_suffixes(suf).cpu().numpy()
    check_suffix_out(got, ref, suf["n_cands"], cfg.dtype, f"{name}/s{seed}")
    sess.close()


@pytest.mark.parametrize("name,n,precision", [("m2", 1, "default"), ("m2", 2, "split"), ("m7", 1, "default"),
                                              ("m7", 2, "f16"), ("m7", 3, "split"), ("m7", 1, "f16_down"),
                                              ("m64", 1, "default"), ("m64", 2, "f16_prefill"),
                                              ("mk", 1, "default"), ("mk", 1, "split"), ("mk", 2, "default"),
                                              ("mk", 4, "split")])
def test_few_rows_vs_oracle(name, n, precision):
    """Scoring calls of one to four suffixes: at most 32 rows take the weight-streaming GEMM
    (one float16 plane or two bf16 planes, split K), more rows the tiled one.  mk adds a
    single-row call, ragged column tiles and a one-stage last K split."""
    cfg = S.CONFIGS[name]
    suf = S.suffix_inputs(cfg, 0, n)
    rows = int(suf["lens"].sum())
    say(f"[parity] score_suffixes {name} seed 0, {n} suffix(es), {rows} rows ({precision})")
    sess, src = gpu_session(cfg, 0, precision=precision)
    pre = S.prefix_inputs(cfg, 0)
    ref = O.score_suffixes(src, cfg, pre, suf)
    sess.prefill(pre["vis"], pre["text_ids"])
    got = sess.score_suffixes(suf).cpu().numpy()
    check_suffix_out(got, ref, suf["n_cands"], cfg.dtype, f"{name}/n{n}/{precision}")
    sess.close()


@pytest.mark.parametrize("name,mlp,n,precision", [("m64", 2560, 1, "default"), ("m64", 2560, 2, "split"),
                                                  ("m2", 2560, 1, "default"), ("m2", 2560, 2, "f16_prefill")])
def test_few_rows_norm_split_groups(name, mlp, n, precision):
    """Few-row calls whose down projection splits K more than eight ways on a narrow hidden size
    (1024 or 1536): the norm that sums those partials shares them out over four or two thread
    groups per row, and the scores still meet the bar."""
    cfg = S.with_overrides(S.CONFIGS[name], mlp=mlp)
    suf = S.suffix_inputs(cfg, 0, n)
    say(f"[parity] score_suffixes {name} (MLP {mlp}) seed 0, {n} suffix(es) ({precision})")
    sess, src = gpu_session(cfg, 0, precision=precision)
    pre = S.prefix_inputs(cfg, 0)
    ref = O.score_suffixes(src, cfg, pre, suf)
    sess.prefill(pre["vis"], pre["text_ids"])
    got = sess.score_suffixes(suf).cpu().numpy()
    check_suffix_out(got, ref, suf["n_cands"], cfg.dtype, f"{name}/mlp{mlp}/n{n}/{precision}")
    sess.close()


@pytest.mark.parametrize("precision", ["default", "split"])
def test_fused_swiglu_ragged_columns(precision):
    """A prefill long enough for the fused SwiGLU GEMM (at least 256 tiles: 4708 rows x 7 column
    tiles of 128) on an MLP of 832, so its last column tile is half empty: the prefix's K/V,
    hence the scores, must still meet the bar (one float16 pass by default, two bfloat16 passes
    with "split")."""
    from vlm_shared_prefix_amd import jev as J
    cfg = S.with_overrides(S.CONFIGS["mk"], n_vis=4700)
    say(f"[parity] mk with a {cfg.prefix_len}-row prefix, MLP {cfg.mlp} ({precision})")
    sess, src = gpu_session(cfg, 0, precision=precision)
    pre, suf = S.prefix_inputs(cfg, 0), S.suffix_inputs(cfg, 0)
    ref = O.score_suffixes(src, cfg, pre, suf)
    J.jev_profile_start(sess.model)
    sess.prefill(pre["vis"], pre["text_ids"])
    kinds = J.jev_profile_stop(sess.model)
    assert ("gemm_swiglu_f16" if precision == "default" else "gemm_swiglu") in kinds, sorted(kinds)
    got = sess.score_suffixes(suf).cpu().numpy()
    check_suffix_out(got, ref, suf["n_cands"], cfg.dtype, f"mk/P{cfg.prefix_len}/{precision}")
    sess.close()


@pytest.mark.parametrize("name,seed,precision", [("t1", 1, "f32"), ("m5", 0, "default"), ("m5", 0, "split"),
                                                 ("m5", 0, "f16"), ("m64", 0, "default")])
def test_score_tree_vs_oracle(name, seed, precision):
    cfg = S.CONFIGS[name]
    say(f"[parity] score_tree {name} seed {seed} ({precision})")
    sess, src = gpu_session(cfg, seed, precision="split" if precision == "f32" else precision)
    pre, tree = S.prefix_inputs(cfg, seed), S.tree_inputs(cfg, seed)
    ref = O.score_tree(src, cfg, pre, tree)
    sess.prefill(pre["vis"], pre["text_ids"])
    outs = {}
    for mode in (0, 1, 2):
        score, norm = sess.score_tree(tree, mode)
        outs[mode] = (score.cpu().numpy(), norm.cpu().numpy())
        for k, got in zip(("score", "norm"), outs[mode]):
            valid = np.isfinite(ref[k])
            err = float(np.max(np.abs(got[valid] - ref[k][valid])))
            say(f"  mode {mode} {k}: max |d| = {err:.3e}")
            assert err <= TOL[cfg.dtype], (mode, k, err)
            assert np.all(np.isneginf(got[~valid]))
    sess.close()


@pytest.mark.parametrize("shared", [0, 2, 3])
def test_score_tree_shared_fraction_vs_oracle(shared):
    """Trees whose candidates share their first `shared` of 4 tokens, every schedule."""
    cfg = S.CONFIGS["m5"]
    say(f"[parity] score_tree m5 seed 0, candidates sharing {shared} of {cfg.cand_len_hi} tokens")
    sess, src = gpu_session(cfg, 0)
    pre, tree = S.prefix_inputs(cfg, 0), S.shared_tree_inputs(cfg, 0, shared)
    ref = O.score_tree(src, cfg, pre, tree)
    sess.prefill(pre["vis"], pre["text_ids"])
    for mode in (0, 1, 2):
        score, norm = sess.score_tree(tree, mode)
        for k, got in (("score", score.cpu().numpy()), ("norm", norm.cpu().numpy())):
            err = float(np.max(np.abs(got - ref[k])))
            say(f"  mode {mode} {k}: max |d| = {err:.3e}")
            assert err <= TOL[cfg.dtype], (mode, k, err)
    sess.close()


@pytest.mark.parametrize("name,seed,skip", [("c1", 0, (1,)), ("m2", 0, (0, 1)), ("m7", 0, (1, 0)),
                                            ("m7l", 0, (1, 0))])
def test_block_skipping_vs_oracle(name, seed, skip):
    """Candidate rows bypass the masked blocks, the prefix keeps them ("FastJEV", §2.3, §3.4)."""
    cfg = S.CONFIGS[name]
    say(f"[parity] score_suffixes {name} seed {seed} skipping blocks {skip}")
    sess, src = gpu_session(cfg, seed)
    pre, suf = S.prefix_inputs(cfg, seed), S.suffix_inputs(cfg, seed)
    mask = np.array(skip, dtype=np.uint8)
    ref = O.score_suffixes(src, cfg, pre, suf, skip=mask)
    sess.set_skip(mask)
    sess.prefill(pre["vis"], pre["text_ids"])          # the prefill keeps every block
    got = sess.score_suffixes(suf).cpu().numpy()
    check_suffix_out(got, ref, suf["n_cands"], cfg.dtype, f"{name}/s{seed}/skip{skip}")
    sess.set_skip(None)
    full = O.score_suffixes(src, cfg, pre, suf)
    back = sess.score_suffixes(suf).cpu().numpy()
    check_suffix_out(back, full, suf["n_cands"], cfg.dtype, f"{name}/s{seed}/no skip")
    sess.close()


@pytest.mark.parametrize("name,seed,skip", [("t1", 1, (1,)), ("m5", 0, (0, 1))])
def test_tree_block_skipping_vs_oracle(name, seed, skip):
    cfg = S.CONFIGS[name]
    say(f"[parity] score_tree {name} seed {seed} skipping blocks {skip}")
    sess, src = gpu_session(cfg, seed)
    pre, tree = S.prefix_inputs(cfg, seed), S.tree_inputs(cfg, seed)
    mask = np.array(skip, dtype=np.uint8)
    ref = O.score_tree(src, cfg, pre, tree, skip=mask)
    sess.set_skip(mask)
    sess.prefill(pre["vis"], pre["text_ids"])
    for mode in (0, 2):
        score, norm = sess.score_tree(tree, mode)
        for k, got in (("score", score.cpu().numpy()), ("norm", norm.cpu().numpy())):
            valid = np.isfinite(ref[k])
            err = float(np.max(np.abs(got[valid] - ref[k][valid])))
            say(f"  mode {mode} {k}: max |d| = {err:.3e}")
            assert err <= TOL[cfg.dtype], (mode, k, err)
    sess.close()
