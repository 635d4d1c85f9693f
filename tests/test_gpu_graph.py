"""HIP-graph replay of the scoring calls: the launch-only entry points captured into a graph.

Each replay must reproduce the eager call bit for bit (same kernels, same inputs, no
atomics) and so stay within the oracle's bar; the program's own eager work (another
request on another workspace) and synchronisations run between the replays.
"""
import numpy as np
import pytest
import torch

import jev_synth as S
from oracle import jev_oracle as O
from tests.gpu_common import TOL, check_suffix_out, gpu_session, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,seed,precision", [("m7", 0, "default"), ("m2", 0, "split"), ("c1", 0, "f32")])
def test_graph_replay_suffixes(name, seed, precision):
    cfg = S.CONFIGS[name]
    say(f"[graph] score_suffixes {name} seed {seed} ({precision})")
    sess, src = gpu_session(cfg, seed, precision="split" if precision == "f32" else precision)
    pre, suf = S.prefix_inputs(cfg, seed), S.suffix_inputs(cfg, seed)
    other = S.suffix_inputs(cfg, seed + 7)
    ref = O.score_suffixes(src, cfg, pre, suf)
    sess.prefill(pre["vis"], pre["text_ids"])
    eager = sess.score_suffixes(suf).clone()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    cap = sess.capture_score_suffixes(suf, stream)
    for i in range(4):
        cap.outs[0].fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            cap.replay()
        stream.synchronize()
        got = cap.outs[0]
        assert torch.equal(got, eager), f"replay {i} differs from the eager call"
        check_suffix_out(got.cpu().numpy(), ref, suf["n_cands"], cfg.dtype, f"{name}/replay{i}")
        sess.score_suffixes(other)          # eager work on the session's own workspace
        torch.cuda.synchronize()
    sess.close()


@pytest.mark.parametrize("name,seed,mode", [("m5", 0, 0), ("t1", 1, 2)])
def test_graph_replay_tree(name, seed, mode):
    cfg = S.CONFIGS[name]
    say(f"[graph] score_tree {name} seed {seed} mode {mode}")
    sess, src = gpu_session(cfg, seed, precision="split" if cfg.dtype == "f32" else "default")
    pre, tree = S.prefix_inputs(cfg, seed), S.tree_inputs(cfg, seed)
    ref = O.score_tree(src, cfg, pre, tree)
    sess.prefill(pre["vis"], pre["text_ids"])
    e_score, e_norm = (t.clone() for t in sess.score_tree(tree, mode))
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    cap = sess.capture_score_tree(tree, mode, stream)
    for i in range(3):
        for t in cap.outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            cap.replay()
        stream.synchronize()
        assert torch.equal(cap.outs[0], e_score) and torch.equal(cap.outs[1], e_norm), f"replay {i}"
        for k, got in zip(("score", "norm"), cap.outs):
            valid = np.isfinite(ref[k])
            err = float(np.max(np.abs(got.cpu().numpy()[valid] - ref[k][valid])))
            say(f"  replay {i} {k}: max |d| = {err:.3e}")
            assert err <= TOL[cfg.dtype], (i, k, err)
        sess.score_tree(tree, 1 if mode != 1 else 0)   # eager work on the session's own workspace
        torch.cuda.synchronize()
    sess.close()
