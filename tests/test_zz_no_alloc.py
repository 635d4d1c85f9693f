"""The allocation-free scoring entry point (static device scratch) against jev_score_suffixes,
through the C ABI: two calls in a row, the second on a smaller request."""
import numpy as np
import pytest
import torch

import jev_synth as S
from oracle import jev_oracle as O
from tests.gpu_common import check_suffix_out, gpu_session, say

pytestmark = pytest.mark.gpu


def _first(suf, n):
    return {k: (v[:n] if isinstance(v, np.ndarray) and v.ndim >= 1 else v) for k, v in suf.items()}


@pytest.mark.parametrize("name", ["m7", "m2"])
def test_noalloc_matches_workspace_call(name):
    from vlm_shared_prefix_amd import jev as J
    cfg = S.CONFIGS[name]
    say(f"[no-alloc] {name} seed 0: static scratch of {J.jev_static_scratch_bytes()} bytes")
    sess, src = gpu_session(cfg, 0)
    pre, suf = S.prefix_inputs(cfg, 0), S.suffix_inputs(cfg, 0)
    sess.prefill(pre["vis"], pre["text_ids"])
    B = int(suf["lens"].shape[0])
    for n in (B, max(1, B // 2)):
        s = _first(suf, n)
        ref = O.score_suffixes(src, cfg, pre, s)
        want = sess.score_suffixes(s).cpu().numpy()
        out = torch.full(s["cands"].shape, float("nan"), dtype=torch.float32, device="cuda:0")
        J.jev_score_suffixes_noalloc(sess.prefix, s["ids"], s["lens"], s["cands"], s["n_cands"], out)
        got = out.cpu().numpy()
        say(f"  {n} suffixes: identical to the workspace call: {np.array_equal(got, want)}")
        assert np.array_equal(got, want)
        check_suffix_out(got, ref, s["n_cands"], cfg.dtype, f"{name} no-alloc, {n} suffixes")
    sess.close()


def test_noalloc_rejects_oversized_request():
    """A request whose workspace exceeds the scratch is refused before anything is enqueued."""
    from vlm_shared_prefix_amd import jev as J
    cfg = S.CONFIGS["m2"]
    sess, _ = gpu_session(cfg, 0)
    pre = S.prefix_inputs(cfg, 0)
    sess.prefill(pre["vis"], pre["text_ids"])
    B, L = 256, 256   # 65536 rows
    ids = np.zeros((B, L), np.int32)
    lens = np.full(B, L, np.int32)
    cands = np.zeros((B, 2), np.int32)
    n = np.full(B, 2, np.int32)
    need = J.jev_workspace_bytes(sess.model, sess.P, B * L, B, 2 * B)
    assert need > J.jev_static_scratch_bytes()
    out = torch.empty((B, 2), dtype=torch.float32, device="cuda:0")
    with pytest.raises(J.JevError) as e:
        J.jev_score_suffixes_noalloc(sess.prefix, ids, lens, cands, n, out)
    assert e.value.code == J.JEV_E_WORKSPACE
    sess.close()
