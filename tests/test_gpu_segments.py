"""GPU parity of segmented prefixes: one question over several images.

Every image's prefix sits in one store and is prefilled in one batched forward;
each suffix continues one image and must equal the plain definition over that
image alone ("Ochevid Jev-VL 2B", One question, multiple images).  Images of
mixed sizes put segment edges inside 64-key tiles and 128-row attention tiles.
"""
import numpy as np
import pytest

import jev_synth as S
from oracle import jev_oracle as O
from tests.gpu_common import check_suffix_out, gpu_session, say

pytestmark = pytest.mark.gpu


def _mixed_suffixes(cfg, seed, n_images, order):
    """Several suffixes per image: lengths 1..S_max, segment of row b = order[b]."""
    base = S.with_overrides(S.CONFIGS["m7"] if cfg.dtype == "bf16" else S.CONFIGS["c1"],
                            vocab=cfg.vocab, n_suffix=len(order), len_lo=1, len_hi=cfg.s_max, s_max=cfg.s_max,
                            n_cands=cfg.n_cands, fixed_lens=None)
    return S.suffix_inputs(base, seed), np.asarray(order, np.int32)


@pytest.mark.parametrize("name,seed,precision", [("mi1", 0, "f32"), ("mi7", 0, "default"), ("mi7", 1, "split"),
                                                 ("mi7", 2, "f16")])
def test_segments_vs_oracle(name, seed, precision):
    cfg = S.CONFIGS[name]
    say(f"[parity] segments {name} seed {seed} ({precision})")
    sess, src = gpu_session(cfg, seed, precision="split" if precision == "f32" else precision)
    inp = S.images_inputs(cfg, seed)
    images = inp["images"]
    say(f"  image prefix lengths {inp['seg_lens'].tolist()}, question length {int(inp['suf']['lens'][0])}")
    sess.prefill_segments(images)
    # the one-question layout: row i asks the question of image i
    ref = O.score_segments(src, cfg, images, inp["suf"], inp["seg"])
    got = sess.score_segments(inp["seg"], inp["suf"]).cpu().numpy()
    check_suffix_out(got, ref, inp["suf"]["n_cands"], cfg.dtype, f"{name}/s{seed}/one question")
    # several suffixes per image, grouped by image, then in a shuffled order
    for order in ([0, 0, 0, 1, 1, 2, 2, 2, 2], [2, 0, 1, 2, 0, 1, 0]):
        suf, seg = _mixed_suffixes(cfg, seed, len(images), order)
        ref = O.score_segments(src, cfg, images, suf, seg)
        got = sess.score_segments(seg, suf).cpu().numpy()
        check_suffix_out(got, ref, suf["n_cands"], cfg.dtype, f"{name}/s{seed}/order {order}")
    sess.close()


@pytest.mark.parametrize("name,seed", [("mi7", 0), ("mi1", 1)])
def test_segments_match_separate_prefixes(name, seed):
    """The batched segmented prefill and scoring against one plain prefix per image on the
    same device path (each image prefilled and scored on its own)."""
    cfg = S.CONFIGS[name]
    say(f"[parity] segments vs separate prefixes {name} seed {seed}")
    sess, src = gpu_session(cfg, seed, precision="split" if cfg.dtype == "f32" else "default")
    inp = S.images_inputs(cfg, seed)
    sess.prefill_segments(inp["images"])
    got = sess.score_segments(inp["seg"], inp["suf"]).cpu().numpy()
    tol = 1e-4 if cfg.dtype == "f32" else 2e-2
    for i, im in enumerate(inp["images"]):
        sess.prefill(im["vis"], im["text_ids"])
        one = {k: v[i:i + 1] for k, v in inp["suf"].items()}
        alone = sess.score_suffixes(one).cpu().numpy()
        err = float(np.max(np.abs(alone[0] - got[i])))
        say(f"  image {i}: max |d| vs its own prefix = {err:.3e}")
        assert err <= tol, (i, err)
    sess.close()


@pytest.mark.parametrize("name,seed", [("mi1", 2), ("mi7", 3)])
def test_segments_edge_cases(name, seed):
    """Degenerate segments: one with no rows at all (its suffix sees only its own rows, the
    P = 0 case) and one of text only; suffixes of length 1 included."""
    cfg = S.CONFIGS[name]
    say(f"[parity] segment edge cases {name} seed {seed}")
    sess, src = gpu_session(cfg, seed, precision="split" if cfg.dtype == "f32" else "default")
    inp = S.images_inputs(cfg, seed)
    H = cfg.hidden
    empty = np.zeros((0, H), np.float32)
    images = [inp["images"][0], {"vis": empty, "text_ids": np.zeros(0, np.int32)},
              {"vis": empty, "text_ids": inp["images"][1]["text_ids"]}, inp["images"][2]]
    sess.prefill_segments(images)
    suf, seg = _mixed_suffixes(cfg, seed, len(images), [0, 1, 1, 2, 3, 3])
    suf["lens"][1] = 1
    ref = O.score_segments(src, cfg, images, suf, seg)
    got = sess.score_segments(seg, suf).cpu().numpy()
    check_suffix_out(got, ref, suf["n_cands"], cfg.dtype, f"{name}/s{seed}/edge segments")
    sess.close()
