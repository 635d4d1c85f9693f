"""Pins for the CPU oracle (no GPU).

Each test ties a part of the oracle to something other than itself: a closed
form, a textbook or library routine, an independent float64 brute force, or
an invariant the pages state for the method.
"""
import numpy as np
import pytest
import scipy.special as sps

import jev_synth as S
from oracle import brute
from oracle import jev_oracle as O


def _small(name, **kw):
    return S.with_overrides(S.CONFIGS[name], **kw)


# ---------------------------------------------------------------- building blocks
def test_rmsnorm_closed_form():
    g = np.array([1.0, 2.0, -0.5, 3.0], np.float32)
    for c in (0.0, 0.3, -7.0):
        x = np.full(4, c, np.float32)
        expect = g * c / np.sqrt(c * c + 1e-6)
        np.testing.assert_allclose(O.rmsnorm(x, g, 1e-6), expect, rtol=1e-6, atol=1e-7)
    rng = np.random.default_rng(0)
    x = rng.standard_normal(64).astype(np.float32)
    g = rng.standard_normal(64).astype(np.float32)
    # scale invariance (eps negligible)
    np.testing.assert_allclose(O.rmsnorm(3.5 * x, g, 0.0), O.rmsnorm(x, g, 0.0), rtol=1e-5)
    # mean of squares of the normalised vector with unit gain is 1
    y = O.rmsnorm(x, np.ones(64, np.float32), 0.0)
    assert abs(float(np.mean(y.astype(np.float64) ** 2)) - 1.0) < 1e-5


def test_rope_is_complex_rotation():
    """Rotate-half RoPE on (u_t, u_{t+D/2}) equals multiplying u_t + i u_{t+D/2} by exp(i pos w_t)."""
    rng = np.random.default_rng(1)
    D, theta = 16, 1e4
    pos = np.array([0, 1, 5, 100, 8191])
    u = rng.standard_normal((len(pos), 3, D)).astype(np.float32)
    cos, sin = O.rope_cos_sin(pos, D, theta)
    got = O.apply_rope(u, cos, sin)
    w = theta ** (-np.arange(D // 2) * 2.0 / D)
    z = (u[..., :D // 2] + 1j * u[..., D // 2:]).astype(np.complex128)
    z = z * np.exp(1j * pos[:, None, None] * w[None, None, :])
    np.testing.assert_allclose(got[..., :D // 2], z.real, atol=2e-5)
    np.testing.assert_allclose(got[..., D // 2:], z.imag, atol=2e-5)
    # position 0 is the identity, norms are preserved
    np.testing.assert_array_equal(got[0], u[0])
    np.testing.assert_allclose(np.linalg.norm(got, axis=-1), np.linalg.norm(u, axis=-1), rtol=1e-5)


def test_rope_relative_position():
    rng = np.random.default_rng(2)
    D = 64
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    k = rng.standard_normal((1, 1, D)).astype(np.float32)

    def score(i, j):
        ci, si = O.rope_cos_sin(np.array([i]), D, 1e4)
        cj, sj = O.rope_cos_sin(np.array([j]), D, 1e4)
        return float(np.sum(O.apply_rope(q, ci, si) * O.apply_rope(k, cj, sj)))

    assert abs(score(10, 3) - score(110, 103)) < 1e-4
    assert abs(score(7, 7) - float(np.sum(q * k))) < 1e-4


def test_attention_special_cases():
    rng = np.random.default_rng(3)
    Nq, Nk, Hq, Hkv, D = 5, 9, 4, 2, 8
    q = rng.standard_normal((Nq, Hq, D)).astype(np.float32)
    k = rng.standard_normal((Nk, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((Nk, Hkv, D)).astype(np.float32)
    # one visible key -> output is that key's value (for the right kv head)
    vis = np.zeros((Nq, Nk), bool)
    vis[np.arange(Nq), [0, 3, 3, 8, 1]] = True
    o = O.attention(q, k, v, vis)
    for i, j in enumerate([0, 3, 3, 8, 1]):
        for h in range(Hq):
            np.testing.assert_allclose(o[i, h], v[j, h // 2], rtol=1e-6)
    # zero queries -> uniform weights -> mean of the visible values
    vis = np.tril(np.ones((Nq, Nk), bool), k=4)
    o = O.attention(np.zeros_like(q), k, v, vis)
    for i in range(Nq):
        for h in range(Hq):
            np.testing.assert_allclose(o[i, h], v[vis[i], h // 2].mean(axis=0), rtol=1e-5, atol=1e-6)
    # against scipy's softmax on one head
    vis = np.ones((Nq, Nk), bool)
    o = O.attention(q, k, v, vis)
    p = sps.softmax((q[:, 3].astype(np.float64) @ k[:, 1].T.astype(np.float64)) / np.sqrt(D), axis=1)
    np.testing.assert_allclose(o[:, 3], p @ v[:, 1], rtol=1e-5, atol=1e-6)


def test_silu_logsumexp_textbook():
    y = np.linspace(-30, 30, 101).astype(np.float32)
    np.testing.assert_allclose(O.silu(y), y * sps.expit(y.astype(np.float64)), rtol=1e-5, atol=1e-7)
    z = np.random.default_rng(4).standard_normal((3, 50)).astype(np.float32) * 10
    np.testing.assert_allclose(O.logsumexp(z, -1), sps.logsumexp(z.astype(np.float64), axis=-1), rtol=1e-6)


def test_candidate_readout_properties():
    lp = np.log(sps.softmax(np.random.default_rng(5).standard_normal(100))).astype(np.float32)
    cands = np.array([7, 3, 99, 0], np.int32)
    out = O.candidate_readout(lp, cands, 3, 4)
    assert np.isneginf(out[3])
    assert abs(np.exp(out[:3].astype(np.float64)).sum() - 1.0) < 1e-6
    # renormalising full-vocab log-probs == softmax over raw candidate logits (Step 3)
    np.testing.assert_allclose(out[:3], np.log(sps.softmax(lp[cands[:3]].astype(np.float64))), atol=1e-6)
    assert O.candidate_readout(lp, cands, 1, 4)[0] == 0.0
    perm = O.candidate_readout(lp, cands[[2, 0, 1, 3]], 3, 4)
    np.testing.assert_allclose(perm[:3], out[[2, 0, 1]], atol=1e-7)


# ---------------------------------------------------------------- whole-model pins
def test_oracle_matches_fp64_brute_force_c1():
    cfg = S.CONFIGS["c1"]
    ws = S.WeightSource(cfg, 0)
    pre, suf = S.prefix_inputs(cfg, 0), S.suffix_inputs(cfg, 0)
    ref = brute.score_suffixes(cfg, ws, pre, suf)
    got_serial = O.score_suffixes_serial(ws, cfg, pre, suf)
    got = O.score_suffixes(ws, cfg, pre, suf)
    assert np.max(np.abs(got_serial - ref)) < 1e-5
    assert np.max(np.abs(got - ref)) < 1e-5


def test_oracle_matches_fp64_brute_force_two_layers():
    cfg = _small("c1", n_layers=2, n_vis=10, n_text=3, s_max=5, fixed_lens=(5, 1, 3), n_suffix=3,
                 n_cands=4, hidden=64, mlp=96, vocab=200, n_q_heads=4, n_kv_heads=1, head_dim=16)
    ws = S.WeightSource(cfg, 3)
    pre, suf = S.prefix_inputs(cfg, 3), S.suffix_inputs(cfg, 3)
    ref = brute.score_suffixes(cfg, ws, pre, suf)
    assert np.max(np.abs(O.score_suffixes(ws, cfg, pre, suf) - ref)) < 1e-5


def test_oracle_tree_matches_brute_force():
    cfg = S.CONFIGS["t1"]
    ws = S.WeightSource(cfg, 1)
    pre, tree = S.prefix_inputs(cfg, 1), S.tree_inputs(cfg, 1)
    ref = brute.score_tree(cfg, ws, pre, tree)
    got = O.score_tree(ws, cfg, pre, tree)
    got_serial = O.score_tree_serial(ws, cfg, pre, tree)
    for k in ("score", "norm"):
        assert np.max(np.abs(got[k] - ref[k])) < 1e-5
        assert np.max(np.abs(got_serial[k] - ref[k])) < 1e-5


def test_zero_layers_is_textbook_readout():
    """L = 0: out = log-softmax over candidates of RMSNorm(E[last]) W_lm^T."""
    cfg = _small("c1", n_layers=0)
    ws = S.WeightSource(cfg, 0)
    pre, suf = S.prefix_inputs(cfg, 0), S.suffix_inputs(cfg, 0)
    got = O.score_suffixes(ws, cfg, pre, suf)
    g = ws.glob
    for b in range(len(suf["lens"])):
        e = g["embed"][suf["ids"][b, suf["lens"][b] - 1]].astype(np.float64)
        h = g["final_norm"] * e / np.sqrt(np.mean(e * e) + cfg.rms_eps)
        z = g["lm_head"][suf["cands"][b]].astype(np.float64) @ h
        np.testing.assert_allclose(got[b], sps.log_softmax(z), atol=2e-6)


def test_identity_blocks_ignore_context():
    """W_o = W_down = 0 makes every block the identity: the result ignores the prefix."""
    cfg = S.CONFIGS["c1"]
    ws = S.WeightSource(cfg, 0)
    for l in range(cfg.n_layers):
        ws.layer(l)["wo"][:] = 0.0
        ws.layer(l)["w_down"][:] = 0.0
    pre, suf = S.prefix_inputs(cfg, 0), S.suffix_inputs(cfg, 0)
    a = O.score_suffixes(ws, cfg, pre, suf)
    pre2 = S.prefix_inputs(cfg, 9)
    b = O.score_suffixes(ws, cfg, pre2, suf)
    np.testing.assert_array_equal(a, b)
    zero = O.score_suffixes(ws, S.with_overrides(cfg, n_layers=0), pre, suf)
    np.testing.assert_allclose(a, zero, atol=1e-6)


def test_block_skipping_matches_brute_force():
    """Candidate rows bypassing selected blocks ("FastJEV", §2.3, §3.4), prefix at full depth:
    the prefix-once oracle, its serial definition and the fp64 brute force agree, for suffixes
    and trees, and the skip changes the result."""
    cfg = _small("c1", n_layers=3, n_vis=10, n_text=3, s_max=5, fixed_lens=(5, 1, 3), n_suffix=3,
                 n_cands=4, hidden=64, mlp=96, vocab=200, n_q_heads=4, n_kv_heads=1, head_dim=16)
    ws = S.WeightSource(cfg, 5)
    pre, suf = S.prefix_inputs(cfg, 5), S.suffix_inputs(cfg, 5)
    skip = np.array([0, 1, 0], dtype=np.uint8)
    ref = brute.score_suffixes(cfg, ws, pre, suf, skip)
    assert np.max(np.abs(O.score_suffixes(ws, cfg, pre, suf, skip=skip) - ref)) < 1e-5
    assert np.max(np.abs(O.score_suffixes_serial(ws, cfg, pre, suf, skip) - ref)) < 1e-5
    assert np.max(np.abs(O.score_suffixes(ws, cfg, pre, suf) - ref)) > 1e-3
    tcfg = S.CONFIGS["t1"]
    tws = S.WeightSource(tcfg, 1)
    tpre, tree = S.prefix_inputs(tcfg, 1), S.tree_inputs(tcfg, 1)
    tskip = np.array([1], dtype=np.uint8)
    tref = brute.score_tree(tcfg, tws, tpre, tree, tskip)
    got = O.score_tree(tws, tcfg, tpre, tree, skip=tskip)
    got_serial = O.score_tree_serial(tws, tcfg, tpre, tree, tskip)
    for k in ("score", "norm"):
        assert np.max(np.abs(got[k] - tref[k])) < 1e-5
        assert np.max(np.abs(got_serial[k] - tref[k])) < 1e-5


def test_skipping_every_block_is_textbook_readout():
    """All blocks bypassed: the candidate row is its own embedding, so the answer is
    log-softmax over the candidates of RMSNorm(E[last]) W_lm^T, whatever the prefix."""
    cfg = S.CONFIGS["c1"]
    ws = S.WeightSource(cfg, 0)
    pre, suf = S.prefix_inputs(cfg, 0), S.suffix_inputs(cfg, 0)
    got = O.score_suffixes(ws, cfg, pre, suf, skip=np.ones(cfg.n_layers, np.uint8))
    g = ws.glob
    for b in range(len(suf["lens"])):
        e = g["embed"][suf["ids"][b, suf["lens"][b] - 1]].astype(np.float64)
        h = g["final_norm"] * e / np.sqrt(np.mean(e * e) + cfg.rms_eps)
        z = g["lm_head"][suf["cands"][b]].astype(np.float64) @ h
        np.testing.assert_allclose(got[b], sps.log_softmax(z), atol=2e-6)
    none = O.score_suffixes(ws, cfg, pre, suf, skip=np.zeros(cfg.n_layers, np.uint8))
    np.testing.assert_array_equal(none, O.score_suffixes(ws, cfg, pre, suf))


# ---------------------------------------------------------------- method invariants
@pytest.mark.parametrize("seed", [0, 1])
def test_segments_match_brute_force(seed):
    """One question over several images (Ochevid, One question, multiple images): each
    image's answer is the plain definition over that image's prefix alone, checked against
    the float64 brute force; images of different sizes, several suffixes per image in a
    shuffled order, and an image with no suffix."""
    cfg = S.CONFIGS["mi1"]
    src = S.WeightSource(cfg, seed)
    inp = S.images_inputs(cfg, seed)
    images = inp["images"] + [S.images_inputs(cfg, seed + 5)["images"][0]]
    suf = S.suffix_inputs(_small("c1", n_suffix=5, fixed_lens=(3, 8, 1, 6, 5)), seed)
    seg = np.array([2, 0, 2, 1, 0], np.int32)       # image 3 gets no suffix
    got = O.score_segments(src, cfg, images, suf, seg)
    ref = brute.score_segments(cfg, src, images, suf, seg)
    np.testing.assert_allclose(got, ref, atol=2e-5)
    # the one-question layout of the generator: the same question of every image
    got1 = O.score_segments(src, cfg, inp["images"], inp["suf"], inp["seg"])
    ref1 = brute.score_segments(cfg, src, inp["images"], inp["suf"], inp["seg"])
    np.testing.assert_allclose(got1, ref1, atol=2e-5)
    assert np.ptp(got1[:, 0]) > 1e-4                   # different images, different answers


def test_one_segment_is_the_single_prefix_call():
    cfg = S.CONFIGS["mi1"]
    src = S.WeightSource(cfg, 0)
    inp = S.images_inputs(cfg, 0)
    suf = S.suffix_inputs(_small("c1", n_suffix=3, fixed_lens=(2, 8, 4)), 0)
    np.testing.assert_array_equal(O.score_segments(src, cfg, inp["images"][:1], suf, np.zeros(3, np.int32)),
                                  O.score_suffixes(src, cfg, inp["images"][0], suf))


@pytest.fixture(scope="module")
def m2_small():
    cfg = _small("m2", hidden=256, n_q_heads=2, n_kv_heads=1, head_dim=128, mlp=256, vocab=512)
    ws = S.WeightSource(cfg, 0)
    return cfg, ws, S.prefix_inputs(cfg, 0), S.suffix_inputs(cfg, 0)


def test_shared_equals_serial(m2_small):
    """Shared-prefix answers equal serial execution (Ochevid, Evidence)."""
    cfg, ws, pre, suf = m2_small
    a = O.score_suffixes(ws, cfg, pre, suf)
    b = O.score_suffixes_serial(ws, cfg, pre, suf)
    assert np.max(np.abs(a - b)) < 2e-6


def test_order_padding_isolation(m2_small):
    """Question order, added questions, pad width/content and other questions do not matter."""
    cfg, ws, pre, suf = m2_small
    base = O.score_suffixes(ws, cfg, pre, suf)
    perm = np.random.default_rng(0).permutation(len(suf["lens"]))
    s2 = {k: v[perm] for k, v in suf.items()}
    np.testing.assert_array_equal(O.score_suffixes(ws, cfg, pre, s2), base[perm])
    wide = dict(suf)
    wide["ids"] = np.concatenate([suf["ids"], np.full((len(suf["lens"]), 9), 17, np.int32)], axis=1)
    np.testing.assert_array_equal(O.score_suffixes(ws, cfg, pre, wide), base)
    other = {k: v.copy() for k, v in suf.items()}
    other["ids"][0, :] = (other["ids"][0, :] + 1) % cfg.vocab
    got = O.score_suffixes(ws, cfg, pre, other)
    np.testing.assert_array_equal(got[1:], base[1:])
    assert np.any(got[0] != base[0])


def test_prefix_suffix_split(m2_small):
    """Moving the first suffix token into the prefix leaves that question's answer unchanged."""
    cfg, ws, pre, suf = m2_small
    b = int(np.argmax(suf["lens"]))
    base = O.score_suffixes(ws, cfg, pre, suf)[b]
    pre2 = {"vis": pre["vis"], "text_ids": np.concatenate([pre["text_ids"], suf["ids"][b, :1]])}
    cfg2 = S.with_overrides(cfg, n_text=cfg.n_text + 1)
    one = {"ids": suf["ids"][b:b + 1, 1:], "lens": suf["lens"][b:b + 1] - 1,
           "cands": suf["cands"][b:b + 1], "n_cands": suf["n_cands"][b:b + 1]}
    got = O.score_suffixes(ws, cfg2, pre2, one)[0]
    assert np.max(np.abs(got - base)) < 2e-6


def test_duplicates_and_single_candidate(m2_small):
    cfg, ws, pre, suf = m2_small
    d = {k: v.copy() for k, v in suf.items()}
    d["ids"][1], d["lens"][1], d["cands"][1] = d["ids"][0], d["lens"][0], d["cands"][0]
    d["cands"][3, 1] = d["cands"][3, 0]
    d["n_cands"][2] = 1
    out = O.score_suffixes(ws, cfg, pre, d)
    np.testing.assert_array_equal(out[1], out[0])
    assert out[3, 0] == out[3, 1]
    assert out[2, 0] == 0.0 and np.all(np.isneginf(out[2, 1:]))


def test_tree_single_token_equals_suffix_readout():
    """One-token candidates: the renormalised tree score is the suffix readout."""
    cfg = S.with_overrides(S.CONFIGS["t1"], cand_len_lo=1, cand_len_hi=1, overlap=False)
    ws = S.WeightSource(cfg, 2)
    pre, tree = S.prefix_inputs(cfg, 2), S.tree_inputs(cfg, 2)
    got = O.score_tree(ws, cfg, pre, tree)
    Q, C, _ = tree["cand_tok"].shape
    suf = {"ids": tree["stem_ids"], "lens": tree["stem_lens"],
           "cands": tree["cand_tok"][:, :, 0].copy(), "n_cands": tree["n_cands"]}
    out = O.score_suffixes(ws, cfg, pre, suf)
    np.testing.assert_allclose(got["norm"], out, atol=2e-6)


def test_margins_and_argmax():
    out = np.array([[-0.1, -2.4, -np.inf], [-0.7, -0.7, -np.inf], [0.0, -np.inf, -np.inf]], np.float32)
    n = np.array([2, 2, 1])
    assert list(O.argmax_first(out, n)) == [0, 0, 0]
    m = O.margins(out, n)
    assert abs(m[0] - 2.3) < 1e-6 and m[1] == 0.0 and np.isinf(m[2])


# ---------------------------------------------------------------- generator
def test_generator_deterministic_and_bf16_exact():
    cfg = S.CONFIGS["m2"]
    a = S.weights_layer(cfg, 5, 1)
    b = S.weights_layer(cfg, 5, 1)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
        S.to_bf16_bits(a[k])            # raises unless exactly representable
    c = S.weights_layer(cfg, 6, 1)
    assert not np.array_equal(a["wq"], c["wq"])
    # chunked draws do not depend on the thread count
    g1 = S._normal((9000, 8), 1, 0, 0, 1.0, 0.0, "bf16")
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(1) as ex:
        g2 = S._normal((9000, 8), 1, 0, 0, 1.0, 0.0, "bf16", pool=ex)
    np.testing.assert_array_equal(g1, g2)
    # gains are 1 + 0.02 N(0,1); matrices 0.02 N(0,1)
    assert abs(float(a["attn_norm"].mean()) - 1.0) < 0.01
    assert abs(float(a["wq"].std()) - 0.02) < 0.001


def test_round_bf16_ties_to_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5], np.float32)
    r = S.round_bf16(x)
    np.testing.assert_array_equal(r, np.array([1.0, 1.0, 1.0 + 4 * 2 ** -8, 1.0, -2.5], np.float32))


def test_suffix_pool_prefix_property():
    cfg = S.CONFIGS["c4"]
    big = S.suffix_inputs(cfg, 0)
    small = S.suffix_inputs(cfg, 0, n=8)
    for k in small:
        np.testing.assert_array_equal(small[k], big[k][:8])
    assert big["lens"].min() >= 8 and big["lens"].max() <= 24
