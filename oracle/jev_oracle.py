"""CPU oracle for shared-prefix candidate scoring.  TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The product path (the HIP library and its Python binding) never
does, and this module never imports the product path.  Inputs come from
`jev_synth`, which draws numbers and holds none of the arithmetic below.

What is computed (plain float32 NumPy, one operation at a time):

The method scores many question suffixes against one prefix whose KV cache is
computed once, and its claim is that the answers equal the ones obtained by
running every question separately over the full prefix ("Ochevid Jev-VL 2B",
Evidence: all tested answers matched original serial execution; "FastJEV",
TL;DR and §3.2-§3.3: sharing is valid when histories, positions and masks are
identical).  So the oracle is that plain definition: for every question, an
independent causal decoder forward over prefix ‖ suffix, full-vocabulary
logits at the question's last valid position, and the candidate readout of
"How to Deploy Visual Jev ...", Step 3 (softmax over the candidate logits),
taken in log space.

Decoder layer (pre-norm, rotate-half RoPE, grouped-query attention, SwiGLU):
    a  = RMSNorm(x; g1)                  RMSNorm(x; g) = g * x / sqrt(mean(x^2) + eps)
    q, k, v = a Wq^T, a Wk^T, a Wv^T     heads of width D; q head h uses kv head h // G
    q, k  <- RoPE at the row's position  (pair t with t + D/2, angle pos * theta^(-2t/D))
    o_i   = sum_j softmax_j(q_i . k_j / sqrt(D)) v_j   over the keys row i may see
    x    <- x + concat_h(o) Wo^T
    m     = RMSNorm(x; g2)
    x    <- x + (silu(m Wg^T) * (m Wu^T)) Wd^T          silu(y) = y / (1 + exp(-y))
Readout at the last valid row:  z = RMSNorm(x; g_f) W_lm^T (all V logits);
    l = z - logsumexp(z);  out_c = l[c] - logsumexp_{c' in C_b} l[c'].
Tree workload ("FastJEV" §3.3): a candidate w = (w_0..w_{K-1}) of question q is
scored as sum_k l_{row(k)}[w_k] over the sequence prefix ‖ stem_q ‖ w_0..w_{K-2},
where row(k) is the row right before w_k; `norm` renormalises those scores
over the question's candidates.

Readings where the pages are silent (each listed in the design notes):
positions are 0..P-1 for the prefix and P+j for suffix token j; visual rows
come first, then prefix text; RoPE tables are computed in float64 and used in
float32; the softmax scale is 1/sqrt(D); no biases; the LM head is untied.

Two ways of running the same definition are provided:
  * `score_suffixes_serial` / `score_tree_serial`: the definition itself, one
    full forward over prefix ‖ suffix per question (small configs only);
  * `score_suffixes` / `score_tree`: the prefix rows are computed once, layer
    by layer, and every question's rows attend to that layer's prefix K/V.
    Prefix rows never see later rows (causality), so the two are the same
    computation; the tests check that they agree.  This variant keeps one
    layer's weights resident, which makes the 2B/7B shapes affordable.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

F32 = np.float32


# ----------------------------------------------------------------------------
# building blocks
# ----------------------------------------------------------------------------
def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """g * x / sqrt(mean(x^2) + eps) over the last axis, float32."""
    x = x.astype(F32, copy=False)
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=F32)
    return (x / np.sqrt(ms + F32(eps))) * g.astype(F32)


def rope_cos_sin(positions: np.ndarray, head_dim: int, theta: float):
    """cos/sin tables [N, D/2]: angle = pos * theta^(-2t/D), computed in float64."""
    half = head_dim // 2
    t = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * t / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(F32), np.sin(ang).astype(F32)


def apply_rope(u: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE on u [N, heads, D]: (u_t, u_{t+D/2}) rotated by the row's angle_t."""
    half = u.shape[-1] // 2
    a, b = u[..., :half], u[..., half:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1).astype(F32)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, visible: np.ndarray) -> np.ndarray:
    """Grouped-query softmax attention.

    q [Nq, Hq, D], k/v [Nk, Hkv, D], visible [Nq, Nk] bool.  q head h reads kv
    head h // (Hq/Hkv).  Every query row must see at least one key.
    """
    Nq, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = F32(1.0 / np.sqrt(D))
    out = np.empty_like(q, dtype=F32)
    neg = np.where(visible, F32(0.0), F32(-np.inf)).astype(F32)
    for h in range(Hq):
        kv = h // G
        s = (q[:, h, :] @ k[:, kv, :].T) * scale + neg
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, kv, :]
    return out


def silu(y: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return (y / (F32(1.0) + np.exp(-y))).astype(F32)


def logsumexp(z: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(z, axis=axis, keepdims=True)
    return (m + np.log(np.sum(np.exp(z - m), axis=axis, keepdims=True))).squeeze(axis)


def layer_forward(W: Dict[str, np.ndarray], cfg, x: np.ndarray, positions: np.ndarray,
                  ctx_k: Optional[np.ndarray] = None, ctx_v: Optional[np.ndarray] = None):
    """One decoder layer over rows x [N,H] at `positions`.

    The rows attend causally to each other and to every row of an optional
    context (ctx_k/ctx_v [Nc,Hkv,D], already rotated), which precedes them.
    Returns (x_out, k, v) with this layer's rotated k and v of the rows.
    """
    N = x.shape[0]
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    a = rmsnorm(x, W["attn_norm"], cfg.rms_eps)
    q = (a @ W["wq"].T).reshape(N, Hq, D)
    k = (a @ W["wk"].T).reshape(N, Hkv, D)
    v = (a @ W["wv"].T).reshape(N, Hkv, D)
    cos, sin = rope_cos_sin(positions, D, cfg.rope_theta)
    q = apply_rope(q, cos, sin)
    k = apply_rope(k, cos, sin)
    nc = 0 if ctx_k is None else ctx_k.shape[0]
    if nc:
        K = np.concatenate([ctx_k, k], axis=0)
        V = np.concatenate([ctx_v, v], axis=0)
    else:
        K, V = k, v
    visible = np.ones((N, nc + N), dtype=bool)
    visible[:, nc:] = np.tril(np.ones((N, N), dtype=bool))
    o = attention(q, K, V, visible)
    x = x + o.reshape(N, Hq * D) @ W["wo"].T
    m = rmsnorm(x, W["mlp_norm"], cfg.rms_eps)
    x = x + (silu(m @ W["w_gate"].T) * (m @ W["w_up"].T)) @ W["w_down"].T
    return x.astype(F32), k, v


def log_probs(ws, cfg, h_last: np.ndarray) -> np.ndarray:
    """Full-vocabulary log-probabilities for final hidden rows [N,H] -> [N,V]."""
    g = ws.glob
    z = rmsnorm(h_last, g["final_norm"], cfg.rms_eps) @ g["lm_head"].T
    return (z - logsumexp(z, axis=-1)[:, None]).astype(F32)


def candidate_readout(lp_row: np.ndarray, cands: np.ndarray, n: int, c_max: int) -> np.ndarray:
    """out_c = l[c] - logsumexp over the first n candidates; pad slots are -inf."""
    out = np.full(c_max, -np.inf, dtype=F32)
    sel = lp_row[cands[:n]].astype(F32)
    out[:n] = sel - logsumexp(sel)
    return out


# ----------------------------------------------------------------------------
# inputs -> rows
# ----------------------------------------------------------------------------
def prefix_rows(ws, cfg, prefix: Dict[str, np.ndarray]) -> np.ndarray:
    """Visual rows first (given embeddings), then the text prefix's embedding rows."""
    E = ws.glob["embed"]
    rows = [prefix["vis"].astype(F32)]
    if len(prefix["text_ids"]):
        rows.append(E[prefix["text_ids"]])
    return np.concatenate(rows, axis=0) if rows else np.zeros((0, cfg.hidden), F32)


def forward_sequence(ws, cfg, x0: np.ndarray, skip=None, bypass_from: int = 0) -> np.ndarray:
    """All layers over one sequence at positions 0..N-1 (plain causal LM).

    Block skipping ("FastJEV", §2.3 and §3.4): where skip[l] is set, rows from
    bypass_from on (the candidate rows) pass block l unchanged, while the rows
    before them (the shared context) run it.  Only rows that also skip block l
    could read the bypassed rows' keys there, so computing the block for every
    row and then restoring the bypassed rows is exact.
    """
    x = x0.astype(F32)
    pos = np.arange(x.shape[0])
    for l in range(cfg.n_layers):
        x_new, _, _ = layer_forward(ws.layer(l), cfg, x, pos)
        if skip is not None and skip[l]:
            x_new[bypass_from:] = x[bypass_from:]
        x = x_new
    return x


# ----------------------------------------------------------------------------
# scoring: the definition (serial) and the prefix-once variant
# ----------------------------------------------------------------------------
def score_suffixes_serial(ws, cfg, prefix, suf, skip=None) -> np.ndarray:
    """out[b, c]: one independent full forward over prefix ‖ suffix_b per question
    (suffix rows bypass the blocks marked in skip)."""
    P = prefix_rows(ws, cfg, prefix)
    E = ws.glob["embed"]
    B, C = suf["cands"].shape
    out = np.full((B, C), -np.inf, dtype=F32)
    for b in range(B):
        L = int(suf["lens"][b])
        x = np.concatenate([P, E[suf["ids"][b, :L]]], axis=0)
        h = forward_sequence(ws, cfg, x, skip, P.shape[0])
        lp = log_probs(ws, cfg, h[-1:])[0]
        out[b] = candidate_readout(lp, suf["cands"][b], int(suf["n_cands"][b]), C)
    return out


def _run_groups(ws, cfg, prefix, groups: List[np.ndarray], free_layers: bool = False, skip=None):
    """Layer-major forward of the prefix once plus independent row groups over it.

    groups[i] = token ids of one independent continuation (positions P..).
    Where skip[l] is set the groups pass block l unchanged; the prefix runs every
    block ("FastJEV", §3.4: the shared context keeps all layers).
    Returns the final hidden rows of every group.
    """
    E = ws.glob["embed"]
    xp = prefix_rows(ws, cfg, prefix)
    Pn = xp.shape[0]
    pos_p = np.arange(Pn)
    xs = [E[g] for g in groups]
    for l in range(cfg.n_layers):
        W = ws.layer(l)
        kp = vp = None
        if Pn:
            xp, kp, vp = layer_forward(W, cfg, xp, pos_p)
        if skip is None or not skip[l]:
            for i, g in enumerate(groups):
                pos = Pn + np.arange(len(g))
                xs[i], _, _ = layer_forward(W, cfg, xs[i], pos, kp, vp)
        if free_layers:
            ws.drop_layer(l)
    return xs


def score_suffixes(ws, cfg, prefix, suf, free_layers: bool = False,
                   return_full: bool = False, skip=None):
    """Same definition as score_suffixes_serial with the prefix rows computed once."""
    B, C = suf["cands"].shape
    groups = [suf["ids"][b, :int(suf["lens"][b])] for b in range(B)]
    xs = _run_groups(ws, cfg, prefix, groups, free_layers, skip)
    out = np.full((B, C), -np.inf, dtype=F32)
    lps = []
    for b in range(B):
        lp = log_probs(ws, cfg, xs[b][-1:])[0]
        out[b] = candidate_readout(lp, suf["cands"][b], int(suf["n_cands"][b]), C)
        if return_full:
            lps.append(lp)
    return (out, np.stack(lps)) if return_full else out


def score_segments(ws, cfg, images, suf, seg) -> np.ndarray:
    """One question over several images ("Ochevid Jev-VL 2B", One question, multiple
    images): each image goes through the model on its own and is answered separately,
    nothing passing between images.  Suffix b continues image seg[b] alone, so out[b] is
    the single-prefix definition over that image's prefix: score_suffixes with
    prefix = images[seg[b]] and the suffixes of that image."""
    seg = np.asarray(seg)
    B, C = suf["cands"].shape
    out = np.full((B, C), -np.inf, dtype=F32)
    for i, pre in enumerate(images):
        sel = np.nonzero(seg == i)[0]
        if len(sel):
            out[sel] = score_suffixes(ws, cfg, pre, {k: v[sel] for k, v in suf.items()})
    return out


def _tree_sequences(tree):
    """Per (question, candidate): the fed ids stem ‖ w_0..w_{K-2} and the targets w."""
    Q, C, _ = tree["cand_tok"].shape
    seqs = {}
    for q in range(Q):
        s = int(tree["stem_lens"][q])
        stem = tree["stem_ids"][q, :s]
        for c in range(int(tree["n_cands"][q])):
            K = int(tree["cand_lens"][q, c])
            w = tree["cand_tok"][q, c, :K]
            seqs[(q, c)] = (np.concatenate([stem, w[:K - 1]]).astype(np.int32), w, s)
    return seqs


def _tree_finish(tree, lp_rows) -> Dict[str, np.ndarray]:
    Q, C, _ = tree["cand_tok"].shape
    score = np.full((Q, C), -np.inf, dtype=F32)
    norm = np.full((Q, C), -np.inf, dtype=F32)
    for (q, c), (w, lp) in lp_rows.items():
        # lp[k] holds the log-probs of the row right before w_k (fed row s-1+k)
        score[q, c] = np.sum([lp[k, w[k]] for k in range(len(w))], dtype=np.float64)
    for q in range(Q):
        n = int(tree["n_cands"][q])
        norm[q, :n] = score[q, :n] - logsumexp(score[q, :n])
    return {"score": score, "norm": norm}


def score_tree_serial(ws, cfg, prefix, tree, skip=None) -> Dict[str, np.ndarray]:
    """Flat definition: every candidate its own full forward over prefix ‖ stem ‖ w[:-1]
    (stem and candidate rows bypass the blocks marked in skip)."""
    P = prefix_rows(ws, cfg, prefix)
    E = ws.glob["embed"]
    rows = {}
    for key, (fed, w, s) in _tree_sequences(tree).items():
        h = forward_sequence(ws, cfg, np.concatenate([P, E[fed]], axis=0), skip, P.shape[0])
        rows[key] = (w, log_probs(ws, cfg, h[h.shape[0] - len(w):]))
    return _tree_finish(tree, rows)


def score_tree(ws, cfg, prefix, tree, free_layers: bool = False, skip=None) -> Dict[str, np.ndarray]:
    """Flat definition with the prefix rows computed once (see module docstring)."""
    seqs = _tree_sequences(tree)
    keys = list(seqs.keys())
    xs = _run_groups(ws, cfg, prefix, [seqs[k][0] for k in keys], free_layers, skip)
    rows = {}
    for key, x in zip(keys, xs):
        fed, w, s = seqs[key]
        rows[key] = (w, log_probs(ws, cfg, x[x.shape[0] - len(w):]))
    return _tree_finish(tree, rows)


def margins(out: np.ndarray, n_cands: np.ndarray) -> np.ndarray:
    """Top-1 minus top-2 of each row over its valid candidates (inf when only one)."""
    m = np.full(out.shape[0], np.inf)
    for b in range(out.shape[0]):
        n = int(n_cands[b])
        if n >= 2:
            s = np.sort(out[b, :n].astype(np.float64))[::-1]
            m[b] = s[0] - s[1]
    return m


def argmax_first(out: np.ndarray, n_cands: np.ndarray) -> np.ndarray:
    """Index of the best candidate; ties go to the first (lowest index)."""
    return np.array([int(np.argmax(out[b, :int(n_cands[b])])) for b in range(out.shape[0])])
