"""Float64 brute force for tiny configurations.  TEST INFRASTRUCTURE ONLY.

An independent second writing of the same definition as `jev_oracle`, used to
pin it: every question is run as its own sequence, row by row, head by head
and key by key, in float64, with `math` functions for the transcendental
parts.  It shares no code with `jev_oracle` (or with the HIP path); it is slow
and only meant for configurations with a few hundred hidden units.

Definition followed (the same pages as the oracle): a causal pre-norm decoder
over prefix ‖ suffix ("How to Deploy Visual Jev ...", Steps 2-3), candidate
probabilities read from the logits at the last valid position (Step 3), the
tree score of a multi-token candidate as the sum of its tokens'
log-probabilities along its own history ("FastJEV", §3.3).
"""
from __future__ import annotations

import math

import numpy as np


def _norm(vec, gain, eps):
    n = len(vec)
    acc = 0.0
    for i in range(n):
        acc += float(vec[i]) * float(vec[i])
    r = 1.0 / math.sqrt(acc / n + eps)
    return np.array([float(gain[i]) * float(vec[i]) * r for i in range(n)])


def _rotate(head_vec, pos, theta):
    D = len(head_vec)
    half = D // 2
    out = np.empty(D)
    for t in range(half):
        ang = pos * theta ** (-(2.0 * t) / D)
        c, s = math.cos(ang), math.sin(ang)
        a, b = head_vec[t], head_vec[t + half]
        out[t] = a * c - b * s
        out[t + half] = a * s + b * c
    return out


def _hidden_states(cfg, W, rows, skip=None, first_candidate=0):
    """Run every layer over `rows` (list of float64 vectors); returns the final rows.

    Where skip[l] is set, rows from first_candidate on leave block l with the value
    they entered it with ("FastJEV", §2.3: candidate evaluation bypasses the
    selected complete blocks; the context rows keep every block)."""
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    per_kv = Hq // Hkv
    eps, theta = cfg.rms_eps, cfg.rope_theta
    x = [np.array(r, dtype=np.float64) for r in rows]
    N = len(x)
    for l in range(cfg.n_layers):
        Lw = {k: np.asarray(v, dtype=np.float64) for k, v in W.layer(l).items()}
        qs, ks, vs = [], [], []
        for i in range(N):
            a = _norm(x[i], Lw["attn_norm"], eps)
            q = Lw["wq"].dot(a)
            k = Lw["wk"].dot(a)
            v = Lw["wv"].dot(a)
            qs.append([_rotate(q[h * D:(h + 1) * D], i, theta) for h in range(Hq)])
            ks.append([_rotate(k[h * D:(h + 1) * D], i, theta) for h in range(Hkv)])
            vs.append([v[h * D:(h + 1) * D] for h in range(Hkv)])
        new_x = []
        for i in range(N):
            heads_out = []
            for h in range(Hq):
                g = h // per_kv
                scores = []
                for j in range(i + 1):          # causal: keys 0..i
                    dot = 0.0
                    qv, kv = qs[i][h], ks[j][g]
                    for d in range(D):
                        dot += qv[d] * kv[d]
                    scores.append(dot / math.sqrt(D))
                mx = max(scores)
                ws = [math.exp(s - mx) for s in scores]
                tot = sum(ws)
                o = np.zeros(D)
                for j in range(i + 1):
                    o += (ws[j] / tot) * vs[j][g]
                heads_out.append(o)
            attn = np.concatenate(heads_out)
            h1 = x[i] + Lw["wo"].dot(attn)
            m = _norm(h1, Lw["mlp_norm"], eps)
            gate = Lw["w_gate"].dot(m)
            up = Lw["w_up"].dot(m)
            act = np.array([gate[t] / (1.0 + math.exp(-gate[t])) * up[t] for t in range(len(gate))])
            bypass = skip is not None and skip[l] and i >= first_candidate
            new_x.append(x[i] if bypass else h1 + Lw["w_down"].dot(act))
        x = new_x
    return x


def _full_log_probs(cfg, W, h):
    G = {k: np.asarray(v, dtype=np.float64) for k, v in W.glob.items()}
    z = G["lm_head"].dot(_norm(h, G["final_norm"], cfg.rms_eps))
    mx = max(z)
    lse = mx + math.log(sum(math.exp(t - mx) for t in z))
    return z - lse


def _prefix_rows(W, prefix):
    E = W.glob["embed"]
    rows = [np.asarray(r, dtype=np.float64) for r in prefix["vis"]]
    rows += [np.asarray(E[t], dtype=np.float64) for t in prefix["text_ids"]]
    return rows


def score_suffixes(cfg, W, prefix, suf, skip=None):
    """float64 out[b, c] = log-softmax over the candidates of the last-row logits."""
    E = W.glob["embed"]
    pre = _prefix_rows(W, prefix)
    B, C = suf["cands"].shape
    out = np.full((B, C), -np.inf)
    for b in range(B):
        L = int(suf["lens"][b])
        rows = pre + [np.asarray(E[t], dtype=np.float64) for t in suf["ids"][b, :L]]
        lp = _full_log_probs(cfg, W, _hidden_states(cfg, W, rows, skip, len(pre))[-1])
        n = int(suf["n_cands"][b])
        sel = [lp[int(c)] for c in suf["cands"][b, :n]]
        mx = max(sel)
        lse = mx + math.log(sum(math.exp(s - mx) for s in sel))
        for c in range(n):
            out[b, c] = sel[c] - lse
    return out


def score_segments(cfg, W, images, suf, seg):
    """float64 out[b]: suffix b evaluated over the prefix of image seg[b] only."""
    B, C = suf["cands"].shape
    out = np.full((B, C), -np.inf)
    for b in range(B):
        one = {k: v[b:b + 1] for k, v in suf.items()}
        out[b] = score_suffixes(cfg, W, images[int(seg[b])], one)[0]
    return out


def score_tree(cfg, W, prefix, tree, skip=None):
    """float64 flat tree scores: sum of the candidate tokens' full-vocab log-probs."""
    E = W.glob["embed"]
    pre = _prefix_rows(W, prefix)
    Q, C, _ = tree["cand_tok"].shape
    score = np.full((Q, C), -np.inf)
    norm = np.full((Q, C), -np.inf)
    for q in range(Q):
        s = int(tree["stem_lens"][q])
        stem = [int(t) for t in tree["stem_ids"][q, :s]]
        n = int(tree["n_cands"][q])
        for c in range(n):
            K = int(tree["cand_lens"][q, c])
            w = [int(t) for t in tree["cand_tok"][q, c, :K]]
            fed = stem + w[:K - 1]
            hs = _hidden_states(cfg, W, pre + [np.asarray(E[t], dtype=np.float64) for t in fed], skip, len(pre))
            tot = 0.0
            for k in range(K):
                lp = _full_log_probs(cfg, W, hs[len(pre) + s - 1 + k])
                tot += lp[w[k]]
            score[q, c] = tot
        mx = max(score[q, :n])
        lse = mx + math.log(sum(math.exp(v - mx) for v in score[q, :n]))
        norm[q, :n] = score[q, :n] - lse
    return {"score": score, "norm": norm}
