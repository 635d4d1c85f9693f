"""Write the oracle's expected outputs for the full-size workloads.

Calls only `oracle/` (and the shared input generator).  Each output file
tests/golden/<config>_s<seed>.json holds the oracle's float32 results plus a
fingerprint of the generated inputs, so a consumer can check that it rebuilt
the same inputs before comparing.

    python tests/golden/make_golden.py c2 c3 c4 c5 c6 c3_skip    # all seeds listed below
"""
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import jev_synth as S                      # noqa: E402
from oracle import jev_oracle as O         # noqa: E402

SEEDS = {"c2": (0, 1, 2), "c3": (0,), "c4": (0,), "c5": (0, 1), "c6": (0,)}
# Block-skipping cases ("FastJEV", §2.3 and §3.4): the candidate rows bypass the later blocks
# but the last: n_skip = (3 L + 3) // 7 of them (12 of 28), the prefix keeps every block.
SKIP_SEEDS = {"c3": (0,)}


def skip_mask(cfg):
    n_skip = (cfg.n_layers * 3 + 3) // 7
    mask = np.zeros(cfg.n_layers, np.uint8)
    mask[cfg.n_layers - 1 - n_skip:cfg.n_layers - 1] = 1
    return mask
HERE = os.path.dirname(os.path.abspath(__file__))


def fingerprint(cfg, seed):
    """Hash of the generated request inputs and a few weight values."""
    h = hashlib.sha256()
    pre = S.prefix_inputs(cfg, seed)
    h.update(pre["text_ids"].tobytes())
    h.update(pre["vis"][:4].tobytes())
    if cfg.n_suffix:
        for v in S.suffix_inputs(cfg, seed).values():
            h.update(v.tobytes())
    if cfg.n_questions:
        for v in S.tree_inputs(cfg, seed).values():
            h.update(v.tobytes())
    if cfg.n_images:
        inp = S.images_inputs(cfg, seed)
        for im in inp["images"]:
            h.update(im["vis"][:4].tobytes())
            h.update(im["text_ids"].tobytes())
        for v in inp["suf"].values():
            h.update(v.tobytes())
        h.update(inp["seg_lens"].tobytes())
    w = S.weights_layer(S.with_overrides(cfg, hidden=cfg.hidden), seed, 0)
    h.update(w["wq"][:2].tobytes())
    return h.hexdigest()


def run_skip(name, seed):
    """The suffix workload with the block-skip mask of skip_mask()."""
    cfg = S.CONFIGS[name]
    ws = S.WeightSource(cfg, seed, cache_layers=False)
    pre, suf = S.prefix_inputs(cfg, seed), S.suffix_inputs(cfg, seed)
    mask = skip_mask(cfg)
    t0 = time.time()
    out = O.score_suffixes(ws, cfg, pre, suf, free_layers=True, skip=mask)
    rec = {"config": name, "seed": seed, "fingerprint": fingerprint(cfg, seed),
           "method": "oracle prefix-once (layer-major), float32 numpy, candidate rows skipping the masked blocks",
           "skip": [int(v) for v in mask], "out": out.astype(float).tolist(),
           "margin": O.margins(out, suf["n_cands"]).astype(float).tolist(), "oracle_seconds": time.time() - t0}
    path = os.path.join(HERE, f"{name}_skip_s{seed}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, allow_nan=True)
    print(f"{name} skip seed {seed}: {rec['oracle_seconds']:.1f} s -> {path}", flush=True)


def run(name, seed):
    cfg = S.CONFIGS[name]
    ws = S.WeightSource(cfg, seed, cache_layers=False)
    pre = S.prefix_inputs(cfg, seed)
    t0 = time.time()
    rec = {"config": name, "seed": seed, "fingerprint": fingerprint(cfg, seed),
           "method": "oracle prefix-once (layer-major), float32 numpy"}
    if cfg.n_images:
        inp = S.images_inputs(cfg, seed)
        out = O.score_segments(ws, cfg, inp["images"], inp["suf"], inp["seg"])
        rec["out"] = out.astype(float).tolist()
        rec["margin"] = O.margins(out, inp["suf"]["n_cands"]).astype(float).tolist()
    elif cfg.n_questions:
        tree = S.tree_inputs(cfg, seed)
        r = O.score_tree(ws, cfg, pre, tree, free_layers=True)
        rec["score"] = r["score"].astype(float).tolist()
        rec["norm"] = r["norm"].astype(float).tolist()
    else:
        suf = S.suffix_inputs(cfg, seed)
        out = O.score_suffixes(ws, cfg, pre, suf, free_layers=True)
        rec["out"] = out.astype(float).tolist()
        rec["margin"] = O.margins(out, suf["n_cands"]).astype(float).tolist()
    rec["oracle_seconds"] = time.time() - t0
    path = os.path.join(HERE, f"{name}_s{seed}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, allow_nan=True)
    print(f"{name} seed {seed}: {rec['oracle_seconds']:.1f} s -> {path}", flush=True)


if __name__ == "__main__":
    # names: configs (c2 ... c6) or <config>_skip for the block-skipping cases
    names = sys.argv[1:] or list(SEEDS) + [f"{k}_skip" for k in SKIP_SEEDS]
    for n in names:
        if n.endswith("_skip"):
            for s in SKIP_SEEDS[n[:-5]]:
                run_skip(n[:-5], s)
        else:
            for s in SEEDS[n]:
                run(n, s)
