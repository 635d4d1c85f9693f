#!/usr/bin/env python3
"""Benchmark of shared-prefix candidate scoring on one MI355X.

One step = the whole per-image path on one batch: prefill the prefix once
(jev_prefill_prefix) and score every suffix's candidates in one batched
forward over it (jev_score_suffixes).  Default workload: the Qwen2.5-VL-7B-
shaped decoder (28 layers, hidden 3584, 28/4 heads of 128, MLP 18944,
vocab 152064, bf16 random-init weights), a 1024-position prefix (1000 visual
embeddings + 24 text ids) and 32 suffixes of 6..16 tokens with 2 candidates
each; all inputs synthetic and seeded, resident in HBM before timing.

Prints ONE JSON line.  `value` = candidates scored per second over whole
steps (prefill + score).  Extra fields give the score-only and prefill-only
times, the per-kernel breakdown from the library's event timing, the
roofline of the dominant kernel and of the shared-prefix attention, and the
CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload c3]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "candidates scored/sec + attention MFMA util, 7B-shaped prefix 1024, 32 suffixes"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0
PRECISION = None               # GEMM precision mode (set in main)
PRECISION_NOTE = {
    "f16_down": "f16_down: down projection as one float16 pass on a float16 weight mirror; q|k|v, o and "
                "gate|up as two bfloat16 passes (hi + lo of the float32 activation); float32 accumulation",
    "split": "split: every decoder GEMM as two bfloat16 passes (hi + lo of the float32 activation)",
    "f16_down_gup": "f16_down_gup: down projection as one float16 pass on a float16 weight mirror; gate|up as "
                    "one float16 pass in the prefill and two bfloat16 passes (hi + lo of the float32 "
                    "activation) in the scoring call; q|k|v and o as two bfloat16 passes; float32 accumulation",
    "f16_prefill": "f16_prefill: down projection as one float16 pass on a float16 weight mirror; in prefills "
                   "every projection as one float16 pass (q|k|v only for prefixes of at most 2048 rows, "
                   "else two bfloat16 passes); in the scoring call gate|up, o and q|k|v as two bfloat16 "
                   "passes (hi + lo of the float32 activation); float32 accumulation",
    "f16_score_gup": "f16_score_gup: down projection as one float16 pass on a float16 weight mirror; gate|up as "
                     "one float16 pass in prefills and suffix-scoring calls (two bfloat16 passes in tree "
                     "calls); in prefills q|k|v (prefixes of at most 2048 rows) and o as one float16 pass, in "
                     "scoring calls as two bfloat16 passes (hi + lo of the float32 activation); float32 "
                     "accumulation",
    "f16_down_gup_o": "f16_down_gup_o: down projection as one float16 pass on a float16 weight mirror; gate|up "
                      "and o as one float16 pass in the prefill and two bfloat16 passes (hi + lo of the float32 "
                      "activation) in the scoring call; q|k|v as two bfloat16 passes; float32 accumulation",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def workload_name(cfg):
    return (f"{cfg.name}: {cfg.n_layers}-layer decoder, hidden {cfg.hidden}, {cfg.n_q_heads}/{cfg.n_kv_heads} "
            f"heads x {cfg.head_dim}, MLP {cfg.mlp}, vocab {cfg.vocab}, {cfg.dtype}; prefix {cfg.prefix_len} "
            f"({cfg.n_vis} visual + {cfg.n_text} text); {cfg.n_suffix} suffixes of {cfg.len_lo}-{cfg.len_hi} "
            f"tokens, {cfg.n_cands} candidates each")


def roofline(kind, d, traffic_md=None):
    """Roofline entry of one kernel kind from the library's event timing.

    achieved = algorithmic flops per launch (each product counted once) / average
    launch time.  The two-term bf16 GEMMs (gemm_qkv, gemm_o, gemm_gate_up, gemm_down,
    gemm_swiglu, lm_head_lse) run every product twice (hi and lo planes of the float32
    activations), so the MFMA pipes execute 2x the algorithmic flops: reported as
    executed_tflops / executed_frac.  The float16 GEMMs (kinds ending in _f16) execute
    each product once.  traffic_md: the counter summary of this launch shape under profiles/
    (default {kind}_traffic.md).
    """
    from vlm_shared_prefix_amd import profiling
    n = d["launches"]
    avg_s = d["ms"] / n * 1e-3
    traffic = None
    stored = profiling.stored_traffic(os.path.join(ROOT, "profiles", traffic_md or f"{kind}_traffic.md"))
    if stored and stored[1] == profiling.source_digest():
        traffic = stored[0]
    if d["flops"] > 0:
        ach = d["flops"] / n / avg_s / 1e12
        r = {"kernel": kind, "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
             "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
             "avg_launch_us": round(avg_s * 1e6, 2), "launches": n,
             "algorithmic_flops_per_launch": d["flops"] / n}
        # two passes: the bf16 kinds (the float16 kinds end in _f16)
        passes = 2 if (kind.startswith("gemm") or kind == "lm_head_lse") and not kind.endswith("_f16") else 1
        if kind.startswith("gemm") or kind == "lm_head_lse":
            r["executed_tflops"] = round(passes * ach, 2)
            r["executed_frac"] = round(passes * ach / PEAK_BF16_TFLOPS, 4)
        return r
    ach = d["bytes"] / n / avg_s / 1e9
    return {"kernel": kind, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic, "avg_launch_us": round(avg_s * 1e6, 2),
            "launches": n}


def step_rooflines(prof_step, prof_prefill, prof_score, cfg):
    """(roofline, score_call_roofline) of a step's profiles (kind -> launches, ms, flops, bytes).

    The step's entry is the kind with the most time in the step.  When the prefill and the
    scoring call both launch it (the float16 SwiGLU), it is taken over the prefill's launches
    alone, one launch shape, with its traffic from {kind}_traffic.md; the scoring call's own
    dominant kind gets the second entry, with its traffic from {kind}_score_traffic.md.
    """
    roof = score_roof = None
    if prof_step:
        dom = max(prof_step, key=lambda k: prof_step[k]["ms"])
        roof = roofline(dom, prof_prefill[dom] if dom in prof_prefill else prof_step[dom])
        if dom in prof_prefill:
            roof["launches_of"] = f"prefill ({cfg.prefix_len} rows)"
    if prof_score:
        dom_s = max(prof_score, key=lambda k: prof_score[k]["ms"])
        score_roof = roofline(dom_s, prof_score[dom_s], f"{dom_s}_score_traffic.md")
        score_roof["launches_of"] = f"scoring call ({cfg.n_suffix} suffixes)"
    return roof, score_roof


def attention_entry(prof, prefix_kv_bytes, what):
    """MFMA utilisation of the attention launches of one call kind (+ its split merge)."""
    at = prof.get("attn_fwd")
    if not at:
        return None
    a_s = at["ms"] / at["launches"] * 1e-3
    a_tf = at["flops"] / at["launches"] / a_s / 1e12
    e = {"what": what, "achieved_tflops": round(a_tf, 2), "mfma_util": round(a_tf / PEAK_BF16_TFLOPS, 4),
         "avg_launch_us": round(a_s * 1e6, 2), "launches": at["launches"],
         "algorithmic_flops_per_launch": at["flops"] / at["launches"]}
    if prefix_kv_bytes:
        e["prefix_kv_gbs"] = round(prefix_kv_bytes / a_s / 1e9, 1)
        e["prefix_kv_hbm_frac"] = round(prefix_kv_bytes / a_s / 1e9 / PEAK_HBM_GBS, 4)
    mg = prof.get("attn_merge")
    if mg:
        e["merge_avg_us"] = round(mg["ms"] / mg["launches"] * 1e3, 2)
        e["with_merge_mfma_util"] = round(at["flops"] / (at["ms"] + mg["ms"]) * 1e3 / 1e12 / PEAK_BF16_TFLOPS, 4)
    return e


def _prefill_flops(cfg):
    """Algorithmic flops of a prefill: 2 x decoder matrix parameters x rows for every layer but
    the last (which only writes K/V: q|k|v), plus the causal attention 4·D·Hq·P(P+1)/2 per layer
    that runs it (all but the last)."""
    P, H, D, I = cfg.prefix_len, cfg.hidden, cfg.head_dim, cfg.mlp
    qkv = H * (cfg.n_q_heads + 2 * cfg.n_kv_heads) * D
    per = qkv + cfg.n_q_heads * D * H + 3 * H * I
    L = cfg.n_layers
    attn = 4.0 * D * cfg.n_q_heads * P * (P + 1) / 2
    return 2.0 * P * (per * (L - 1) + qkv) + attn * (L - 1)


def step_stats(stream, fn, k):
    """fn() enqueued k times on `stream` with an event pair around each call: the total time
    between the first and the last event (ms per call, the mean) and the median, p10 and p90
    of the per-call times."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(k + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(k):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(k)])
    return {"mean_ms": round(float(ev[0].elapsed_time(ev[k]) / k), 4), "median_ms": round(float(np.median(per)), 4),
            "p10_ms": round(float(np.percentile(per, 10)), 4), "p90_ms": round(float(np.percentile(per, 90)), 4)}


def timed_on(stream, fn, k, warm=0):
    """ms per call of fn() enqueued k times on `stream`, between events recorded on that stream."""
    import torch
    with torch.cuda.stream(stream):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(k):
            fn()
        b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / k


def tree_section(seed, dev, profile_steps, name="c5", sweep=True):
    """Secondary measurement: the long-prefix tree workload (prefix 8192, 16 questions with
    4 multi-token candidates each, trie sharing) on the same 7B shape; not the headline value."""
    import torch
    import jev_synth as S
    from vlm_shared_prefix_amd import jev as J
    from vlm_shared_prefix_amd.session import Session
    cfg = S.CONFIGS[name]
    t = time.time()
    sess = Session.generated(cfg, seed, dev, precision=PRECISION)
    pre, tree = S.prefix_inputs(cfg, seed), S.tree_inputs(cfg, seed)
    log(f"[bench] {name}: weights drawn and uploaded in {time.time() - t:.1f} s")
    sess.prefill(pre["vis"], pre["text_ids"])
    sess.score_tree(tree, J.JEV_TREE_TRIE)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def timed(fn, k):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(k):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / k

    ms_tree = timed(lambda: sess.score_tree(tree, J.JEV_TREE_TRIE), 3)
    gstream = torch.cuda.Stream()
    cap = sess.capture_score_tree(tree, J.JEV_TREE_TRIE, gstream)
    ms_tree_graph = timed_on(gstream, cap.replay, 3, warm=1)
    e_score, _ = sess.score_tree(tree, J.JEV_TREE_TRIE)
    torch.cuda.synchronize()
    tree_graph = {"tree_call_ms": round(ms_tree_graph, 3),
                  "bitwise_equal_to_eager": bool(torch.equal(cap.outs[0], e_score))}
    del cap
    ms_prefill = timed(lambda: sess.prefill(pre["vis"], pre["text_ids"]), 1)
    # the long-prefix prefill's kernels (causal attention over 8192 rows, GEMMs of 8192 rows)
    J.jev_profile_start(sess.model)
    sess.prefill(pre["vis"], pre["text_ids"])
    prof_pre = J.jev_profile_stop(sess.model)
    prefill_kernels = {"attention": attention_entry(prof_pre, 0, f"causal self-attention of the {cfg.prefix_len} "
                                                                  f"prefix rows")}
    for kind in ("gemm_swiglu", "gemm_swiglu_f16", "gemm_qkv", "gemm_qkv_f16", "gemm_o", "gemm_o_f16", "gemm_down",
                 "gemm_down_f16"):
        if prof_pre.get(kind):
            k = prof_pre[kind]
            prefill_kernels[kind] = {"launches": k["launches"], "avg_launch_us": round(k["ms"] * 1e3 / k["launches"], 1),
                                     "algorithmic_tflops": round(k["flops"] / (k["ms"] * 1e-3) / 1e12, 1)}
    J.jev_profile_start(sess.model)
    for _ in range(max(1, profile_steps)):
        sess.score_tree(tree, J.JEV_TREE_TRIE)
    prof = J.jev_profile_stop(sess.model)
    rows = J.jev_tree_plan_size(tree["stem_ids"], tree["stem_lens"], tree["cand_tok"], tree["cand_lens"],
                                tree["n_cands"], J.JEV_TREE_TRIE)[0]
    n_c = int(np.sum(tree["n_cands"]))
    desc = (f"{name}: {cfg.n_layers}-layer decoder, hidden {cfg.hidden}, {cfg.n_q_heads}/{cfg.n_kv_heads} heads x "
            f"{cfg.head_dim}, MLP {cfg.mlp}, vocab {cfg.vocab}, {cfg.dtype}; prefix {cfg.prefix_len}; "
            f"{cfg.n_questions} questions, {cfg.stem_len}-token stems, {cfg.tree_cands} candidates of "
            f"{cfg.cand_len_lo}-{cfg.cand_len_hi} tokens; trie sharing, full-vocabulary log-probs")
    out = {"workload": desc, "tree_rows": int(rows),
           "tree_call_ms": round(ms_tree, 3), "candidates_per_s": round(n_c / (ms_tree * 1e-3), 1),
           "graph_replay": tree_graph, "prefill_ms": round(ms_prefill, 3),
           "prefill_algorithmic_tflops": round(_prefill_flops(cfg) / (ms_prefill * 1e-3) / 1e12, 1),
           "prefill_kernels": prefill_kernels,
           "attention": attention_entry(prof, cfg.prefix_len * cfg.n_kv_heads * cfg.head_dim * 4,
                                        f"shared prefix ({cfg.prefix_len} keys) + tree rows ({rows})")}
    # trie vs stem-only vs flat schedules ("FastJEV" §4.7, Table 5): the same questions with
    # independent candidates and with overlapping ones (candidate k+1 repeating a leading run
    # of candidate k half the time), rows fed and call time per mode
    schedules = {}
    for label, tcfg in (("independent", cfg), ("overlapping", S.with_overrides(cfg, overlap=True)))[:2 if sweep else 0]:
        tt = S.tree_inputs(tcfg, seed)
        runs = {}
        for mode, mname in ((J.JEV_TREE_TRIE, "trie"), (J.JEV_TREE_STEM_ONLY, "stem_only"), (J.JEV_TREE_FLAT, "flat")):
            sess.score_tree(tt, mode)
            ms = timed(lambda: sess.score_tree(tt, mode), 3)
            r = J.jev_tree_plan_size(tt["stem_ids"], tt["stem_lens"], tt["cand_tok"], tt["cand_lens"],
                                     tt["n_cands"], mode)[0]
            runs[mname] = {"rows": int(r), "call_ms": round(ms, 3)}
        schedules[label] = runs
    out["schedules"] = schedules
    # the flat schedule's attention (64 sequences of 12-15 rows: the largest shared-prefix
    # attention launch of the workload)
    sess.score_tree(tree, J.JEV_TREE_FLAT)
    J.jev_profile_start(sess.model)
    for _ in range(max(1, profile_steps)):
        sess.score_tree(tree, J.JEV_TREE_FLAT)
    flat_rows = J.jev_tree_plan_size(tree["stem_ids"], tree["stem_lens"], tree["cand_tok"], tree["cand_lens"],
                                     tree["n_cands"], J.JEV_TREE_FLAT)[0]
    out["attention_flat"] = attention_entry(J.jev_profile_stop(sess.model),
                                            cfg.prefix_len * cfg.n_kv_heads * cfg.head_dim * 4,
                                            f"shared prefix ({cfg.prefix_len} keys) + flat rows ({flat_rows})")
    modes_ms = {}
    for mode, mname in ((J.JEV_TREE_TRIE, "trie"), (J.JEV_TREE_STEM_ONLY, "stem_only"), (J.JEV_TREE_FLAT, "flat")):
        st = step_stats(stream, lambda: sess.score_tree(tree, mode), 5)
        modes_ms[mname] = {"ms": st["median_ms"], "p10_ms": st["p10_ms"], "p90_ms": st["p90_ms"],
                           "candidates_per_s": round(n_c / (st["median_ms"] * 1e-3), 1)}
    out["modes"] = modes_ms
    # the same comparison at a controlled shared fraction: every candidate has cand_len_hi
    # tokens and a question's candidates agree on their first s of them
    sweep_out = []
    for shared in range(cfg.cand_len_hi if sweep else 0):
        tt = S.shared_tree_inputs(cfg, seed, shared)
        e = {"shared_tokens": shared, "shared_fraction": round(shared / cfg.cand_len_hi, 3)}
        modes = ((J.JEV_TREE_TRIE, "trie"), (J.JEV_TREE_STEM_ONLY, "stem_only"), (J.JEV_TREE_FLAT, "flat"))
        for mode, _ in modes:
            sess.score_tree(tt, mode)
        # two interleaved passes over the modes, 5 calls each: call_ms is their mean,
        # pass_ms both pass means (the spread between them is the run's noise)
        passes = {mname: [] for _, mname in modes}
        for _ in range(2):
            for mode, mname in modes:
                passes[mname].append(timed(lambda: sess.score_tree(tt, mode), 5))
        for mode, mname in modes:
            r = J.jev_tree_plan_size(tt["stem_ids"], tt["stem_lens"], tt["cand_tok"], tt["cand_lens"],
                                     tt["n_cands"], mode)[0]
            e[mname] = {"rows": int(r), "call_ms": round(float(np.mean(passes[mname])), 3),
                        "pass_ms": [round(x, 3) for x in passes[mname]]}
        e["fastest"] = min(("trie", "stem_only", "flat"), key=lambda k: e[k]["call_ms"])
        sweep_out.append(e)
    out["shared_fraction_sweep"] = sweep_out

    # the memory-bound end: the same prefix with only the first q question stems (few query
    # rows per KV head), where the attention is bound by streaming the prefix KV
    kv_bytes = cfg.prefix_len * cfg.n_kv_heads * cfg.head_dim * 2 * 2 * cfg.n_layers
    stream_rows = []
    for q in (1, 3):
        tq = {k: np.ascontiguousarray(v[:q]) for k, v in tree.items()}
        sess.score_tree(tq, J.JEV_TREE_TRIE)
        J.jev_profile_start(sess.model)
        for _ in range(max(1, profile_steps)):
            sess.score_tree(tq, J.JEV_TREE_TRIE)
        pq = J.jev_profile_stop(sess.model)
        a = pq["attn_fwd"]
        a_s = a["ms"] / a["launches"] * 1e-3
        e = {"questions": q, "rows": int(J.jev_tree_plan_size(tq["stem_ids"], tq["stem_lens"], tq["cand_tok"],
                                                             tq["cand_lens"], tq["n_cands"], J.JEV_TREE_TRIE)[0]),
             "attn_avg_launch_us": round(a_s * 1e6, 2),
             "prefix_kv_gbs": round(kv_bytes / cfg.n_layers / a_s / 1e9, 1),
             "prefix_kv_hbm_frac": round(kv_bytes / cfg.n_layers / a_s / 1e9 / PEAK_HBM_GBS, 4)}
        if pq.get("attn_merge"):
            e["merge_avg_us"] = round(pq["attn_merge"]["ms"] / pq["attn_merge"]["launches"] * 1e3, 2)
        stream_rows.append(e)
    out["prefix_kv_stream"] = {"what": f"prefix KV ({kv_bytes // cfg.n_layers / 1e6:.1f} MB per layer) read by the "
                                       f"attention of the first 1 / 3 questions (trie)", "runs": stream_rows}
    log(f"[bench] {name}: tree call {ms_tree:.2f} ms, prefill {ms_prefill:.1f} ms; prefix-KV stream "
        + ", ".join(f"Q={e['questions']} {e['prefix_kv_gbs']} GB/s" for e in stream_rows))
    sess.close()
    return out


def images_section(seed, dev, name="c6"):
    """Secondary measurement: one typed question over 8 images ("Ochevid Jev-VL 2B", One
    question, multiple images) on the 7B shape.  Batched: every image's prefix in one
    segmented store, prefilled in one forward, then one scoring call that asks the question
    of every image.  Separate: one prefix, one prefill and one scoring call per image (the
    same kernels).  Not the headline value."""
    import torch
    import jev_synth as S
    from vlm_shared_prefix_amd import jev as J
    from vlm_shared_prefix_amd.session import Session
    cfg = S.CONFIGS[name]
    t = time.time()
    sess = Session.generated(cfg, seed, dev, precision=PRECISION)
    inp = S.images_inputs(cfg, seed)
    log(f"[bench] {name}: weights drawn and uploaded in {time.time() - t:.1f} s")
    images, suf, seg = inp["images"], inp["suf"], inp["seg"]
    n = len(images)
    sess.prefill_segments(images)
    out = sess.score_segments(seg, suf)
    n_vis = np.array([im["vis"].shape[0] for im in images], np.int32)
    n_text = np.array([len(im["text_ids"]) for im in images], np.int32)
    text = np.concatenate([im["text_ids"] for im in images]).astype(np.int32)
    P = int(sess.P)
    ws = sess.workspace(max(J.jev_workspace_bytes(sess.model, P, P, 1, 0), sess.suffix_ws_bytes(suf)))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def timed(fn, k):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(k):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / k

    def batched_prefill():
        J.jev_prefill_segments(sess.prefix, sess.vis, n_vis, text, n_text, ws)

    def batched_score():
        J.jev_score_segments(sess.prefix, seg, suf["ids"], suf["lens"], suf["cands"], suf["n_cands"], out, ws)

    # one plain prefix per image over the same device inputs
    offs = np.concatenate([[0], np.cumsum(n_vis)])
    kvs, pfx, outs = [], [], []
    for i in range(n):
        Pi = int(n_vis[i] + n_text[i])
        kv = torch.empty(J.jev_prefix_bytes(sess.model, Pi), dtype=torch.uint8, device=dev)
        kvs.append(kv)
        pfx.append(J.jev_prefix_create(sess.model, Pi, kv))
        outs.append(torch.empty((1, suf["cands"].shape[1]), dtype=torch.float32, device=dev))
    singles = [{k: np.ascontiguousarray(v[i:i + 1]) for k, v in suf.items()} for i in range(n)]

    def separate_prefill():
        for i in range(n):
            J.jev_prefill_prefix(pfx[i], sess.vis[int(offs[i]):int(offs[i + 1])], int(n_vis[i]),
                                 images[i]["text_ids"], ws)

    def separate_score():
        for i in range(n):
            sb = singles[i]
            J.jev_score_suffixes(pfx[i], sb["ids"], sb["lens"], sb["cands"], sb["n_cands"], outs[i], ws)

    batched_prefill(); batched_score(); separate_prefill(); separate_score()
    ms_bp = timed(batched_prefill, 2)
    ms_bs = timed(batched_score, 5)
    ms_sp = timed(separate_prefill, 1)
    ms_ss = timed(separate_score, 3)
    diff = max(float((outs[i][0] - out[i]).abs().max()) for i in range(n))
    J.jev_profile_start(sess.model)
    batched_score()
    prof = J.jev_profile_stop(sess.model)
    for p in pfx:
        J.jev_prefix_destroy(p)
    desc = (f"{name}: {cfg.n_layers}-layer decoder, hidden {cfg.hidden}, {cfg.n_q_heads}/{cfg.n_kv_heads} heads x "
            f"{cfg.head_dim}, MLP {cfg.mlp}, vocab {cfg.vocab}, {cfg.dtype}; {n} images of "
            f"{int(n_vis[0])} visual + {int(n_text[0])} text rows; one question of {int(suf['lens'][0])} tokens, "
            f"{cfg.n_cands} options")
    res = {"workload": desc, "images": n,
           "batched": {"prefill_ms": round(ms_bp, 3), "score_ms": round(ms_bs, 3),
                       "answers_per_s": round(n / ((ms_bp + ms_bs) * 1e-3), 2)},
           "separate": {"prefill_ms": round(ms_sp, 3), "score_ms": round(ms_ss, 3),
                        "answers_per_s": round(n / ((ms_sp + ms_ss) * 1e-3), 2)},
           "speedup_batched_vs_separate": round((ms_sp + ms_ss) / (ms_bp + ms_bs), 3),
           "max_abs_diff_batched_vs_separate": round(diff, 6),
           "attention": attention_entry(prof, P * cfg.n_kv_heads * cfg.head_dim * 4,
                                        f"each suffix over its own image's {int(n_vis[0] + n_text[0])} keys")}
    log(f"[bench] {name}: batched prefill {ms_bp:.1f} ms + score {ms_bs:.2f} ms vs separate "
        f"{ms_sp:.1f} ms + {ms_ss:.2f} ms")
    sess.close()
    return res


def _timer(dev):
    import torch
    stream = torch.cuda.current_stream(dev)

    def timed(fn, k):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(k):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / k
    return timed


def configs_report(seed, dev, reps=5, names=("c1", "c2", "c4")):
    """Per-config call times: c1, c2 (scoring), c4 (each B, one batched call vs B single-suffix
    calls on the same prefix; the shared-prefix attention's MFMA utilisation at B = 32 and 100),
    c5 (trie, stem-only, flat).  ms per call (median, p10/p90), candidates per second."""
    import torch
    import jev_synth as S
    from vlm_shared_prefix_amd import jev as J
    from vlm_shared_prefix_amd.session import Session
    timed = _timer(dev)
    rep = {}
    stream = torch.cuda.current_stream(dev)
    for name in names:
        cfg = S.CONFIGS[name]
        sess = Session.generated(cfg, seed, dev, precision=PRECISION)
        pre = S.prefix_inputs(cfg, seed)
        sess.prefill(pre["vis"], pre["text_ids"])
        ms_pre = timed(lambda: sess.prefill(pre["vis"], pre["text_ids"]), 1)
        r = {"prefix_len": cfg.prefix_len, "prefill_ms": round(ms_pre, 3)}
        if name == "c5":
            tree = S.tree_inputs(cfg, seed)
            n_c = int(np.sum(tree["n_cands"]))
            for mode, mname in ((J.JEV_TREE_TRIE, "trie"), (J.JEV_TREE_STEM_ONLY, "stem_only"),
                                (J.JEV_TREE_FLAT, "flat")):
                sess.score_tree(tree, mode)
                ms = timed(lambda: sess.score_tree(tree, mode), reps)
                r[mname] = {"ms": round(ms, 3), "candidates_per_s": round(n_c / (ms * 1e-3), 1)}
        else:
            batches = S.C4_BATCHES if name == "c4" else (None,)
            for B in batches:
                suf = S.suffix_inputs(cfg, seed, n=B) if B else S.suffix_inputs(cfg, seed)
                nb = len(suf["lens"])
                n_c = int(np.sum(suf["n_cands"]))
                out = sess.score_suffixes(suf)
                sess.workspace(sess.suffix_ws_bytes(suf))
                st = step_stats(stream, lambda: sess.score_suffixes(suf, out), reps)
                ms = st["median_ms"]
                e = {"B": nb, "rows": int(np.sum(suf["lens"])), "ms": round(ms, 3), "p10_ms": st["p10_ms"],
                     "p90_ms": st["p90_ms"], "candidates_per_s": round(n_c / (ms * 1e-3), 1)}
                if name == "c4" and nb >= 32:
                    J.jev_profile_start(sess.model)
                    for _ in range(2):
                        sess.score_suffixes(suf, out)
                    e["attention"] = attention_entry(J.jev_profile_stop(sess.model),
                                                     cfg.prefix_len * cfg.n_kv_heads * cfg.head_dim * 4,
                                                     f"shared prefix ({cfg.prefix_len} keys) + own rows of "
                                                     f"{nb} suffixes")
                if name == "c4":
                    singles = [{k: v[b:b + 1] for k, v in suf.items()} for b in range(nb)]
                    o1 = torch.empty((1, out.shape[1]), dtype=torch.float32, device=dev)

                    def serial():
                        for sb in singles:
                            sess.score_suffixes(sb, o1)
                    serial()
                    ms_s = timed(serial, 1)
                    e.update({"serial_ms": round(ms_s, 3), "speedup": round(ms_s / ms, 2)})
                r[f"B{nb}" if name == "c4" else "score"] = e
        rep[name] = r
        log(f"[bench] {name}: {r}")
        sess.close()
        del sess
        torch.cuda.empty_cache()
    return rep


def host_info():
    """CPU model, memory and the BLAS NumPy calls (with its thread count) of this host."""
    info = {"cpu_count": os.cpu_count()}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal"):
                    info["ram_gib"] = round(int(line.split()[1]) / 2 ** 20, 1)
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            info["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
            info["blas_threads"] = int(blas[0].get("num_threads", 0))
    except Exception:
        pass
    return info


def cpu_baseline(cfg, seed, budget_layers=2):
    """The oracle as it stands on a bounded sample, scaled to the whole step.

    Sample: the oracle's prefix-once scoring (jev_oracle.score_suffixes) of all
    suffixes with the model cut to 0 and to `budget_layers` layers (same shapes).
    The 0-layer run is the embedding + readout cost; the difference gives the
    per-layer cost; estimate = readout + n_layers * per-layer.
    """
    import jev_synth as S
    from oracle import jev_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 0) for i in threadpool_info()), default=os.cpu_count())
    except Exception:
        cores = os.cpu_count()
    pre, suf = S.prefix_inputs(cfg, seed), S.suffix_inputs(cfg, seed)
    c0 = S.with_overrides(cfg, n_layers=0)
    ck = S.with_overrides(cfg, n_layers=budget_layers)
    ws = S.WeightSource(ck, seed)
    ws.glob
    for l in range(budget_layers):
        ws.layer(l)
    t = time.perf_counter()
    O.score_suffixes(ws, c0, pre, suf)
    t0 = time.perf_counter() - t
    t = time.perf_counter()
    O.score_suffixes(ws, ck, pre, suf)
    tk = time.perf_counter() - t
    per_layer = max(tk - t0, 0.0) / budget_layers
    est = t0 + cfg.n_layers * per_layer
    n_c = int(np.sum(suf["n_cands"]))
    return {"value": n_c / est, "unit": "candidates/s", "cores": int(cores), "kind": "oracle", "host": host_info(),
            "seconds_per_question": est / cfg.n_suffix,
            "sample": (f"jev_oracle.score_suffixes (prefix once, layer-major, float32 numpy) on all "
                       f"{cfg.n_suffix} suffixes with the model cut to 0 and {budget_layers} of "
                       f"{cfg.n_layers} layers; measured {t0:.2f} s and {tk:.2f} s, scaled to "
                       f"{cfg.n_layers} layers = {est:.1f} s per step"),
            "seconds_per_step": est}


def cpu_crosscheck(name, seed):
    """Host only: the oracle's full scoring call on one configuration (every layer, all
    suffixes) against the bounded-sample estimate cpu_baseline reports for it."""
    import jev_synth as S
    from oracle import jev_oracle as O
    cfg = S.CONFIGS[name]
    est = cpu_baseline(cfg, seed)
    ws = S.WeightSource(cfg, seed, cache_layers=False)
    pre, suf = S.prefix_inputs(cfg, seed), S.suffix_inputs(cfg, seed)
    # the full call draws each layer's weights as it reaches it; drawing them alone is timed
    # too and taken out, as the estimate's runs use weights drawn beforehand
    t = time.perf_counter()
    for l in range(cfg.n_layers):
        S.WeightSource(cfg, seed, cache_layers=False).layer(l)
        log(f"crosscheck {name}: drew layer {l + 1} of {cfg.n_layers} alone")
    draw = time.perf_counter() - t

    class _Reporting:
        """The weight source, reporting each layer the oracle reaches."""
        def __init__(self, src):
            self.src = src

        @property
        def glob(self):
            return self.src.glob

        def layer(self, l):
            log(f"crosscheck {name}: oracle at layer {l + 1} of {cfg.n_layers}")
            return self.src.layer(l)

        def drop_layer(self, l):
            self.src.drop_layer(l)

    t = time.perf_counter()
    O.score_suffixes(_Reporting(ws), cfg, pre, suf, free_layers=True)
    full = time.perf_counter() - t - draw
    n_c = int(np.sum(suf["n_cands"]))
    print(json.dumps({"config": name, "host": host_info(), "full_seconds": round(full, 2),
                      "weight_draw_seconds_excluded": round(draw, 2),
                      "full_candidates_per_s": round(n_c / full, 3),
                      "estimate_seconds": round(est["seconds_per_step"], 2),
                      "estimate_candidates_per_s": round(est["value"], 3),
                      "estimate_over_full": round(est["seconds_per_step"] / full, 3)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c3")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--profile-steps", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tree", action="store_true",
                    help="skip the secondary long-prefix tree measurement (config c5)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the tree section's schedule comparisons (shorter profiled runs)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config calls of c1, c2 and c4 (every B, batched and serial)")
    ap.add_argument("--cpu-crosscheck", default=None, metavar="CONFIG",
                    help="host only: time the oracle's full scoring call on CONFIG and the bounded-sample "
                         "estimate the bench reports, then exit (no GPU needed)")
    ap.add_argument("--precision", default=None,
                    help="GEMM precision mode of the bf16 models (see Session; default: the library default)")
    ap.add_argument("--no-serial", action="store_true",
                    help="skip the serial-vs-batched section (one call per suffix)")
    ap.add_argument("--no-images", action="store_true",
                    help="skip the one-question-over-8-images measurement (config c6)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay of the score call")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a device copy of a known size (the counter calibration for traffic)")
    args = ap.parse_args()
    if args.cpu_crosscheck:
        cpu_crosscheck(args.cpu_crosscheck, args.seed)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (--gpus {args.gpus} "
              f"requested). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import jev_synth as S
    from vlm_shared_prefix_amd import jev as J
    from vlm_shared_prefix_amd import session as SE
    from vlm_shared_prefix_amd.session import Session

    global PRECISION
    PRECISION = args.precision or SE.DEFAULT_PRECISION
    cfg = S.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    t = time.time()
    sess = Session.generated(cfg, args.seed, dev, precision=PRECISION)
    pre, suf = S.prefix_inputs(cfg, args.seed), S.suffix_inputs(cfg, args.seed)
    log(f"[bench] weights drawn and uploaded in {time.time() - t:.1f} s")
    n_cand = int(np.sum(suf["n_cands"]))
    T = int(np.sum(suf["lens"]))

    # resident inputs and buffers
    sess.prefill(pre["vis"], pre["text_ids"])
    out = sess.score_suffixes(suf)
    ws_bytes = max(sess.suffix_ws_bytes(suf), J.jev_workspace_bytes(sess.model, sess.P, sess.P, 1, 0))
    sess.workspace(ws_bytes)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def prefill_only():
        J.jev_prefill_prefix(sess.prefix, sess.vis, int(pre["vis"].shape[0]), pre["text_ids"], sess.ws)

    def score_only():
        J.jev_score_suffixes(sess.prefix, suf["ids"], suf["lens"], suf["cands"], suf["n_cands"], out, sess.ws)

    def step():
        prefill_only()
        score_only()

    def timed(fn, k):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(k):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / k

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")
    t_wall = time.perf_counter()
    step_st = step_stats(stream, step, args.steps)
    ms_step = step_st["mean_ms"]
    wall_ms = (time.perf_counter() - t_wall) * 1e3 / args.steps
    log(f"[bench] timed {args.steps} steps: {ms_step:.3f} ms/step (wall {wall_ms:.3f}); median "
        f"{step_st['median_ms']:.3f}, p10 {step_st['p10_ms']:.3f}, p90 {step_st['p90_ms']:.3f}")
    score_st = step_stats(stream, score_only, max(args.steps, 50))   # median / p10 / p90 over >= 50 calls
    ms_score = score_st["median_ms"]
    prefill_st = step_stats(stream, prefill_only, max(3, args.steps // 2))
    ms_prefill = prefill_st["median_ms"]
    log(f"[bench] score-only {ms_score:.3f} ms, prefill-only {ms_prefill:.3f} ms")

    # the score call replayed from a HIP graph (its launch-only entry point captured once; no
    # host planning or metadata copy per replay), on a stream of its own
    graph = None
    if not args.no_graph:
        gstream = torch.cuda.Stream()
        cap = sess.capture_score_suffixes(suf, gstream)
        ms_graph = timed_on(gstream, cap.replay, args.steps, warm=2)
        graph = {"score_ms": round(ms_graph, 4), "candidates_per_s": round(n_cand / (ms_graph * 1e-3), 2),
                 "speedup_vs_eager_score": round(ms_score / ms_graph, 3),
                 "bitwise_equal_to_eager": bool(torch.equal(cap.outs[0], out))}
        log(f"[bench] graph replay of the score call: {ms_graph:.3f} ms (eager {ms_score:.3f} ms)")
        del cap

    # the same suffixes scored one call per suffix over the same prefix (the serial baseline
    # the method replaces), and with a fresh prefill per question (image-per-question)
    singles = [{k: v[b:b + 1] for k, v in suf.items()} for b in range(len(suf["lens"]))]
    outs = [torch.empty((1, out.shape[1]), dtype=torch.float32, device=dev) for _ in singles]

    def serial_calls():
        for sb, ob in zip(singles, outs):
            J.jev_score_suffixes(sess.prefix, sb["ids"], sb["lens"], sb["cands"], sb["n_cands"], ob, sess.ws)

    serial = None
    if not args.no_serial:
        serial_calls()
        ms_serial = timed(serial_calls, 2)
        serial = {"suffixes": len(singles), "batched_score_ms": round(ms_score, 4),
                  "serial_score_ms": round(ms_serial, 4), "single_suffix_call_ms": round(ms_serial / len(singles), 4),
                  "speedup_vs_serial_calls": round(ms_serial / ms_score, 2),
                  "per_question_prefill_ms": round(len(singles) * (ms_prefill + ms_serial / len(singles)), 3),
                  "speedup_vs_per_question_prefill": round(len(singles) * (ms_prefill + ms_serial / len(singles)) /
                                                           ms_step, 2)}
        log(f"[bench] serial: {len(singles)} single-suffix calls {ms_serial:.2f} ms vs batched {ms_score:.2f} ms")

    # decision-guided block skipping ("FastJEV", §3.4): the candidate rows bypass a block mask
    # (here a fixed synthetic one: 12 of 28 blocks, the later ones but not the final block, near
    # the pages' 43.75-45.83% budgets; ranking blocks needs trained weights and calibration
    # inputs), the prefix keeps every block.  Not part of `value`.
    skip = None
    if cfg.n_layers >= 4:
        n_skip = (cfg.n_layers * 3 + 3) // 7           # 12 of 28
        mask = np.zeros(cfg.n_layers, np.uint8)
        mask[cfg.n_layers - 1 - n_skip:cfg.n_layers - 1] = 1
        sess.set_skip(mask)
        score_only()
        ms_skip = timed(score_only, args.steps)
        sess.set_skip(None)
        skip = {"skipped_blocks": [int(i) for i in np.nonzero(mask)[0]], "score_ms": round(ms_skip, 4),
                "candidates_per_s": round(n_cand / (ms_skip * 1e-3), 2),
                "speedup_vs_full_depth_score": round(ms_score / ms_skip, 3)}
        log(f"[bench] block skipping ({int(mask.sum())} of {cfg.n_layers}): score call {ms_skip:.3f} ms "
            f"vs {ms_score:.3f} ms")

    # per-kernel event timing (separate passes over the same calls)
    J.jev_profile_start(sess.model)
    for _ in range(args.profile_steps):
        step()
    prof_step = J.jev_profile_stop(sess.model)
    J.jev_profile_start(sess.model)
    for _ in range(args.profile_steps):
        score_only()
    prof_score = J.jev_profile_stop(sess.model)
    J.jev_profile_start(sess.model)
    for _ in range(args.profile_steps):
        prefill_only()
    prof_prefill = J.jev_profile_stop(sess.model)
    roof, score_roof = step_rooflines(prof_step, prof_prefill, prof_score, cfg)
    attn = {"score_call": attention_entry(prof_score, cfg.prefix_len * cfg.n_kv_heads * cfg.head_dim * 4,
                                          f"shared prefix ({cfg.prefix_len} keys) + own rows of the "
                                          f"{cfg.n_suffix} suffixes"),
            "prefill": attention_entry(prof_prefill, 0,
                                       f"causal self-attention of the {cfg.prefix_len} prefix rows"),
            "query_rows": cfg.group * T, "padded_rows": cfg.group * cfg.n_suffix * cfg.s_max}
    kernels = {k: {"launches": v["launches"], "ms_total": round(v["ms"], 4),
                   "us_avg": round(v["ms"] * 1e3 / v["launches"], 2)} for k, v in prof_step.items()}
    if args.calib_copy:   # plain copy of a known size for the FETCH_SIZE / WRITE_SIZE scale factors
        from vlm_shared_prefix_amd import profiling
        src = torch.empty(profiling.CALIB_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    configs = None
    if not args.no_configs:
        sess.close()
        torch.cuda.empty_cache()
        configs = configs_report(args.seed, dev, reps=max(3, args.steps // 4))

    tree = None
    if not args.no_tree:
        if args.no_configs:
            sess.close()
        del sess
        torch.cuda.empty_cache()
        tree = tree_section(args.seed, dev, args.profile_steps, sweep=not args.no_sweep)

    images = None
    if not args.no_images:
        if args.no_tree and args.no_configs:
            sess.close()
            del sess
        torch.cuda.empty_cache()
        images = images_section(args.seed, dev)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline on a bounded sample ...")
        cpu = cpu_baseline(cfg, args.seed)
        log(f"[bench] CPU oracle: {cpu['value']:.3f} candidates/s")

    res = {
        "metric": METRIC,
        "value": round(n_cand / (ms_step * 1e-3), 2),
        "unit": "candidates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_ms": step_st,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+f16",
        "data": "synthetic (seeded random-init weights and inputs of the workload's shapes)",
        "config": {"workload": workload_name(cfg), "prefix_len": cfg.prefix_len, "suffixes": cfg.n_suffix,
                   "suffix_rows": T, "candidates": n_cand, "seed": args.seed,
                   "gemm_precision": PRECISION_NOTE.get(PRECISION, PRECISION),
                   "step": "jev_prefill_prefix + jev_score_suffixes"},
        "score_only": {"ms": round(ms_score, 4), "p10_ms": score_st["p10_ms"], "p90_ms": score_st["p90_ms"],
                       "candidates_per_s": round(n_cand / (ms_score * 1e-3), 2)},
        "prefill_ms": round(ms_prefill, 4),
        "prefill_p10_p90_ms": [prefill_st["p10_ms"], prefill_st["p90_ms"]],
        "roofline": roof,
        "score_call_roofline": score_roof,
        "attention": attn,
        "graph_replay": graph,
        "serial_vs_batched": serial,
        "block_skipping": skip,
        "kernels": kernels,
        "long_prefix_tree": tree,
        "one_question_many_images": images,
        "configs": configs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
