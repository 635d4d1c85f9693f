"""Host logic of the bench line (no GPU): the roofline entries and the attention entry
built from the library's per-kind event timing, on made-up profiles whose answers follow
by arithmetic."""
import importlib.util
import os
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)   # defines functions only; main() runs under __main__
    return mod


def kind(launches, ms, flops=0.0, nbytes=0.0):
    return {"launches": launches, "ms": ms, "flops": flops, "bytes": nbytes}


def test_roofline_counts_each_product_once(bench):
    """achieved = algorithmic flops per launch / mean launch time; two-pass bf16 kinds
    execute twice that, float16 kinds (suffix _f16) once; byte-only kinds are HBM-bound."""
    r = bench.roofline("gemm_gate_up", kind(4, 2.0, flops=4 * 1e15 * 0.5e-3))   # 1e15 flop/s x 0.5 ms each
    assert r["bound"] == "mfma" and r["achieved"] == pytest.approx(1000.0)
    assert r["frac"] == pytest.approx(1000.0 / bench.PEAK_BF16_TFLOPS, abs=1e-4)
    assert r["executed_tflops"] == pytest.approx(2000.0) and r["avg_launch_us"] == pytest.approx(500.0)
    f = bench.roofline("gemm_swiglu_f16", kind(2, 1.0, flops=2 * 0.25e12 * 0.5e-3 * 4))
    assert f["executed_tflops"] == pytest.approx(f["achieved"])
    h = bench.roofline("residual_norm", kind(10, 1.0, nbytes=10 * 4e12 * 0.1e-3))   # 4e12 B/s x 0.1 ms
    assert h["bound"] == "hbm" and h["achieved"] == pytest.approx(4000.0) and h["unit"] == "GB/s"


def test_traffic_only_from_a_summary_of_the_current_sources(bench, tmp_path, monkeypatch):
    """The stored traffic figure is reported only while its digest is the sources' own."""
    from vlm_shared_prefix_amd import profiling as PR
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    for digest, expect in ((PR.source_digest(), 1.5e8), ("0000000000000000", None)):
        (tmp_path / "profiles" / "gemm_down_f16_traffic.md").write_text(
            f"# t\n- traffic_bytes_per_launch: 1.5e8\n- source_digest: {digest}\n")
        assert bench.roofline("gemm_down_f16", kind(1, 1.0, flops=1e9))["traffic"] == expect


def test_step_roofline_takes_the_prefill_launches_of_a_shared_kind(bench):
    """The step's dominant kind, launched by both calls, is measured over the prefill's
    launches (one launch shape); the scoring call gets its own dominant kind's entry."""
    cfg = types.SimpleNamespace(prefix_len=1024, n_suffix=32)
    pre = {"gemm_swiglu_f16": kind(28, 28 * 0.3, flops=28 * 278e9), "gemm_down_f16": kind(28, 28 * 0.16, flops=1)}
    score = {"gemm_swiglu_f16": kind(28, 28 * 0.13, flops=28 * 103e9), "gemm_qkv": kind(28, 28 * 0.04, flops=1)}
    step = {k: kind(pre.get(k, kind(0, 0))["launches"] + score.get(k, kind(0, 0))["launches"],
                    pre.get(k, kind(0, 0))["ms"] + score.get(k, kind(0, 0))["ms"],
                    flops=pre.get(k, kind(0, 0))["flops"] + score.get(k, kind(0, 0))["flops"])
            for k in set(pre) | set(score)}
    roof, sroof = bench.step_rooflines(step, pre, score, cfg)
    assert roof["kernel"] == "gemm_swiglu_f16" and roof["launches"] == 28
    assert roof["avg_launch_us"] == pytest.approx(300.0)
    assert roof["achieved"] == pytest.approx(278e9 / 0.3e-3 / 1e12, rel=1e-4)
    assert roof["launches_of"].startswith("prefill")
    assert sroof["kernel"] == "gemm_swiglu_f16" and sroof["avg_launch_us"] == pytest.approx(130.0)
    assert sroof["launches_of"].startswith("scoring call")
    # a kind the prefill never launches is measured over the whole step
    only_score = {"attn_fwd": kind(28, 100.0, flops=28 * 1e9)}
    roof2, _ = bench.step_rooflines(only_score, {}, only_score, cfg)
    assert roof2["launches"] == 28 and "launches_of" not in roof2


def test_attention_entry_with_its_merge(bench):
    """MFMA utilisation of the attention alone and with its split merge; prefix-KV rate."""
    prof = {"attn_fwd": kind(10, 10 * 0.02, flops=10 * 5e9), "attn_merge": kind(10, 10 * 0.005)}
    e = bench.attention_entry(prof, 2.0e6, "x")
    assert e["achieved_tflops"] == pytest.approx(250.0) and e["mfma_util"] == pytest.approx(0.1)
    assert e["merge_avg_us"] == pytest.approx(5.0)
    assert e["with_merge_mfma_util"] == pytest.approx(5e9 / 25e-6 / 1e12 / bench.PEAK_BF16_TFLOPS, abs=1e-4)
    assert e["prefix_kv_gbs"] == pytest.approx(100.0)
    assert bench.attention_entry({}, 0, "x") is None
