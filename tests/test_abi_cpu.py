"""C-ABI checks that need no GPU: the library loads, exports every function
include/jev.h declares, validates arguments before any HIP call, and plans
suffix batches and candidate trees as the pages describe.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

import jev_synth as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "jev.h")
LIB = os.path.join(ROOT, "vlm_shared_prefix_amd", "libjev.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libjev.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(jev_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_function():
    lib = C.CDLL(LIB)
    names = declared_functions()
    assert len(names) >= 15
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    from vlm_shared_prefix_amd import jev as J
    assert set(J.EXPORTED) == set(names), set(names) ^ set(J.EXPORTED)


def _cfg(**kw):
    from vlm_shared_prefix_amd import jev as J
    base = dict(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128, mlp=512, vocab=1000,
                rope_theta=1e4, rms_eps=1e-6, dtype=J.JEV_BF16)
    base.update(kw)
    return J.make_config(**base)


def _fake_weights(n_layers):
    """Non-null dummy pointers: creation only records them (no HIP call)."""
    from vlm_shared_prefix_amd import jev as J
    arr = (J.jev_layer * max(n_layers, 1))()
    for i in range(n_layers):
        arr[i] = J.jev_layer(*([0x1000 + i] * 9))
    return J.jev_weights(0x100, 0x200, 0x300, arr), arr


def test_model_create_validation():
    from vlm_shared_prefix_amd import jev as J
    w, keep = _fake_weights(2)
    m = J.jev_model_create(_cfg(), w)
    assert m
    st = J.jev_get_stats(m)
    assert st == {"prefills": 0, "forwards": 0, "rows": 0, "launches": 0}
    J.jev_model_destroy(m)
    cases = [
        (dict(n_q_heads=5), J.JEV_E_UNSUPPORTED),          # Hq % Hkv
        (dict(head_dim=96), J.JEV_E_UNSUPPORTED),          # D in {64, 128}
        (dict(hidden=250), J.JEV_E_UNSUPPORTED),           # bf16 needs H % 64 == 0
        (dict(vocab=0), J.JEV_E_INVALID),
        (dict(dtype=7), J.JEV_E_INVALID),
        (dict(rope_theta=-1.0), J.JEV_E_INVALID),
    ]
    for kw, code in cases:
        with pytest.raises(J.JevError) as e:
            J.jev_model_create(_cfg(**kw), w)
        assert e.value.code == code, kw
    # float32 models accept head_dim 64 and any hidden size
    m = J.jev_model_create(_cfg(dtype=J.JEV_F32, head_dim=64, hidden=250, mlp=688), w)
    assert J.jev_prefix_bytes(m, 100) == 2 * 2 * 2 * 128 * 64 * 4
    J.jev_model_destroy(m)
    # bf16 models take head_dim 64 too; their float16 store keeps 128-dim heads (zero-padded)
    m = J.jev_model_create(_cfg(head_dim=64), w)
    assert J.jev_prefix_bytes(m, 100) == 2 * 2 * 2 * 128 * 128 * 2
    J.jev_model_destroy(m)
    bad = J.jev_weights(0, 0x200, 0x300, keep)
    with pytest.raises(J.JevError) as e:
        J.jev_model_create(_cfg(), bad)
    assert e.value.code == J.JEV_E_INVALID


@pytest.fixture
def model():
    from vlm_shared_prefix_amd import jev as J
    w, keep = _fake_weights(2)
    m = J.jev_model_create(_cfg(), w)
    yield m, keep
    J.jev_model_destroy(m)


class _FakeDev:
    """Stands in for a device tensor: a pointer and a size, never dereferenced on this path."""

    def __init__(self, nbytes, ptr=0x7000):
        self._n, self._p = nbytes, ptr

    def data_ptr(self):
        return self._p

    def numel(self):
        return self._n

    def element_size(self):
        return 1


def test_prefix_and_workspace_sizes(model):
    from vlm_shared_prefix_amd import jev as J
    m, _ = model
    # store = L * 2 * Hkv * round64(P) * D * 2 bytes (f16)
    assert J.jev_prefix_bytes(m, 100) == 2 * 2 * 2 * 128 * 128 * 2
    assert J.jev_prefix_bytes(m, 0) == 0
    a = J.jev_workspace_bytes(m, 100, 50, 4, 12)
    b = J.jev_workspace_bytes(m, 100, 100, 8, 24)
    assert 0 < a < b
    with pytest.raises(J.JevError) as e:
        J.jev_prefix_create(m, 100, _FakeDev(10))
    assert e.value.code == J.JEV_E_WORKSPACE
    with pytest.raises(J.JevError) as e:
        J.jev_prefix_create(m, 40000, _FakeDev(1 << 40))
    assert e.value.code == J.JEV_E_UNSUPPORTED


def test_mirror_and_skip_arguments(model):
    """Float16 mirror sizes per matrix group and the block-skip mask's checks (no HIP call)."""
    from vlm_shared_prefix_amd import jev as J
    m, _ = model
    # _cfg: 2 layers, H 256, Hq 4 / Hkv 2 x 128, I 512 -> per layer q 512x256, k/v 256x256, o 256x512,
    # gate/up 512x256, down 256x512 (bytes = 2 x elements, each 256-byte aligned) + a 256-byte flag
    per = {J.JEV_F16_QKV: 2 * (512 * 256 + 2 * 256 * 256), J.JEV_F16_O: 2 * 256 * 512,
           J.JEV_F16_GATE_UP: 2 * 2 * 512 * 256, J.JEV_F16_DOWN: 2 * 256 * 512}
    for g, b in per.items():
        assert J.jev_model_f16_bytes(m, g) == 2 * b + 256
    # the prefill-only bits mirror the same matrices
    for g, gp in ((J.JEV_F16_GATE_UP, J.JEV_F16_GATE_UP_PREFILL), (J.JEV_F16_QKV, J.JEV_F16_QKV_PREFILL),
                  (J.JEV_F16_O, J.JEV_F16_O_PREFILL), (J.JEV_F16_GATE_UP, J.JEV_F16_GATE_UP_SCORE)):
        assert J.jev_model_f16_bytes(m, gp) == J.jev_model_f16_bytes(m, g)
    assert J.jev_model_f16_bytes(m, J.JEV_F16_GATE_UP_PREFILL | J.JEV_F16_GATE_UP_SCORE) == \
        J.jev_model_f16_bytes(m, J.JEV_F16_GATE_UP)
    assert J.jev_model_f16_bytes(m, 256) == 0
    with pytest.raises(J.JevError) as e:
        J.jev_model_attach_f16(m, J.JEV_F16_DOWN, _FakeDev(100), stream=0)
    assert e.value.code == J.JEV_E_WORKSPACE
    J.jev_model_attach_f16(m, J.JEV_F16_DOWN, None, stream=0)   # detach: no HIP call
    assert J.jev_model_f16_groups(m) == 0
    with pytest.raises(J.JevError) as e:
        J.jev_model_set_skip(m, [1, 0, 1])                  # 3 flags for 2 layers
    assert e.value.code == J.JEV_E_INVALID
    J.jev_model_set_skip(m, [0, 1])
    J.jev_model_set_skip(m, None)


def test_score_validation_before_any_launch(model):
    """Every bad argument is rejected on the host; B = 0 does no work (Ochevid: all-skipped requests)."""
    from vlm_shared_prefix_amd import jev as J
    m, _ = model
    p = J.jev_prefix_create(m, 10, _FakeDev(J.jev_prefix_bytes(m, 10)))
    ws = _FakeDev(1 << 30)
    out = _FakeDev(1 << 20)
    ids = np.zeros((2, 4), np.int32)
    lens = np.array([4, 2], np.int32)
    cands = np.array([[1, 2], [3, 4]], np.int32)
    nc = np.array([2, 2], np.int32)
    bad = [
        (dict(lens=np.array([5, 2], np.int32)), J.JEV_E_INVALID),      # L_b > S_max
        (dict(lens=np.array([0, 2], np.int32)), J.JEV_E_INVALID),      # L_b < 1
        (dict(ids=np.full((2, 4), 1000, np.int32)), J.JEV_E_INVALID),  # id >= V
        (dict(cands=np.array([[1, -1], [3, 4]], np.int32)), J.JEV_E_INVALID),
        (dict(nc=np.array([3, 2], np.int32)), J.JEV_E_INVALID),        # n_cands > C_max
        (dict(nc=np.array([0, 2], np.int32)), J.JEV_E_INVALID),
        (dict(ids=np.zeros((2, 300), np.int32), lens=np.array([4, 2], np.int32)), J.JEV_E_UNSUPPORTED),
    ]
    for kw, code in bad:
        a = dict(ids=ids, lens=lens, cands=cands, nc=nc)
        a.update(kw)
        with pytest.raises(J.JevError) as e:
            J.jev_score_suffixes(p, a["ids"], a["lens"], a["cands"], a["nc"], out, ws, stream=0)
        assert e.value.code == code, kw
    # too small a workspace
    with pytest.raises(J.JevError) as e:
        J.jev_score_suffixes(p, ids, lens, cands, nc, out, _FakeDev(100), stream=0)
    assert e.value.code == J.JEV_E_WORKSPACE
    # B = 0: OK and nothing launched
    J.jev_score_suffixes(p, np.zeros((0, 4), np.int32), np.zeros(0, np.int32), np.zeros((0, 2), np.int32),
                         np.zeros(0, np.int32), None, None, stream=0)
    assert J.jev_get_stats(m)["launches"] == 0
    # prefill: counts must add up to the prefix length; ids in range
    with pytest.raises(J.JevError) as e:
        J.jev_prefill_prefix(p, _FakeDev(1), 3, np.zeros(5, np.int32), ws, stream=0)
    assert e.value.code == J.JEV_E_INVALID
    with pytest.raises(J.JevError) as e:
        J.jev_prefill_prefix(p, _FakeDev(1), 5, np.full(5, 5000, np.int32), ws, stream=0)
    assert e.value.code == J.JEV_E_INVALID
    J.jev_prefix_destroy(p)


def test_segment_validation(model):
    """Segmented prefixes (one question over several images): argument checks, and the
    single-prefix calls refuse a store of several segments (no HIP call on these paths)."""
    from vlm_shared_prefix_amd import jev as J
    m, _ = model
    kv = _FakeDev(J.jev_prefix_bytes(m, 30))
    for lens, code in (([], J.JEV_E_INVALID), ([4, -1], J.JEV_E_INVALID), ([1] * 65, J.JEV_E_UNSUPPORTED),
                       ([20000, 20000], J.JEV_E_UNSUPPORTED)):
        with pytest.raises(J.JevError) as e:
            J.jev_prefix_create_segments(m, np.array(lens, np.int32), _FakeDev(1 << 40))
        assert e.value.code == code, lens
    with pytest.raises(J.JevError) as e:
        J.jev_prefix_create_segments(m, np.array([10, 60], np.int32), kv)   # 70 rows: a larger store
    assert e.value.code == J.JEV_E_WORKSPACE
    p = J.jev_prefix_create_segments(m, np.array([10, 0, 20], np.int32), kv)
    ws, out = _FakeDev(1 << 30), _FakeDev(1 << 20)
    ids = np.zeros((2, 4), np.int32)
    lens = np.array([4, 2], np.int32)
    cands = np.array([[1, 2], [3, 4]], np.int32)
    nc = np.array([2, 2], np.int32)
    with pytest.raises(J.JevError) as e:                      # single-prefix calls refuse it
        J.jev_score_suffixes(p, ids, lens, cands, nc, out, ws, stream=0)
    assert e.value.code == J.JEV_E_INVALID and "jev_score_segments" in J.jev_last_error()
    with pytest.raises(J.JevError) as e:
        J.jev_prefill_prefix(p, _FakeDev(1), 10, np.zeros(20, np.int32), ws, stream=0)
    assert e.value.code == J.JEV_E_INVALID
    for seg in ([0, 3], [-1, 0]):                             # segment index out of range
        with pytest.raises(J.JevError) as e:
            J.jev_score_segments(p, np.array(seg, np.int32), ids, lens, cands, nc, out, ws, stream=0)
        assert e.value.code == J.JEV_E_INVALID, seg
    with pytest.raises(J.JevError) as e:                      # counts must fill every segment
        J.jev_prefill_segments(p, _FakeDev(1), np.array([5, 0, 20], np.int32), np.zeros(5, np.int32),
                               np.array([4, 0, 0], np.int32), ws, stream=0)
    assert e.value.code == J.JEV_E_INVALID
    with pytest.raises(J.JevError) as e:
        J.jev_prefill_segments(p, _FakeDev(1), np.array([5, 0, 20], np.int32), np.full(5, 5000, np.int32),
                               np.array([5, 0, 0], np.int32), ws, stream=0)
    assert e.value.code == J.JEV_E_INVALID                    # text id >= V
    J.jev_score_segments(p, np.zeros(0, np.int32), np.zeros((0, 4), np.int32), np.zeros(0, np.int32),
                         np.zeros((0, 2), np.int32), np.zeros(0, np.int32), None, None, stream=0)   # B = 0
    assert J.jev_get_stats(m)["launches"] == 0
    J.jev_prefix_destroy(p)


def _segment_tiles_reference(pseg, G):
    """Per 128-row block of the G*T query rows: the 64-key tile hull of its rows' prefix key
    ranges and the keys every one of its rows sees (plain loops)."""
    T = len(pseg)
    out = []
    for r0 in range(0, G * T, 128):
        rows = sorted({r // G for r in range(r0, min(G * T, r0 + 128))})
        rng = [pseg[t] for t in rows]
        nonempty = [(b, e) for b, e in rng if e > b]
        if nonempty:
            lo, hi = min(b for b, _ in nonempty), max(e for _, e in nonempty)
            tiles = (lo // 64, -(-hi // 64))
        else:
            tiles = (0, 0)
        vis = (max(b for b, _ in rng), min(e for _, e in rng))
        out.append([tiles[0], tiles[1], vis[0], vis[1]])
    return np.array(out, np.int32).reshape(-1, 4)


@pytest.mark.parametrize("seed", range(6))
def test_segment_tile_table(seed):
    """The attention's per-block segment table (host logic) against a plain reference, for
    random image layouts: mixed sizes, empty segments, grouped and shuffled suffix orders."""
    from vlm_shared_prefix_amd import jev as J
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 9))
    lens = rng.integers(0, 400, size=n)
    lens[rng.integers(0, n)] = 0 if n > 1 else lens[0]
    offs = np.concatenate([[0], np.cumsum(lens)])[:-1]
    B = int(rng.integers(1, 40))
    seg = rng.integers(0, n, size=B)
    if seed % 2 == 0:
        seg = np.sort(seg)
    L = rng.integers(1, 17, size=B)
    pseg = [(int(offs[s]), int(offs[s] + lens[s])) for s, l in zip(seg, L) for _ in range(l)]
    for G in (1, 6, 7):
        got, mx = J.jev_segment_plan_tiles(pseg, G)
        ref = _segment_tiles_reference(pseg, G)
        np.testing.assert_array_equal(got, ref)
        assert mx == int(np.max(ref[:, 1] - ref[:, 0]))
    with pytest.raises(J.JevError):
        J.jev_segment_plan_tiles([(5, 3)], 7)


@pytest.mark.parametrize("shape", [
    (858, 7, 4, 8192, 1),    # 7B-shaped flat tree rows over an 8192-key prefix: equal splits give 376 blocks
    (861, 7, 4, 8192, 2),
    (470, 7, 4, 2560, 1),    # the "mb" parity workload (equal splits: 216 blocks of 256)
    (470, 7, 4, 2560, 2),
    (700, 6, 2, 4096, 1),
    (2000, 6, 2, 2816, 2),
    (378, 7, 4, 1024, 1),    # 7B scoring rows over 1024 keys: equal splits (252 blocks)
    (282, 7, 4, 8192, 2),    # trie rows: equal splits fill the chip (512 blocks)
    (54, 7, 4, 8192, 1),
    (1600, 6, 2, 1296, 1),
])
def test_attention_balanced_schedule_covers_every_tile_once(shape):
    """The balanced attention schedule (the enumeration the kernel runs, from the library):
    every (KV head, row tile) item's nominal key tiles are processed exactly once, in block
    order, its partial slots are 0.. in block order and within n_split, the merge's slot count
    for the item is the number of blocks on it, exactly its final run is marked last, every
    block holds `chunk` tiles (the last block fewer) and the launch fits the resident blocks."""
    from vlm_shared_prefix_amd import jev as J
    T, G, Hkv, P, own = shape
    ns, chunk, blocks, spans = J.jev_attn_schedule(T, G, Hkv, P, own, False, 1 << 16)
    n_rt = -(-G * T // 128)
    nt_u = -(-P // 64) + own
    if chunk == 0:
        assert len(spans) == 0 and blocks == n_rt * Hkv * ns
        assert T not in (858, 861, 470)   # the flat tree rows and "mb" take the balanced schedule
        return
    assert blocks <= 512 and 16 <= chunk < nt_u and 2 <= ns <= 32
    seen = {}
    per_block = np.zeros(blocks, np.int64)
    prev = (-1, -1)
    for b, u, z, vb, ve, last, slots in spans.tolist():
        assert (b, u) > prev
        prev = (b, u)
        assert 0 <= u < n_rt * Hkv and 0 <= vb < ve <= nt_u
        per_block[b] += ve - vb
        seen.setdefault(u, []).append((b, z, vb, ve, last, slots))
    assert sorted(seen) == list(range(n_rt * Hkv))
    for u, runs in seen.items():
        assert [r[1] for r in runs] == list(range(len(runs))), u          # slots 0.. in block order
        assert len(runs) <= ns and all(r[5] == len(runs) for r in runs), u
        edges = [0] + [r[3] for r in runs]
        assert [r[2] for r in runs] == edges[:-1] and edges[-1] == nt_u, u   # tiles once, in order
        assert [r[4] for r in runs] == [0] * (len(runs) - 1) + [1], u
    assert np.all(per_block[:-1] == chunk) and 0 < per_block[-1] <= chunk
    # segmented prefixes keep equal splits
    assert J.jev_attn_schedule(T, G, Hkv, P, own, True)[1] == 0


def test_launch_only_calls_need_staged_metadata(model):
    """The launch-only (graph-capturable) scoring calls refuse a workspace whose staged
    metadata is not this request's; nothing is launched (no HIP call on this path)."""
    from vlm_shared_prefix_amd import jev as J
    m, _ = model
    p = J.jev_prefix_create(m, 10, _FakeDev(J.jev_prefix_bytes(m, 10)))
    ws, out = _FakeDev(1 << 30, ptr=0x9000), _FakeDev(1 << 20)
    ids = np.zeros((2, 4), np.int32)
    lens = np.array([4, 2], np.int32)
    cands = np.array([[1, 2], [3, 4]], np.int32)
    nc = np.array([2, 2], np.int32)
    with pytest.raises(J.JevError) as e:
        J.jev_score_suffixes_launch(p, ids, lens, cands, nc, out, ws, stream=0)
    assert e.value.code == J.JEV_E_INVALID and "metadata" in J.jev_last_error()
    tree = dict(stem_ids=np.ones((1, 3), np.int32), stem_lens=np.array([3], np.int32),
                cand_tok=np.array([[[1, 2], [1, 3]]], np.int32), cand_lens=np.array([[2, 2]], np.int32),
                n_cands=np.array([2], np.int32))
    with pytest.raises(J.JevError) as e:
        J.jev_score_tree_launch(p, tree["stem_ids"], tree["stem_lens"], tree["cand_tok"], tree["cand_lens"],
                                tree["n_cands"], 0, out, None, ws, stream=0)
    assert e.value.code == J.JEV_E_INVALID
    # argument checks come first, as in the staging calls
    with pytest.raises(J.JevError) as e:
        J.jev_score_suffixes_launch(p, ids, np.array([5, 2], np.int32), cands, nc, out, ws, stream=0)
    assert e.value.code == J.JEV_E_INVALID and "metadata" not in J.jev_last_error()
    assert J.jev_get_stats(m)["launches"] == 0
    J.jev_prefix_destroy(p)


# ---------------------------------------------------------------- tree planning
def reference_trie(tree, mode):
    """Independent pure-Python packer: rows (token, depth, group), visibility and predictor rows."""
    Q, C, K = tree["cand_tok"].shape
    rows, target = [], {}
    for q in range(Q):
        s = int(tree["stem_lens"][q])
        stem = [int(x) for x in tree["stem_ids"][q, :s]]

        def chain(tokens, depth0, parent, group, anc):
            out = []
            for i, tkn in enumerate(tokens):
                rows.append({"tok": tkn, "depth": depth0 + i, "group": group, "anc": set(anc) | {len(rows)}})
                anc = rows[-1]["anc"]
                out.append(len(rows) - 1)
            return out

        n = int(tree["n_cands"][q])
        if mode != 2:
            g = q
            stem_rows = chain(stem, 0, None, g, set())
            last = stem_rows[-1]
            children = {}
        for c in range(n):
            Kc = int(tree["cand_lens"][q, c])
            w = [int(x) for x in tree["cand_tok"][q, c, :Kc]]
            if mode == 2:
                g = ("flat", q, c)
                stem_rows = chain(stem, 0, None, g, set())
                last = stem_rows[-1]
                children = {}
            parent = last
            for k in range(Kc):
                target[(q, c, k)] = parent
                if k == Kc - 1:
                    break
                key = (parent, w[k])
                if mode == 0 and key in children:
                    parent = children[key]
                    continue
                rows.append({"tok": w[k], "depth": s + k, "group": g, "anc": rows[parent]["anc"] | {len(rows)}})
                if mode == 0:
                    children[key] = len(rows) - 1
                parent = len(rows) - 1
    return rows, target


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("name,seed", [("t1", 1), ("m5", 0), ("c5", 0)])
def test_tree_plan_matches_reference(name, seed, mode):
    from vlm_shared_prefix_amd import jev as J
    tree = S.tree_inputs(S.CONFIGS[name], seed)
    plan = J.jev_tree_plan_rows(tree["stem_ids"], tree["stem_lens"], tree["cand_tok"], tree["cand_lens"],
                                tree["n_cands"], mode)
    rows, target = reference_trie(tree, mode)
    assert len(plan["tok"]) == len(rows)
    np.testing.assert_array_equal(plan["tok"], [r["tok"] for r in rows])
    np.testing.assert_array_equal(plan["depth"], [r["depth"] for r in rows])
    # groups: same partition of rows
    ref_g = [r["group"] for r in rows]
    for i in range(len(rows)):
        for j in range(i + 1, min(len(rows), i + 70)):
            assert (plan["group"][i] == plan["group"][j]) == (ref_g[i] == ref_g[j])
    # visibility: bit j of row r <-> row (group start + j) is an ancestor-or-self of r
    start = {}
    for i, g in enumerate(plan["group"]):
        start.setdefault(int(g), i)
    for r, row in enumerate(rows):
        s0 = start[int(plan["group"][r])]
        vis = {s0 + b for b in range(64) if (int(plan["mask"][r]) >> b) & 1}
        assert vis == row["anc"], r
    Q, C, K = tree["cand_tok"].shape
    for q in range(Q):
        for c in range(C):
            for k in range(K):
                want = target.get((q, c, k), -1)
                assert plan["target_row"][q, c, k] == want


@pytest.mark.parametrize("shared", [0, 1, 2, 3])
def test_tree_plan_sizes_shared_fraction(shared):
    """Trees whose candidates share their first `shared` tokens (the 7B tree workload's
    shape): a candidate of K tokens is predicted by its stem's last row and K - 1 rows of its
    own tokens, so per question the trie feeds stem + shared + C (K - 1 - shared) rows,
    stem-only stem + C (K - 1) and flat C (stem + K - 1)."""
    from vlm_shared_prefix_amd import jev as J
    cfg = S.CONFIGS["c5"]
    tree = S.shared_tree_inputs(cfg, 0, shared)
    Q, C, K, st = cfg.n_questions, cfg.tree_cands, cfg.cand_len_hi, cfg.stem_len
    want = {0: Q * (st + shared + C * (K - 1 - shared)), 1: Q * (st + C * (K - 1)), 2: Q * C * (st + K - 1)}
    got = {m: J.jev_tree_plan_size(tree["stem_ids"], tree["stem_lens"], tree["cand_tok"], tree["cand_lens"],
                                   tree["n_cands"], m)[0] for m in (0, 1, 2)}
    assert got == want
    rows, _ = reference_trie(tree, 0)
    assert len(rows) == want[0]


def test_trie_merges_only_same_parent_and_token():
    """Equal tokens after different histories stay separate ("FastJEV" §3.3)."""
    from vlm_shared_prefix_amd import jev as J
    stem = np.array([[7, 8]], np.int32)
    cand = np.array([[[1, 2, 3], [1, 2, 4], [5, 2, 3], [1, 2, 3]]], np.int32)
    lens = np.array([[3, 3, 3, 3]], np.int32)
    nc = np.array([4], np.int32)
    sizes = {m: J.jev_tree_plan_size(stem, np.array([2], np.int32), cand, lens, nc, m)[0] for m in (0, 1, 2)}
    # trie: stem 2 + {1, 1->2} shared by cands 0,1,3 + {5, 5->2} for cand 2  = 6 rows
    # stem-only: 2 + 4 * 2 = 10 rows; flat: 4 * (2 + 2) = 16 rows
    assert sizes == {0: 6, 1: 10, 2: 16}
    plan = J.jev_tree_plan_rows(stem, np.array([2], np.int32), cand, lens, nc, 0)
    # identical candidates 0 and 3 share every predictor row
    np.testing.assert_array_equal(plan["target_row"][0, 0], plan["target_row"][0, 3])
    # token 2 under parent 1 and under parent 5 are different rows
    assert plan["target_row"][0, 0, 2] != plan["target_row"][0, 2, 2]


def test_tree_validation():
    from vlm_shared_prefix_amd import jev as J
    stem = np.zeros((1, 70), np.int32)
    cand = np.zeros((1, 1, 2), np.int32)
    with pytest.raises(J.JevError) as e:
        J.jev_tree_plan_size(stem, np.array([70], np.int32), cand, np.array([[2]], np.int32),
                             np.array([1], np.int32), 0)
    assert e.value.code == J.JEV_E_UNSUPPORTED          # S_max > 64
    stem = np.zeros((1, 60), np.int32)
    cand = np.zeros((1, 3, 4), np.int32)
    cand[0, :, 0] = [1, 2, 3]
    with pytest.raises(J.JevError) as e:                 # group of 60 + 3*3 rows > 64
        J.jev_tree_plan_size(stem, np.array([60], np.int32), cand, np.full((1, 3), 4, np.int32),
                             np.array([3], np.int32), 1)
    assert e.value.code == J.JEV_E_UNSUPPORTED
    with pytest.raises(J.JevError) as e:
        J.jev_tree_plan_size(stem, np.array([60], np.int32), cand, np.full((1, 3), 4, np.int32),
                             np.array([3], np.int32), 5)
    assert e.value.code == J.JEV_E_INVALID


def test_failed_attach_leaves_model_detached(model):
    """An attach that fails once the conversion has begun (here: no device to convert on)
    leaves every GEMM on the two-term path."""
    import torch
    from vlm_shared_prefix_amd import jev as J
    if torch.cuda.device_count() > 0:
        pytest.skip("exercises the failure of the conversion launch on a host without a GPU")
    m, _ = model
    nb = J.jev_model_f16_bytes(m, J.JEV_F16_DOWN | J.JEV_F16_QKV)
    with pytest.raises(J.JevError) as e:
        J.jev_model_attach_f16(m, J.JEV_F16_DOWN | J.JEV_F16_QKV, _FakeDev(nb), stream=0)
    assert e.value.code == J.JEV_E_HIP
    assert J.jev_model_f16_groups(m) == 0


def test_attn_q_terms_and_flags_arguments(model):
    """The q-terms setting takes 0, 1 or 2; the flag read rejects null arguments (no HIP call)."""
    from vlm_shared_prefix_amd import jev as J
    m, _ = model
    for t in (0, 1, 2, 0):
        J.jev_model_set_attn_q_terms(m, t)
    with pytest.raises(J.JevError) as e:
        J.jev_model_set_attn_q_terms(m, 3)
    assert e.value.code == J.JEV_E_INVALID
    with pytest.raises(J.JevError) as e:
        J.jev_workspace_flags(None, stream=0)
    assert e.value.code == J.JEV_E_INVALID


def test_one_hip_runtime_in_process():
    """Importing the binding before torch must not leave two HIP runtimes in the process (the
    library's runtime would not know torch's device buffers)."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r); from vlm_shared_prefix_amd import jev; import torch; "
            "print(sorted(set(l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l)))" % ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    libs = eval(r.stdout.strip().splitlines()[-1])
    assert len(libs) == 1, libs
