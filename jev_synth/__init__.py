"""Seeded synthetic inputs for shared-prefix candidate scoring.

This module is the ONLY code shared by the CPU oracle and the HIP path.  It
draws numbers and nothing else: it holds none of the method's arithmetic
(no norm, no attention, no softmax, no readout).  Both sides call it with the
same (config, seed) and receive the same values.

Workload shapes follow the five synthetic configurations of the build target
(a tiny fp32 decoder, a Qwen2-VL-2B-shaped and a Qwen2.5-VL-7B-shaped bf16
decoder, a batch-size sweep and a prefix-tree candidate workload).  The pages
measure on real images and real weights (a COCO fixture and a movie frame on
the Ochevid Jev-VL 2B catalog page, "Evidence"; the FastJEV benchmarks, §4.1);
none of those are available, so random-init weights and N(0,1) "visual"
embeddings of the same shapes stand in for them.

Draw recipe (fixed, so every consumer sees identical values):
  * Generator: NumPy PCG64 seeded by SeedSequence([seed, stream, item, chunk]).
    Streams: 0 global tensors (embedding, final norm, LM head); 1+l layer l;
    1000 prefix inputs; 2000 suffixes and candidates; 3000 trees.
    Large tensors are drawn in row chunks of CHUNK_ROWS rows, each chunk from
    its own SeedSequence, so generation can run on several threads and stay
    bit-identical.
  * Matrices: 0.02 * N(0,1); norm gains: 1 + 0.02 * N(0,1); visual
    embeddings: N(0,1).  Everything is drawn in float32 and, for bf16
    configs, rounded to bfloat16 with round-to-nearest-even.  The float32
    arrays returned here are therefore exactly representable in bfloat16.
  * Token ids uniform in [0, vocab).  Suffix lengths uniform on the inclusive
    range.  Candidate ids distinct within one set.  Pad slots of right-padded
    arrays hold random junk ids (they must never be read).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np

CHUNK_ROWS = 4096

STREAM_GLOBAL = 0
STREAM_LAYER0 = 1
STREAM_PREFIX = 1000
STREAM_SUFFIX = 2000
STREAM_TREE = 3000
STREAM_IMAGES = 4000


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    mlp: int
    vocab: int
    rope_theta: float
    rms_eps: float
    dtype: str                    # "f32" or "bf16": storage type of weights / embeddings
    n_vis: int                    # visual prefix rows (given embeddings)
    n_text: int                   # text prefix rows (token ids)
    # flat suffix workload
    n_suffix: int = 0
    len_lo: int = 1
    len_hi: int = 1
    s_max: int = 1
    fixed_lens: Optional[tuple] = None
    n_cands: int = 2
    shared_cands: bool = False    # one candidate set for every suffix (Yes/No/Cannot style)
    # tree workload
    n_questions: int = 0
    stem_len: int = 0
    tree_cands: int = 0
    cand_len_lo: int = 1
    cand_len_hi: int = 1
    overlap: bool = False         # force shared candidate prefixes (trie merges fire)
    # one question over several images: n_images prefixes of n_vis visual rows each
    # (drawn in [vis_lo, n_vis] per image when vis_lo > 0: mixed image sizes) + n_text
    n_images: int = 0
    vis_lo: int = 0

    @property
    def prefix_len(self) -> int:
        return self.n_vis + self.n_text

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


_Q2B = dict(n_layers=28, hidden=1536, n_q_heads=12, n_kv_heads=2, head_dim=128,
            mlp=8960, vocab=151936, rope_theta=1e6, rms_eps=1e-6, dtype="bf16")
_Q7B = dict(n_layers=28, hidden=3584, n_q_heads=28, n_kv_heads=4, head_dim=128,
            mlp=18944, vocab=152064, rope_theta=1e6, rms_eps=1e-6, dtype="bf16")

CONFIGS: Dict[str, Config] = {
    # tiny fp32 decoder, fixed suffix lengths 5,7,8,6 padded to 8
    "c1": Config("c1", n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                 mlp=688, vocab=1024, rope_theta=1e4, rms_eps=1e-6, dtype="f32",
                 n_vis=48, n_text=16, n_suffix=4, fixed_lens=(5, 7, 8, 6), s_max=8,
                 n_cands=3),
    # Qwen2-VL-2B shape
    "c2": Config("c2", **_Q2B, n_vis=400, n_text=20, n_suffix=8, len_lo=8, len_hi=20,
                 s_max=20, n_cands=3),
    # Qwen2.5-VL-7B shape: the headline workload
    "c3": Config("c3", **_Q7B, n_vis=1000, n_text=24, n_suffix=32, len_lo=6, len_hi=16,
                 s_max=16, n_cands=2),
    # batch sweep on the 2B shape: a pool of 100 suffixes, B takes the first B
    "c4": Config("c4", **_Q2B, n_vis=1280, n_text=16, n_suffix=100, len_lo=8, len_hi=24,
                 s_max=24, n_cands=3),
    # prefix-tree candidates on the 7B shape, 8192-position visual prefix
    "c5": Config("c5", **_Q7B, n_vis=8192, n_text=0, n_questions=16, stem_len=12,
                 tree_cands=4, cand_len_lo=1, cand_len_hi=4, s_max=12),
    # ---- reduced-size variants used by parity tests (same head structure) ----
    # 2B head structure (G=6, D=128), 2 layers, ragged suffixes incl. length 1
    "m2": Config("m2", n_layers=2, hidden=1536, n_q_heads=12, n_kv_heads=2, head_dim=128,
                 mlp=1024, vocab=4096, rope_theta=1e6, rms_eps=1e-6, dtype="bf16",
                 n_vis=90, n_text=10, n_suffix=7, len_lo=1, len_hi=20, s_max=24, n_cands=3),
    # 7B head structure (G=7, D=128), 2 layers
    "m7": Config("m7", n_layers=2, hidden=3584, n_q_heads=28, n_kv_heads=4, head_dim=128,
                 mlp=1024, vocab=4096, rope_theta=1e6, rms_eps=1e-6, dtype="bf16",
                 n_vis=290, n_text=10, n_suffix=9, len_lo=1, len_hi=16, s_max=16, n_cands=2),
    # 7B head structure with long suffixes: a row tile's own keys span several 64-key tiles,
    # a ragged prefix (300), and key-tile splits that cut through the own-key tiles
    "m7l": Config("m7l", n_layers=2, hidden=3584, n_q_heads=28, n_kv_heads=4, head_dim=128,
                  mlp=1024, vocab=4096, rope_theta=1e6, rms_eps=1e-6, dtype="bf16",
                  n_vis=290, n_text=10, n_suffix=5, len_lo=60, len_hi=200, s_max=200, n_cands=2),
    # tree workload on the 7B head structure, forced candidate overlap
    "m5": Config("m5", n_layers=2, hidden=3584, n_q_heads=28, n_kv_heads=4, head_dim=128,
                 mlp=1024, vocab=4096, rope_theta=1e6, rms_eps=1e-6, dtype="bf16",
                 n_vis=150, n_text=0, n_questions=4, stem_len=5, tree_cands=4,
                 cand_len_lo=1, cand_len_hi=4, s_max=8, overlap=True),
    # one question over 8 images on the 7B shape: 8 prefixes of 1000 visual + 24 text rows
    "c6": Config("c6", **_Q7B, n_vis=1000, n_text=24, n_images=8, len_lo=6, len_hi=16, s_max=16,
                 n_cands=3),
    # one question over 3 images of mixed sizes, 7B head structure, 2 layers
    "mi7": Config("mi7", n_layers=2, hidden=3584, n_q_heads=28, n_kv_heads=4, head_dim=128,
                  mlp=1024, vocab=4096, rope_theta=1e6, rms_eps=1e-6, dtype="bf16",
                  n_vis=230, n_text=10, n_images=3, vis_lo=60, len_lo=1, len_hi=16, s_max=16, n_cands=3),
    # one question over 3 images of mixed sizes on the tiny fp32 decoder
    "mi1": Config("mi1", n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                  mlp=688, vocab=1024, rope_theta=1e4, rms_eps=1e-6, dtype="f32",
                  n_vis=48, n_text=16, n_images=3, vis_lo=10, len_lo=5, len_hi=7, s_max=8, n_cands=3),
    # bf16 decoder with 64-dim heads (G=4), 2 layers: suffixes and a tree workload
    "m64": Config("m64", n_layers=2, hidden=1024, n_q_heads=16, n_kv_heads=4, head_dim=64,
                  mlp=1024, vocab=4096, rope_theta=1e6, rms_eps=1e-6, dtype="bf16",
                  n_vis=150, n_text=10, n_suffix=6, len_lo=1, len_hi=20, s_max=24, n_cands=3,
                  n_questions=4, stem_len=5, tree_cands=4, cand_len_lo=1, cand_len_hi=4, overlap=True),
    # edge shapes of the few-row product: hidden 320 (ragged 128-column tiles), MLP 832 (the
    # down projection's last K split is a single 64-wide stage, q|k|v an odd stage count),
    # one suffix of one token (a single row)
    "mk": Config("mk", n_layers=2, hidden=320, n_q_heads=5, n_kv_heads=1, head_dim=64,
                 mlp=832, vocab=1024, rope_theta=1e6, rms_eps=1e-6, dtype="bf16",
                 n_vis=40, n_text=8, n_suffix=4, fixed_lens=(1, 7, 10, 4), s_max=10, n_cands=3),
    # 7B head structure (G=7) with 64-dim heads over a 2560-key prefix and 470 suffix rows: 108
    # row tiles of 41 key tiles, where equal key splits would leave the chip unevenly loaded,
    # so the attention takes the balanced schedule (two-term q past 2048 keys)
    "mb": Config("mb", n_layers=1, hidden=512, n_q_heads=28, n_kv_heads=4, head_dim=64,
                 mlp=512, vocab=2048, rope_theta=1e6, rms_eps=1e-6, dtype="bf16",
                 n_vis=2540, n_text=20, n_suffix=32,
                 fixed_lens=(1, 29, 14, 23, 17, 17, 22, 15, 12, 18, 6, 25, 16, 11, 19, 8,
                             13, 20, 2, 24, 15, 10, 21, 7, 16, 14, 23, 5, 12, 18, 9, 8),
                 s_max=29, n_cands=3),
    # fp32 tree workload on the tiny decoder (oracle pins and fp32 parity)
    "t1": Config("t1", n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                 mlp=688, vocab=1024, rope_theta=1e4, rms_eps=1e-6, dtype="f32",
                 n_vis=48, n_text=16, n_questions=3, stem_len=4, tree_cands=4,
                 cand_len_lo=1, cand_len_hi=4, s_max=6, overlap=True),
}

C4_BATCHES = (1, 2, 4, 8, 32, 100)


def with_overrides(cfg: Config, **kw) -> Config:
    return dataclasses.replace(cfg, **kw)


# ----------------------------------------------------------------------------
# primitive draws
# ----------------------------------------------------------------------------
def _rng(seed: int, stream: int, item: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, item, chunk])))


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Re-encode bfloat16-exact float32 values as raw bfloat16 bits (uint16). Lossless."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("array is not bfloat16-representable")
    return (u >> np.uint32(16)).astype(np.uint16)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _normal(shape, seed, stream, item, scale, offset, dtype, pool=None) -> np.ndarray:
    """offset + scale * N(0,1) in float32, drawn in row chunks; bf16-rounded if asked."""
    shape = tuple(int(s) for s in shape)
    rows = shape[0]
    cols = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    out = np.empty((rows, cols), dtype=np.float32)
    n_chunks = (rows + CHUNK_ROWS - 1) // CHUNK_ROWS
    s32 = np.float32(scale)
    o32 = np.float32(offset)

    def work(c):
        r0 = c * CHUNK_ROWS
        r1 = min(rows, r0 + CHUNK_ROWS)
        blk = _rng(seed, stream, item, c).standard_normal((r1 - r0, cols), dtype=np.float32)
        if scale != 1.0:
            blk *= s32
        if offset != 0.0:
            blk += o32
        if dtype == "bf16":
            blk = round_bf16(blk)
        out[r0:r1] = blk

    if n_chunks > 1:
        if pool is not None:
            list(pool.map(work, range(n_chunks)))
        else:
            with ThreadPoolExecutor(_threads()) as ex:
                list(ex.map(work, range(n_chunks)))
    else:
        work(0)
    return out.reshape(shape)


# ----------------------------------------------------------------------------
# weights
# ----------------------------------------------------------------------------
LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")


def layer_shapes(cfg: Config):
    H, D = cfg.hidden, cfg.head_dim
    return {
        "attn_norm": (H,),
        "wq": (cfg.n_q_heads * D, H),
        "wk": (cfg.n_kv_heads * D, H),
        "wv": (cfg.n_kv_heads * D, H),
        "wo": (H, cfg.n_q_heads * D),
        "mlp_norm": (H,),
        "w_gate": (cfg.mlp, H),
        "w_up": (cfg.mlp, H),
        "w_down": (H, cfg.mlp),
    }


def weights_global(cfg: Config, seed: int, pool=None) -> Dict[str, np.ndarray]:
    """Token embedding [V,H], final norm gain [H], untied LM head [V,H] (float32 values)."""
    V, H = cfg.vocab, cfg.hidden
    return {
        "embed": _normal((V, H), seed, STREAM_GLOBAL, 0, 0.02, 0.0, cfg.dtype, pool),
        "final_norm": _normal((H,), seed, STREAM_GLOBAL, 1, 0.02, 1.0, cfg.dtype, pool),
        "lm_head": _normal((V, H), seed, STREAM_GLOBAL, 2, 0.02, 0.0, cfg.dtype, pool),
    }


def weights_layer(cfg: Config, seed: int, layer: int, pool=None) -> Dict[str, np.ndarray]:
    """One decoder layer's parameters, row-major [out, in] matrices (float32 values)."""
    shapes = layer_shapes(cfg)
    out = {}
    for item, key in enumerate(LAYER_KEYS):
        is_gain = key.endswith("_norm")
        out[key] = _normal(shapes[key], seed, STREAM_LAYER0 + layer, item,
                           0.02, 1.0 if is_gain else 0.0, cfg.dtype, pool)
    return out


def iter_layers(cfg: Config, seed: int, workers: int = 0):
    """Yield (l, weights_layer(cfg, seed, l)) in order, drawing up to `workers` layers ahead."""
    workers = workers or _threads()
    if cfg.n_layers == 0:
        return
    with ThreadPoolExecutor(workers) as ex:
        futs = {}
        nxt = 0
        for l in range(cfg.n_layers):
            while nxt < cfg.n_layers and nxt < l + workers:
                futs[nxt] = ex.submit(weights_layer, cfg, seed, nxt)
                nxt += 1
            yield l, futs.pop(l).result()


class WeightSource:
    """Lazy, cached access to a model's weights: .glob and .layer(l)."""

    def __init__(self, cfg: Config, seed: int, cache_layers: bool = True):
        self.cfg, self.seed = cfg, seed
        self._cache_layers = cache_layers
        self._layers: Dict[int, Dict[str, np.ndarray]] = {}
        self._glob = None

    @property
    def glob(self) -> Dict[str, np.ndarray]:
        if self._glob is None:
            self._glob = weights_global(self.cfg, self.seed)
        return self._glob

    def layer(self, l: int) -> Dict[str, np.ndarray]:
        if l in self._layers:
            return self._layers[l]
        w = weights_layer(self.cfg, self.seed, l)
        if self._cache_layers:
            self._layers[l] = w
        return w

    def drop_layer(self, l: int) -> None:
        self._layers.pop(l, None)


# ----------------------------------------------------------------------------
# request inputs
# ----------------------------------------------------------------------------
def prefix_inputs(cfg: Config, seed: int) -> Dict[str, np.ndarray]:
    """Visual prefix embeddings [n_vis,H] ~ N(0,1) and text prefix ids [n_text]."""
    vis = _normal((max(cfg.n_vis, 0), cfg.hidden), seed, STREAM_PREFIX, 0, 1.0, 0.0, cfg.dtype) \
        if cfg.n_vis > 0 else np.zeros((0, cfg.hidden), np.float32)
    ids = _rng(seed, STREAM_PREFIX, 1).integers(0, cfg.vocab, size=cfg.n_text).astype(np.int32)
    return {"vis": vis, "text_ids": ids}


def suffix_inputs(cfg: Config, seed: int, n: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Right-padded suffix ids [B,S_max], lengths [B], candidate ids [B,C], counts [B].

    The full pool of cfg.n_suffix suffixes is always drawn; `n` takes the first n,
    so a smaller batch is a prefix of a larger one.
    """
    B = cfg.n_suffix
    rng = _rng(seed, STREAM_SUFFIX, 0)
    if cfg.fixed_lens is not None:
        lens = np.asarray(cfg.fixed_lens, dtype=np.int32)
    else:
        lens = rng.integers(cfg.len_lo, cfg.len_hi + 1, size=B).astype(np.int32)
    ids = rng.integers(0, cfg.vocab, size=(B, cfg.s_max)).astype(np.int32)   # junk in pads
    C = cfg.n_cands
    if cfg.shared_cands:
        one = rng.choice(cfg.vocab, size=C, replace=False).astype(np.int32)
        cands = np.tile(one, (B, 1))
    else:
        cands = np.stack([rng.choice(cfg.vocab, size=C, replace=False) for _ in range(B)]).astype(np.int32)
    n_cands = np.full(B, C, dtype=np.int32)
    if n is not None:
        ids, lens, cands, n_cands = ids[:n], lens[:n], cands[:n], n_cands[:n]
    return {"ids": np.ascontiguousarray(ids), "lens": np.ascontiguousarray(lens),
            "cands": np.ascontiguousarray(cands), "n_cands": np.ascontiguousarray(n_cands)}


def images_inputs(cfg: Config, seed: int) -> Dict[str, object]:
    """One typed question over cfg.n_images images.

    images[i] = {"vis": [n_vis_i, H], "text_ids": [n_text]} (the instruction text is the
    same for every image; n_vis_i = n_vis, or drawn in [vis_lo, n_vis]); seg_lens [n];
    the question as a suffix batch of n identical rows (ids [n, S_max], lens, cands,
    n_cands) with seg = [0, 1, ..., n-1]: row i asks it of image i.
    """
    n = cfg.n_images
    rng = _rng(seed, STREAM_IMAGES, 0)
    text = rng.integers(0, cfg.vocab, size=cfg.n_text).astype(np.int32)
    nv = [cfg.n_vis if cfg.vis_lo <= 0 else int(rng.integers(cfg.vis_lo, cfg.n_vis + 1)) for _ in range(n)]
    images = []
    for i in range(n):
        vis = _normal((nv[i], cfg.hidden), seed, STREAM_IMAGES, 1 + i, 1.0, 0.0, cfg.dtype) \
            if nv[i] > 0 else np.zeros((0, cfg.hidden), np.float32)
        images.append({"vis": vis, "text_ids": text.copy()})
    q = _rng(seed, STREAM_IMAGES, 100000)
    L = int(q.integers(cfg.len_lo, cfg.len_hi + 1))
    ids = q.integers(0, cfg.vocab, size=cfg.s_max).astype(np.int32)      # junk past L
    cands = q.choice(cfg.vocab, size=cfg.n_cands, replace=False).astype(np.int32)
    suf = {"ids": np.ascontiguousarray(np.tile(ids, (n, 1))), "lens": np.full(n, L, np.int32),
           "cands": np.ascontiguousarray(np.tile(cands, (n, 1))), "n_cands": np.full(n, cfg.n_cands, np.int32)}
    return {"images": images, "seg_lens": np.array([v + cfg.n_text for v in nv], np.int32),
            "seg": np.arange(n, dtype=np.int32), "suf": suf}


def tree_inputs(cfg: Config, seed: int) -> Dict[str, np.ndarray]:
    """Question stems and multi-token candidates.

    stem_ids [Q,S_max] (right-padded), stem_lens [Q], cand_tok [Q,C,K_max]
    (right-padded), cand_lens [Q,C], n_cands [Q].  With cfg.overlap, candidate
    k+1 copies a leading run of candidate k with probability 1/2, and some
    candidates reuse a token under a different parent, so prefix merging has
    both kinds of cases to handle.
    """
    Q, C, K = cfg.n_questions, cfg.tree_cands, cfg.cand_len_hi
    rng = _rng(seed, STREAM_TREE, 0)
    stem_lens = np.full(Q, cfg.stem_len, dtype=np.int32)
    stem_ids = rng.integers(0, cfg.vocab, size=(Q, max(cfg.s_max, cfg.stem_len))).astype(np.int32)
    cand_lens = rng.integers(cfg.cand_len_lo, cfg.cand_len_hi + 1, size=(Q, C)).astype(np.int32)
    cand_tok = rng.integers(0, cfg.vocab, size=(Q, C, K)).astype(np.int32)
    if cfg.overlap:
        for q in range(Q):
            for c in range(1, C):
                if rng.random() < 0.5:
                    m = int(rng.integers(1, min(cand_lens[q, c - 1], cand_lens[q, c]) + 1))
                    cand_tok[q, c, :m] = cand_tok[q, c - 1, :m]
                elif cand_lens[q, c] >= 2 and rng.random() < 0.5:
                    # same token as another candidate's first token, but under a different parent
                    cand_tok[q, c, 1] = cand_tok[q, c - 1, 0]
        # one exact duplicate candidate, if there is room
        if Q > 0 and C >= 2:
            cand_lens[0, C - 1] = cand_lens[0, C - 2]
            cand_tok[0, C - 1] = cand_tok[0, C - 2]
    n_cands = np.full(Q, C, dtype=np.int32)
    return {"stem_ids": np.ascontiguousarray(stem_ids), "stem_lens": stem_lens,
            "cand_tok": np.ascontiguousarray(cand_tok), "cand_lens": cand_lens, "n_cands": n_cands}


def shared_tree_inputs(cfg: Config, seed: int, shared: int) -> Dict[str, np.ndarray]:
    """Trees with a controlled shared fraction: every candidate has cand_len_hi tokens and
    the candidates of a question agree on their first `shared` tokens (0 <= shared <
    cand_len_hi) and differ at the next one, so merging common histories saves exactly
    shared * (C - 1) rows per question.  Same layout as tree_inputs; stems as there."""
    Q, C, K = cfg.n_questions, cfg.tree_cands, cfg.cand_len_hi
    if not 0 <= shared < K:
        raise ValueError(f"shared must be in [0, {K})")
    if C > cfg.vocab:
        raise ValueError("more candidates than vocabulary ids")
    rng = _rng(seed, STREAM_TREE, 1 + shared)
    stem_lens = np.full(Q, cfg.stem_len, dtype=np.int32)
    stem_ids = rng.integers(0, cfg.vocab, size=(Q, max(cfg.s_max, cfg.stem_len))).astype(np.int32)
    cand_tok = rng.integers(0, cfg.vocab, size=(Q, C, K)).astype(np.int32)
    for q in range(Q):
        cand_tok[q, 1:, :shared] = cand_tok[q, 0, :shared]
        # first differing token: distinct across the question's candidates
        cand_tok[q, :, shared] = rng.choice(cfg.vocab, size=C, replace=False)
    cand_lens = np.full((Q, C), K, dtype=np.int32)
    n_cands = np.full(Q, C, dtype=np.int32)
    return {"stem_ids": np.ascontiguousarray(stem_ids), "stem_lens": stem_lens,
            "cand_tok": np.ascontiguousarray(cand_tok), "cand_lens": cand_lens, "n_cands": n_cands}
