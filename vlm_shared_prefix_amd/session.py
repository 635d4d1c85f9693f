"""Device-side convenience around the C-ABI: upload weights, own the prefix KV
store and the workspace, call the three hot-path entry points.

Marshalling only: tensors are torch device buffers, every computation is a
call into libjev.so.  Weights and inputs come as NumPy float32 arrays (for
bfloat16 models they must be bfloat16-representable, as the seeded generator
produces them).
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import jev as J

LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")


def to_device(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """float32 array -> device tensor holding float32 values or raw bfloat16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return torch.from_numpy(a).to(device)
    u = a.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("array is not bfloat16-representable")
    bits = (u >> np.uint32(16)).astype(np.uint16).view(np.int16)
    return torch.from_numpy(bits).to(device)


# mirrored matrix groups per precision mode
PRECISIONS = {"split": 0, "f16_gu": J.JEV_F16_GATE_UP, "f16_down": J.JEV_F16_DOWN,
              "f16_o": J.JEV_F16_O, "f16_out": J.JEV_F16_DOWN | J.JEV_F16_O,
              "f16_mlp": J.JEV_F16_GATE_UP | J.JEV_F16_DOWN,
              "f16_down_gup": J.JEV_F16_DOWN | J.JEV_F16_GATE_UP_PREFILL,
              "f16_prefill": J.JEV_F16_DOWN | J.JEV_F16_GATE_UP_PREFILL | J.JEV_F16_QKV_PREFILL | J.JEV_F16_O_PREFILL,
              "f16_score_gup": J.JEV_F16_DOWN | J.JEV_F16_GATE_UP_SCORE | J.JEV_F16_QKV_PREFILL | J.JEV_F16_O_PREFILL,
              "f16_down_gup_o": J.JEV_F16_DOWN | J.JEV_F16_GATE_UP_PREFILL | J.JEV_F16_O_PREFILL,
              "f16_down_gup_qkv": J.JEV_F16_DOWN | J.JEV_F16_GATE_UP_PREFILL | J.JEV_F16_QKV_PREFILL,
              "f16": J.JEV_F16_GATE_UP | J.JEV_F16_QKV | J.JEV_F16_DOWN | J.JEV_F16_O}
DEFAULT_PRECISION = "f16_score_gup"


class Session:
    """A model on one device plus a prefix and a reusable workspace."""

    def __init__(self, cfg, glob: Dict[str, np.ndarray], layers, device="cuda:0", precision: str = DEFAULT_PRECISION):
        """precision (bf16 models): "split" runs every GEMM on two bfloat16 terms of the activation;
        "f16_gu", "f16_down", "f16_mlp" run the gate|up, the down, or both MLP GEMMs as single
        float16 passes on a float16 mirror of their weights; "f16" does so for every decoder GEMM;
        "f16_down_gup" runs the down projection on one float16 pass everywhere and gate|up on
        one float16 pass in prefills only (scoring calls keep its two terms); "f16_down_gup_o"
        also runs o on one float16 pass in prefills; "f16_prefill" (the default) every prefill
        GEMM, q|k|v only for prefixes of at most 2048 rows (the library's rule); "f16_score_gup"
        as "f16_prefill" with gate|up on one float16 pass in suffix-scoring calls too (tree calls
        keep its two terms)."""
        if precision not in PRECISIONS:
            raise ValueError(f"precision must be one of {PRECISIONS}, not {precision!r}")
        self.cfg = cfg
        self.device = torch.device(device)
        self.dtype = J.JEV_BF16 if cfg.dtype == "bf16" else J.JEV_F32
        dev = self.device
        self.glob = {k: to_device(v, cfg.dtype, dev) for k, v in glob.items()}
        self.layers = []
        for l in range(cfg.n_layers):
            W = layers(l) if callable(layers) else layers[l]
            self.layers.append({k: to_device(W[k], cfg.dtype, dev) for k in LAYER_KEYS})
        self.jcfg = J.make_config(cfg.n_layers, cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
                                  cfg.mlp, cfg.vocab, cfg.rope_theta, cfg.rms_eps, self.dtype)
        self.jw, self._keep = J.make_weights(self.glob["embed"], self.glob["final_norm"], self.glob["lm_head"],
                                             self.layers)
        self.model = J.jev_model_create(self.jcfg, self.jw)
        self.mirror = None
        self.precision = precision if self.dtype == J.JEV_BF16 else "f32"
        groups = PRECISIONS[precision] if self.dtype == J.JEV_BF16 else 0
        if groups:
            self.mirror = torch.empty(J.jev_model_f16_bytes(self.model, groups), dtype=torch.uint8, device=dev)
            J.jev_model_attach_f16(self.model, groups, self.mirror)
        self.prefix = None
        self.kv = None
        self.P = 0
        self.ws = None

    @classmethod
    def generated(cls, cfg, seed, device="cuda:0", precision: str = DEFAULT_PRECISION):
        """Draw the seeded weights (several layers at a time) and upload them layer by layer."""
        import jev_synth as S
        glob = S.weights_global(cfg, seed)
        it = S.iter_layers(cfg, seed)
        cache = {}

        def get(l):
            while l not in cache:
                k, W = next(it)
                cache[k] = W
            return cache.pop(l)
        return cls(cfg, glob, get, device, precision)

    # ------------------------------------------------------------------ buffers
    def workspace(self, nbytes: int) -> torch.Tensor:
        if self.ws is None or self.ws.numel() < nbytes:
            self.ws = None
            torch.cuda.synchronize(self.device)
            self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.ws

    def close(self):
        if self.prefix:
            J.jev_prefix_destroy(self.prefix)
            self.prefix = None
        if self.model:
            J.jev_model_destroy(self.model)
            self.model = None
        self.mirror = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------------ calls
    def prefill(self, vis: np.ndarray, text_ids: np.ndarray, stream=None):
        P = int(vis.shape[0]) + int(len(text_ids))
        if self.prefix:
            J.jev_prefix_destroy(self.prefix)
            self.prefix = None
        nb = J.jev_prefix_bytes(self.model, P)
        self.kv = torch.empty(max(nb, 256), dtype=torch.uint8, device=self.device)
        self.prefix = J.jev_prefix_create(self.model, P, self.kv)
        self.P = P
        self.vis = to_device(vis, self.cfg.dtype, self.device) if vis.shape[0] else None
        ws = self.workspace(J.jev_workspace_bytes(self.model, P, max(P, 1), 1, 0))
        J.jev_prefill_prefix(self.prefix, self.vis, int(vis.shape[0]), text_ids, ws, stream)

    def prefill_segments(self, images, stream=None):
        """One segmented prefix holding every image's prefix (images[i]: "vis", "text_ids"),
        prefilled in one batched forward."""
        if self.prefix:
            J.jev_prefix_destroy(self.prefix)
            self.prefix = None
        n_vis = np.array([im["vis"].shape[0] for im in images], np.int32)
        n_text = np.array([len(im["text_ids"]) for im in images], np.int32)
        seg_lens = n_vis + n_text
        P = int(seg_lens.sum())
        self.kv = torch.empty(max(J.jev_prefix_bytes(self.model, P), 256), dtype=torch.uint8, device=self.device)
        self.prefix = J.jev_prefix_create_segments(self.model, seg_lens, self.kv)
        self.P = P
        vis = np.concatenate([im["vis"] for im in images], axis=0)
        self.vis = to_device(vis, self.cfg.dtype, self.device) if vis.shape[0] else None
        text = np.concatenate([np.asarray(im["text_ids"], np.int32) for im in images])
        ws = self.workspace(J.jev_workspace_bytes(self.model, P, max(P, 1), 1, 0))
        J.jev_prefill_segments(self.prefix, self.vis, n_vis, text, n_text, ws, stream)

    def score_segments(self, seg, suf, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """Suffix b continues segment seg[b] of the segmented prefix."""
        B, C = suf["cands"].shape
        if out is None:
            out = torch.empty((B, C), dtype=torch.float32, device=self.device)
        ws = self.workspace(self.suffix_ws_bytes(suf))
        J.jev_score_segments(self.prefix, seg, suf["ids"], suf["lens"], suf["cands"], suf["n_cands"], out, ws,
                             stream)
        return out

    def suffix_ws_bytes(self, suf) -> int:
        B, C = suf["cands"].shape
        T = int(np.sum(suf["lens"]))
        return J.jev_workspace_bytes(self.model, self.P, T, B, B * C)

    def score_suffixes(self, suf, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        B, C = suf["cands"].shape
        if out is None:
            out = torch.empty((B, C), dtype=torch.float32, device=self.device)
        ws = self.workspace(self.suffix_ws_bytes(suf))
        J.jev_score_suffixes(self.prefix, suf["ids"], suf["lens"], suf["cands"], suf["n_cands"], out, ws, stream)
        return out

    def tree_ws_bytes(self, tree, mode) -> int:
        rows, seqs, targets = J.jev_tree_plan_size(tree["stem_ids"], tree["stem_lens"], tree["cand_tok"],
                                                   tree["cand_lens"], tree["n_cands"], mode)
        return J.jev_workspace_bytes(self.model, self.P, rows, max(seqs, tree["stem_lens"].shape[0]), targets)

    def score_tree(self, tree, mode=J.JEV_TREE_TRIE, stream=None):
        Q, C, _ = tree["cand_tok"].shape
        score = torch.empty((Q, C), dtype=torch.float32, device=self.device)
        norm = torch.empty((Q, C), dtype=torch.float32, device=self.device)
        ws = self.workspace(self.tree_ws_bytes(tree, mode))
        J.jev_score_tree(self.prefix, tree["stem_ids"], tree["stem_lens"], tree["cand_tok"], tree["cand_lens"],
                         tree["n_cands"], mode, score, norm, ws, stream)
        return score, norm

    # ------------------------------------------------------------------ graph capture
    def capture_score_suffixes(self, suf, stream: "torch.cuda.Stream") -> "CapturedCall":
        """Stage the request's metadata with one jev_score_suffixes call on `stream` into a
        workspace of its own, then capture jev_score_suffixes_launch into a HIP graph.  Each
        replay of the returned call rescores the suffixes into its `out`."""
        B, C = suf["cands"].shape
        out = torch.empty((B, C), dtype=torch.float32, device=self.device)
        ws = torch.empty(max(self.suffix_ws_bytes(suf), 256), dtype=torch.uint8, device=self.device)
        args = (self.prefix, suf["ids"], suf["lens"], suf["cands"], suf["n_cands"], out, ws)
        with torch.cuda.stream(stream):
            J.jev_score_suffixes(*args, stream=stream.cuda_stream)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            J.jev_score_suffixes_launch(*args, stream=stream.cuda_stream)
        return CapturedCall(g, ws, (out,))

    def capture_score_tree(self, tree, mode, stream: "torch.cuda.Stream") -> "CapturedCall":
        """As capture_score_suffixes for jev_score_tree; outputs (score, norm)."""
        Q, C, _ = tree["cand_tok"].shape
        score = torch.empty((Q, C), dtype=torch.float32, device=self.device)
        norm = torch.empty((Q, C), dtype=torch.float32, device=self.device)
        ws = torch.empty(max(self.tree_ws_bytes(tree, mode), 256), dtype=torch.uint8, device=self.device)
        args = (self.prefix, tree["stem_ids"], tree["stem_lens"], tree["cand_tok"], tree["cand_lens"],
                tree["n_cands"], mode, score, norm, ws)
        with torch.cuda.stream(stream):
            J.jev_score_tree(*args, stream=stream.cuda_stream)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            J.jev_score_tree_launch(*args, stream=stream.cuda_stream)
        return CapturedCall(g, ws, (score, norm))

    def set_skip(self, skip) -> None:
        """Blocks the candidate rows of scoring calls bypass (None clears); prefills keep every block."""
        J.jev_model_set_skip(self.model, skip)

    def stats(self) -> dict:
        return J.jev_get_stats(self.model)


class CapturedCall:
    """A captured scoring call: the graph, the workspace holding its staged metadata and its
    outputs, kept alive together.  replay() enqueues the graph on the current stream."""

    def __init__(self, graph, ws, outs):
        self.graph, self.ws, self.outs = graph, ws, outs

    def replay(self):
        self.graph.replay()
