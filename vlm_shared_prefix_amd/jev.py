"""Thin ctypes binding of libjev.so (argument marshalling only).

Every function here has the name of the C entry point it wraps and forwards
plain pointers and sizes to it.  Device buffers are torch tensors (PyTorch is
used for device memory and streams only); host arrays are NumPy int32.  All
compute runs in the library's HIP kernels.  If the library is missing this
module raises on import: there is no other path.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np
# torch brings its own HIP runtime (libamdhip64.so.7 in torch/lib).  Loading it before
# libjev.so lets the library's libamdhip64.so.7 dependency resolve to that same, already
# loaded runtime; loaded the other way round a process holds two HIP runtimes, and the
# library's runtime does not know the device buffers torch's runtime allocated.
import torch  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
# JEV_LIBRARY names another build of the same library (the host-sanitized one of the CPU tests)
LIB_PATH = os.environ.get("JEV_LIBRARY") or os.path.join(HERE, "libjev.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing; build it with `python -m vlm_shared_prefix_amd.build`")
_lib = C.CDLL(LIB_PATH)

JEV_OK, JEV_E_INVALID, JEV_E_UNSUPPORTED, JEV_E_WORKSPACE, JEV_E_HIP = 0, -1, -2, -3, -4
JEV_F32, JEV_BF16 = 0, 1
JEV_TREE_TRIE, JEV_TREE_STEM_ONLY, JEV_TREE_FLAT = 0, 1, 2
_STATUS = {0: "JEV_OK", -1: "JEV_E_INVALID", -2: "JEV_E_UNSUPPORTED", -3: "JEV_E_WORKSPACE", -4: "JEV_E_HIP"}


class jev_config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("mlp", C.c_int32),
                ("vocab", C.c_int32), ("rope_theta", C.c_float), ("rms_eps", C.c_float),
                ("dtype", C.c_int32)]


class jev_layer(C.Structure):
    _fields_ = [(k, C.c_void_p) for k in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm",
                                          "w_gate", "w_up", "w_down")]


class jev_weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("final_norm", C.c_void_p), ("lm_head", C.c_void_p),
                ("layers", C.POINTER(jev_layer))]


class jev_stats(C.Structure):
    _fields_ = [("prefills", C.c_uint64), ("forwards", C.c_uint64), ("rows", C.c_uint64),
                ("launches", C.c_uint64)]


class jev_kernel_stat(C.Structure):
    _fields_ = [("name", C.c_char * 32), ("launches", C.c_uint64), ("ms", C.c_double),
                ("flops", C.c_double), ("bytes", C.c_double)]


_i32p = C.POINTER(C.c_int32)
_u64p = C.POINTER(C.c_uint64)
_vp = C.c_void_p

JEV_F16_GATE_UP = 1   # w_gate, w_up
JEV_F16_QKV = 2       # wq, wk, wv
JEV_F16_DOWN = 4      # w_down
JEV_F16_O = 8         # wo
JEV_F16_GATE_UP_PREFILL = 16   # w_gate, w_up; the f16 pass in prefills only
JEV_F16_QKV_PREFILL = 32       # wq, wk, wv; prefills only
JEV_F16_O_PREFILL = 64         # wo; prefills only
JEV_F16_GATE_UP_SCORE = 128    # w_gate, w_up; prefills and suffix-scoring calls (not trees)

_sig = {
    "jev_model_create": (C.c_int32, [C.POINTER(jev_config), C.POINTER(jev_weights), C.POINTER(_vp)]),
    "jev_model_destroy": (None, [_vp]),
    "jev_get_stats": (C.c_int32, [_vp, C.POINTER(jev_stats)]),
    "jev_model_f16_bytes": (C.c_size_t, [_vp, C.c_int32]),
    "jev_model_attach_f16": (C.c_int32, [_vp, C.c_int32, _vp, C.c_size_t, _vp]),
    "jev_model_f16_groups": (C.c_int32, [_vp]),
    "jev_model_set_skip": (C.c_int32, [_vp, C.POINTER(C.c_uint8), C.c_int32]),
    "jev_model_set_attn_q_terms": (C.c_int32, [_vp, C.c_int32]),
    "jev_workspace_flags": (C.c_int32, [_vp, _i32p, _vp]),
    "jev_prefix_bytes": (C.c_size_t, [_vp, C.c_int32]),
    "jev_prefix_create": (C.c_int32, [_vp, C.c_int32, _vp, C.c_size_t, C.POINTER(_vp)]),
    "jev_prefix_destroy": (None, [_vp]),
    "jev_prefix_create_segments": (C.c_int32, [_vp, _i32p, C.c_int32, _vp, C.c_size_t, C.POINTER(_vp)]),
    "jev_prefill_segments": (C.c_int32, [_vp, _vp, _i32p, _i32p, _i32p, _vp, C.c_size_t, _vp]),
    "jev_score_segments": (C.c_int32, [_vp, _i32p, _i32p, _i32p, C.c_int32, C.c_int32, _i32p, _i32p, C.c_int32,
                                       _vp, _vp, C.c_size_t, _vp]),
    "jev_workspace_bytes": (C.c_size_t, [_vp, C.c_int32, C.c_int32, C.c_int32, C.c_int32]),
    "jev_prefill_prefix": (C.c_int32, [_vp, _vp, C.c_int32, _i32p, C.c_int32, _vp, C.c_size_t, _vp]),
    "jev_score_suffixes": (C.c_int32, [_vp, _i32p, _i32p, C.c_int32, C.c_int32, _i32p, _i32p, C.c_int32,
                                       _vp, _vp, C.c_size_t, _vp]),
    "jev_score_tree": (C.c_int32, [_vp, _i32p, _i32p, C.c_int32, C.c_int32, _i32p, _i32p, _i32p, C.c_int32,
                                   C.c_int32, C.c_int32, _vp, _vp, _vp, C.c_size_t, _vp]),
    "jev_static_scratch_bytes": (C.c_size_t, []),
    "jev_score_suffixes_noalloc": (C.c_int32, [_vp, _i32p, _i32p, C.c_int32, C.c_int32, _i32p, _i32p, C.c_int32,
                                               _vp, _vp]),
    "jev_score_suffixes_launch": (C.c_int32, [_vp, _i32p, _i32p, C.c_int32, C.c_int32, _i32p, _i32p, C.c_int32,
                                              _vp, _vp, C.c_size_t, _vp]),
    "jev_score_tree_launch": (C.c_int32, [_vp, _i32p, _i32p, C.c_int32, C.c_int32, _i32p, _i32p, _i32p,
                                          C.c_int32, C.c_int32, C.c_int32, _vp, _vp, _vp, C.c_size_t, _vp]),
    "jev_tree_plan_size": (C.c_int32, [_i32p, _i32p, C.c_int32, C.c_int32, _i32p, _i32p, _i32p, C.c_int32,
                                       C.c_int32, C.c_int32, _i32p, _i32p, _i32p]),
    "jev_tree_plan_rows": (C.c_int32, [_i32p, _i32p, C.c_int32, C.c_int32, _i32p, _i32p, _i32p, C.c_int32,
                                       C.c_int32, C.c_int32, _i32p, _i32p, _i32p, _u64p, _i32p]),
    "jev_segment_plan_tiles": (C.c_int32, [_i32p, C.c_int32, C.c_int32, _i32p, _i32p]),
    "jev_attn_schedule": (C.c_int32, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, _i32p,
                                      _i32p, _i32p, _i32p, C.c_int32, _i32p]),
    "jev_profile_start": (C.c_int32, [_vp]),
    "jev_profile_stop": (C.c_int32, [_vp, C.POINTER(jev_kernel_stat), C.c_int32, _i32p]),
    "jev_last_error": (C.c_char_p, []),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_sig)


class JevError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = _lib.jev_last_error().decode()
        super().__init__(f"{where}: {_STATUS.get(code, code)}: {msg}")


def _check(code: int, where: str) -> None:
    if code != JEV_OK:
        raise JevError(code, where)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr_i32(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_i32p)


def _dptr(t) -> Optional[int]:
    """Device pointer of a torch tensor (or None)."""
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return int(stream)


def jev_last_error() -> str:
    return _lib.jev_last_error().decode()


# ---------------------------------------------------------------------------- model / prefix
def jev_model_create(cfg: jev_config, weights: jev_weights) -> int:
    h = _vp()
    _check(_lib.jev_model_create(C.byref(cfg), C.byref(weights), C.byref(h)), "jev_model_create")
    return h.value


def jev_model_destroy(model: int) -> None:
    _lib.jev_model_destroy(model)


def jev_get_stats(model: int) -> dict:
    st = jev_stats()
    _check(_lib.jev_get_stats(model, C.byref(st)), "jev_get_stats")
    return {k: int(getattr(st, k)) for k, _ in jev_stats._fields_}


def jev_model_f16_bytes(model: int, groups: int) -> int:
    return int(_lib.jev_model_f16_bytes(model, groups))


def jev_model_attach_f16(model: int, groups: int, buf, stream=None) -> None:
    """Convert the decoder matrices of `groups` (an OR of JEV_F16_GATE_UP, JEV_F16_QKV, JEV_F16_DOWN, JEV_F16_O) into `buf` (a device
    tensor of >= jev_model_f16_bytes bytes; None detaches) and run those GEMMs as single float16
    passes."""
    nbytes = 0 if buf is None else buf.numel() * buf.element_size()
    _check(_lib.jev_model_attach_f16(model, groups, _dptr(buf), nbytes, _stream(stream)), "jev_model_attach_f16")


def jev_model_f16_groups(model: int) -> int:
    """Mirror groups whose float16 pass is in effect."""
    return int(_lib.jev_model_f16_groups(model))


def jev_model_set_skip(model: int, skip) -> None:
    """Blocks the candidate rows of scoring calls bypass (host array of n_layers flags; None clears)."""
    if skip is None:
        _check(_lib.jev_model_set_skip(model, None, 0), "jev_model_set_skip")
        return
    arr = np.ascontiguousarray(np.asarray(skip, dtype=np.uint8))
    _check(_lib.jev_model_set_skip(model, arr.ctypes.data_as(C.POINTER(C.c_uint8)), int(arr.size)),
           "jev_model_set_skip")


def jev_model_set_attn_q_terms(model: int, terms: int) -> None:
    """Float16 terms of q in the attention (0: by prefix length, 1 or 2)."""
    _check(_lib.jev_model_set_attn_q_terms(model, terms), "jev_model_set_attn_q_terms")


JEV_FLAG_F16_RANGE = 1


def jev_workspace_flags(ws, stream=None) -> int:
    """Range flag word of the last call that used the workspace (synchronises the stream)."""
    v = C.c_int32(0)
    _check(_lib.jev_workspace_flags(_dptr(ws), C.byref(v), _stream(stream)), "jev_workspace_flags")
    return int(v.value)


def jev_prefix_bytes(model: int, prefix_len: int) -> int:
    return int(_lib.jev_prefix_bytes(model, prefix_len))


def jev_prefix_create(model: int, prefix_len: int, kv_buf) -> int:
    h = _vp()
    _check(_lib.jev_prefix_create(model, prefix_len, _dptr(kv_buf), kv_buf.numel() * kv_buf.element_size()
                                  if kv_buf is not None else 0, C.byref(h)), "jev_prefix_create")
    return h.value


def jev_prefix_destroy(prefix: int) -> None:
    _lib.jev_prefix_destroy(prefix)


def jev_workspace_bytes(model: int, prefix_len: int, max_rows: int, max_seqs: int, max_targets: int) -> int:
    return int(_lib.jev_workspace_bytes(model, prefix_len, max_rows, max_seqs, max_targets))


def jev_profile_start(model: int) -> None:
    _check(_lib.jev_profile_start(model), "jev_profile_start")


def jev_profile_stop(model: int) -> dict:
    """Per-kernel totals {name: {launches, ms, flops, bytes}} since jev_profile_start."""
    arr = (jev_kernel_stat * 32)()
    n = C.c_int32()
    _check(_lib.jev_profile_stop(model, arr, 32, C.byref(n)), "jev_profile_stop")
    out = {}
    for i in range(min(n.value, 32)):
        k = arr[i]
        out[k.name.decode()] = {"launches": int(k.launches), "ms": k.ms, "flops": k.flops, "bytes": k.bytes}
    return out


# ---------------------------------------------------------------------------- hot path
def jev_prefill_prefix(prefix: int, vis_embeds, n_vis: int, text_ids, ws, stream=None) -> None:
    ids = _i32(text_ids)
    _check(_lib.jev_prefill_prefix(prefix, _dptr(vis_embeds), n_vis, _ptr_i32(ids), len(ids),
                                   _dptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "jev_prefill_prefix")


def _score_suffixes(fn, name, prefix, ids, lens, cand_ids, n_cands, out_logp, ws, stream):
    ids, lens, cand_ids, n_cands = _i32(ids), _i32(lens), _i32(cand_ids), _i32(n_cands)
    B = int(lens.shape[0])
    S_max = int(ids.shape[1]) if ids.ndim == 2 else 1
    C_max = int(cand_ids.shape[1]) if cand_ids.ndim == 2 else 1
    _check(fn(prefix, _ptr_i32(ids), _ptr_i32(lens), B, S_max, _ptr_i32(cand_ids), _ptr_i32(n_cands), C_max,
              _dptr(out_logp), _dptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
              _stream(stream)), name)


def jev_score_suffixes(prefix: int, ids, lens, cand_ids, n_cands, out_logp, ws, stream=None) -> None:
    _score_suffixes(_lib.jev_score_suffixes, "jev_score_suffixes", prefix, ids, lens, cand_ids, n_cands,
                    out_logp, ws, stream)


def jev_score_suffixes_launch(prefix: int, ids, lens, cand_ids, n_cands, out_logp, ws, stream=None) -> None:
    """Kernel launches of jev_score_suffixes only (the workspace must hold the metadata a
    jev_score_suffixes call with the same arguments staged); capturable into a HIP graph."""
    _score_suffixes(_lib.jev_score_suffixes_launch, "jev_score_suffixes_launch", prefix, ids, lens, cand_ids,
                    n_cands, out_logp, ws, stream)


def jev_static_scratch_bytes() -> int:
    return int(_lib.jev_static_scratch_bytes())


def jev_score_suffixes_noalloc(prefix: int, ids, lens, cand_ids, n_cands, out_logp, stream=None) -> None:
    """jev_score_suffixes on the library's static device scratch (no workspace, no allocation)."""
    ids, lens, cand_ids, n_cands = _i32(ids), _i32(lens), _i32(cand_ids), _i32(n_cands)
    B = int(lens.shape[0])
    S_max = int(ids.shape[1]) if ids.ndim == 2 else 1
    C_max = int(cand_ids.shape[1]) if cand_ids.ndim == 2 else 1
    _check(_lib.jev_score_suffixes_noalloc(prefix, _ptr_i32(ids), _ptr_i32(lens), B, S_max, _ptr_i32(cand_ids),
                                           _ptr_i32(n_cands), C_max, _dptr(out_logp), _stream(stream)),
           "jev_score_suffixes_noalloc")


def jev_prefix_create_segments(model: int, seg_lens, kv_buf) -> int:
    sl = _i32(seg_lens)
    out = _vp()
    _check(_lib.jev_prefix_create_segments(model, _ptr_i32(sl), len(sl), _dptr(kv_buf),
                                           kv_buf.numel() * kv_buf.element_size() if kv_buf is not None else 0,
                                           C.byref(out)), "jev_prefix_create_segments")
    return out.value


def jev_prefill_segments(prefix: int, vis_embeds, n_vis, text_ids, n_text, ws, stream=None) -> None:
    nv, ti, nt = _i32(n_vis), _i32(text_ids), _i32(n_text)
    _check(_lib.jev_prefill_segments(prefix, _dptr(vis_embeds), _ptr_i32(nv), _ptr_i32(ti), _ptr_i32(nt),
                                     _dptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "jev_prefill_segments")


def jev_score_segments(prefix: int, seg, ids, lens, cand_ids, n_cands, out_logp, ws, stream=None) -> None:
    sg = _i32(seg)
    _score_suffixes(lambda p, *a: _lib.jev_score_segments(p, _ptr_i32(sg), *a), "jev_score_segments", prefix,
                    ids, lens, cand_ids, n_cands, out_logp, ws, stream)


def _tree_args(stem_ids, stem_lens, cand_tok, cand_lens, n_cands):
    stem_ids, stem_lens = _i32(stem_ids), _i32(stem_lens)
    cand_tok, cand_lens, n_cands = _i32(cand_tok), _i32(cand_lens), _i32(n_cands)
    Q = int(stem_lens.shape[0])
    S_max = int(stem_ids.shape[1])
    C_max, K_max = int(cand_tok.shape[1]), int(cand_tok.shape[2])
    return stem_ids, stem_lens, cand_tok, cand_lens, n_cands, Q, S_max, C_max, K_max


def _score_tree(fn, name, prefix, stem_ids, stem_lens, cand_tok, cand_lens, n_cands, mode, out_score, out_norm,
                ws, stream):
    si, sl, ct, cl, nc, Q, S_max, C_max, K_max = _tree_args(stem_ids, stem_lens, cand_tok, cand_lens, n_cands)
    _check(fn(prefix, _ptr_i32(si), _ptr_i32(sl), Q, S_max, _ptr_i32(ct), _ptr_i32(cl), _ptr_i32(nc), C_max,
              K_max, mode, _dptr(out_score), _dptr(out_norm), _dptr(ws),
              ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)), name)


def jev_score_tree(prefix: int, stem_ids, stem_lens, cand_tok, cand_lens, n_cands, mode: int,
                   out_score, out_norm, ws, stream=None) -> None:
    _score_tree(_lib.jev_score_tree, "jev_score_tree", prefix, stem_ids, stem_lens, cand_tok, cand_lens, n_cands,
                mode, out_score, out_norm, ws, stream)


def jev_score_tree_launch(prefix: int, stem_ids, stem_lens, cand_tok, cand_lens, n_cands, mode: int,
                          out_score, out_norm, ws, stream=None) -> None:
    """Kernel launches of jev_score_tree only (see jev_score_suffixes_launch)."""
    _score_tree(_lib.jev_score_tree_launch, "jev_score_tree_launch", prefix, stem_ids, stem_lens, cand_tok,
                cand_lens, n_cands, mode, out_score, out_norm, ws, stream)


def jev_segment_plan_tiles(pseg, G: int):
    """(ptile [blocks][4], max tiles) of the attention's segment table for rows' prefix key
    ranges pseg [T][2] and G query heads per KV head (host only)."""
    ps = np.ascontiguousarray(np.asarray(pseg, dtype=np.int32).reshape(-1, 2))
    T = int(ps.shape[0])
    nb = (G * T + 127) // 128
    out = np.zeros((max(nb, 1), 4), np.int32)
    mx = C.c_int32()
    _check(_lib.jev_segment_plan_tiles(_ptr_i32(ps), T, G, _ptr_i32(out), C.byref(mx)), "jev_segment_plan_tiles")
    return out[:nb], mx.value


def jev_attn_schedule(T: int, G: int, Hkv: int, P: int, own_tiles: int, segmented: bool = False,
                      max_spans: int = 0):
    """(n_split, chunk, blocks, spans [n][7]) of the attention's work split (host only); spans
    (block, item, slot, first tile, end tile, last, item slot count) under the balanced schedule
    when max_spans > 0."""
    ns, ch, nb, n = C.c_int32(), C.c_int32(), C.c_int32(), C.c_int32()
    sp = np.zeros((max(max_spans, 1), 7), np.int32)
    _check(_lib.jev_attn_schedule(T, G, Hkv, P, own_tiles, int(bool(segmented)), C.byref(ns), C.byref(ch),
                                  C.byref(nb), _ptr_i32(sp) if max_spans > 0 else None, max_spans, C.byref(n)),
           "jev_attn_schedule")
    return ns.value, ch.value, nb.value, sp[:n.value]


def jev_tree_plan_size(stem_ids, stem_lens, cand_tok, cand_lens, n_cands, mode: int):
    si, sl, ct, cl, nc, Q, S_max, C_max, K_max = _tree_args(stem_ids, stem_lens, cand_tok, cand_lens, n_cands)
    r, s, t = C.c_int32(), C.c_int32(), C.c_int32()
    _check(_lib.jev_tree_plan_size(_ptr_i32(si), _ptr_i32(sl), Q, S_max, _ptr_i32(ct), _ptr_i32(cl),
                                   _ptr_i32(nc), C_max, K_max, mode, C.byref(r), C.byref(s), C.byref(t)),
           "jev_tree_plan_size")
    return r.value, s.value, t.value


def jev_tree_plan_rows(stem_ids, stem_lens, cand_tok, cand_lens, n_cands, mode: int) -> dict:
    rows, _, targets = jev_tree_plan_size(stem_ids, stem_lens, cand_tok, cand_lens, n_cands, mode)
    si, sl, ct, cl, nc, Q, S_max, C_max, K_max = _tree_args(stem_ids, stem_lens, cand_tok, cand_lens, n_cands)
    tok = np.zeros(rows, np.int32)
    depth = np.zeros(rows, np.int32)
    group = np.zeros(rows, np.int32)
    mask = np.zeros(rows, np.uint64)
    trow = np.zeros(targets, np.int32)
    _check(_lib.jev_tree_plan_rows(_ptr_i32(si), _ptr_i32(sl), Q, S_max, _ptr_i32(ct), _ptr_i32(cl),
                                   _ptr_i32(nc), C_max, K_max, mode, _ptr_i32(tok), _ptr_i32(depth),
                                   _ptr_i32(group), mask.ctypes.data_as(_u64p), _ptr_i32(trow)),
           "jev_tree_plan_rows")
    return {"tok": tok, "depth": depth, "group": group, "mask": mask,
            "target_row": trow.reshape(Q, C_max, K_max)}


def make_config(n_layers, hidden, n_q_heads, n_kv_heads, head_dim, mlp, vocab, rope_theta, rms_eps,
                dtype) -> jev_config:
    return jev_config(n_layers, hidden, n_q_heads, n_kv_heads, head_dim, mlp, vocab, float(rope_theta),
                      float(rms_eps), int(dtype))


def make_weights(embed, final_norm, lm_head, layers: Sequence[dict]):
    """Build jev_weights from device tensors; returns (weights, keepalive)."""
    arr = (jev_layer * max(len(layers), 1))()
    for i, L in enumerate(layers):
        arr[i] = jev_layer(*[_dptr(L[k]) for k in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm",
                                                   "w_gate", "w_up", "w_down")])
    w = jev_weights(_dptr(embed), _dptr(final_norm), _dptr(lm_head), arr)
    return w, arr
