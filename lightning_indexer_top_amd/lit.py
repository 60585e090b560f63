"""ctypes binding of liblit.so (the C ABI in include/lit.h).

Argument marshalling only: every step runs in the HIP kernels of liblit.so.  PyTorch
is used for device memory (outputs and workspace are torch tensors the caller may
pass in) and for the current HIP stream.  There is no fallback: if liblit.so is
missing or a call is refused, a ``LitError`` is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblit.so")

LIT_OK = 0
STATUS_NAMES = {0: "LIT_OK", 1: "LIT_E_NULL", 2: "LIT_E_SHAPE", 3: "LIT_E_ALIGN",
                4: "LIT_E_UNSUPPORTED", 5: "LIT_E_WORKSPACE", 6: "LIT_E_HIP"}

# Every function include/lit.h declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t
_F = ctypes.c_float


class lit_step_args(ctypes.Structure):
    _fields_ = [("B", _I), ("S", _I), ("start_pos", _I), ("ratio", _I),
                ("Hi", _I), ("Di", _I), ("index_topk", _I), ("T_cap", _I),
                ("q8", _P), ("q_sc", _P), ("w", _P), ("k8", _P), ("k_sc", _P),
                ("H", _I), ("D", _I), ("dv", _I), ("W", _I), ("R", _I),
                ("q", _P), ("win_kv", _P), ("comp_kv", _P), ("sink", _P), ("scale", _F),
                ("topk_idx", _P), ("out", _P), ("stage_events", _P * 4), ("state", _P), ("state_bytes", _Z),
                ("flags", _I), ("index_format", _I),
                ("cand_in", _P), ("cand_k", _I), ("cand_out", _P), ("cand_topk_blocks", _I),
                ("cand_block_size", _I), ("win_kv_format", _I), ("win_kv_scales", _P),
                ("comp_kv_format", _I), ("comp_kv_scales", _P), ("layers", _I)]


LIT_STEP_UNFUSED = 1
# lit_index_format: the code format of the index queries and keys
INDEX_FORMATS = {"e4m3": 0, "e2m1": 1}
# lit_kv_format: the attention KV sources (window: bf16 or e4m3; compressed: bf16 or e2m1)
KV_FORMATS = {"bf16": 0, "e4m3": 1, "e2m1": 2}


SIGNATURES = {
    "lit_status_str": (ctypes.c_char_p, [_I]),
    "lit_abi_version": (_I, []),
    "lit_topk_width": (_I, [_I, _I, _I, _I]),
    "lit_compress_writes_row": (_I, [_I, _I]),
    "lit_indexer_scores": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _I, _P]),
    "lit_indexer_scores_fmt": (_I, [_I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _I, _P]),
    "lit_topk": (_I, [_P, _I, _I, _I, _I, _I, _I, _P, _P, _Z, _P]),
    "lit_topk_workspace_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "lit_candidate_blocks": (_I, [_P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _Z, _P]),
    "lit_candidate_blocks_workspace_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "lit_candidate_blocks_width": (_I, [_I, _I, _I, _I, _I]),
    "lit_topk_candidates": (_I, [_P, _I, _I, _I, _I, _I, _I, _P, _I, _I, _P, _P, _Z, _P]),
    "lit_window_indices": (_I, [_I, _I, _I, _I, _I, _P, _P]),
    "lit_window_width": (_I, [_I, _I, _I]),
    "lit_sparse_attn": (_I, [_P, _I, _I, _I, _I, _I, _P, _I, _P, _I, _P, _I, _P, _I, _P, _F,
                             _P, _P, _Z, _P]),
    "lit_sparse_attn_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _I]),
    "lit_sparse_attn_fmt": (_I, [_P, _I, _I, _I, _I, _I, _I, _P, _P, _I, _P, _I, _I, _P, _P, _I, _P,
                                 _I, _P, _F, _P, _P, _Z, _P]),
    "lit_sparse_attn_layers": (_I, [_I, _P, _I, _I, _I, _I, _I, _P, _I, _P, _I, _I, _P, _I, _P, _I,
                                    _P, _F, _P, _P, _Z, _P]),
    "lit_sparse_attn_layers_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _I, _I]),
    "lit_compress_append": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _F, _P, _I, _I, _P, _P, _I, _P,
                                 _P]),
    "lit_window_append": (_I, [_I, _I, _I, _P, _P, _I, _I, _P, _P, _I, _P]),
    "lit_compress_chunk_rows": (_I, [_I, _I, _I]),
    "lit_compress_chunk": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _F, _P, _I, _I, _P, _P, _I, _P, _P]),
    "lit_window_chunk": (_I, [_I, _I, _I, _I, _P, _P, _I, _I, _P, _P, _I, _P]),
    "lit_sparse_step": (_I, [ctypes.POINTER(lit_step_args), _P, _Z, _P]),
    "lit_sparse_step_workspace_bytes": (_Z, [ctypes.POINTER(lit_step_args)]),
    "lit_sparse_step_state_bytes": (_Z, [ctypes.POINTER(lit_step_args)]),
    "lit_sparse_step_noalloc": (_I, [ctypes.POINTER(lit_step_args), _P, _P]),
}


class LitError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)}")


_lib = None


def library() -> ctypes.CDLL:
    """Load liblit.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(fn: str, status: int) -> None:
    if status != LIT_OK:
        raise LitError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t: torch.Tensor, dtype, name: str) -> None:
    if t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous {dtype} tensor, got {t.dtype}")


def topk_width(S: int, start_pos: int, ratio: int, index_topk: int) -> int:
    return library().lit_topk_width(S, start_pos, ratio, index_topk)


def lit_window_width(S: int, start_pos: int, W: int) -> int:
    return library().lit_window_width(S, start_pos, W)


def lit_indexer_scores(q8, q_sc, w, k8, k_sc, start_pos: int, ratio: int, scores=None,
                       stream=None, fmt: str = "e4m3") -> torch.Tensor:
    """Scores [B,S,ld] fp32 (ld = T rounded up to 4); columns >= T are untouched.

    ``fmt`` is the code format of q8 / k8: "e4m3" (lit_indexer_scores) or "e2m1"
    (lit_indexer_scores_fmt; rows of Di/2 bytes).  Di comes from the scale arrays."""
    for t, dt, n in ((q8, torch.uint8, "q8"), (q_sc, torch.uint8, "q_sc"), (w, torch.float32, "w"),
                     (k8, torch.uint8, "k8"), (k_sc, torch.uint8, "k_sc")):
        _need(t, dt, n)
    B, S, Hi, _ = q8.shape
    Di = 32 * q_sc.shape[-1]
    T_cap = k8.shape[1]
    T = (start_pos + S) // ratio
    if scores is None:
        scores = torch.empty((B, S, max(4, (T + 3) // 4 * 4)), dtype=torch.float32, device=q8.device)
    _need(scores, torch.float32, "scores")
    args = (_ptr(q8), _ptr(q_sc), _ptr(w), _ptr(k8), _ptr(k_sc), B, S, Hi, Di, T_cap, start_pos,
            ratio, _ptr(scores), scores.shape[-1], _stream(stream))
    if fmt == "e4m3":
        _check("lit_indexer_scores", library().lit_indexer_scores(*args))
    else:
        _check("lit_indexer_scores_fmt", library().lit_indexer_scores_fmt(INDEX_FORMATS[fmt], *args))
    return scores


def lit_topk(scores, start_pos: int, ratio: int, index_topk: int, idx=None, ws=None,
             stream=None) -> torch.Tensor:
    """Top-k row lists [B,S,k_eff] int32 (ascending, -1 padded)."""
    _need(scores, torch.float32, "scores")
    B, S, ld = scores.shape
    keff = topk_width(S, start_pos, ratio, index_topk)
    if idx is None:
        idx = torch.empty((B, S, keff), dtype=torch.int32, device=scores.device)
    _need(idx, torch.int32, "idx")
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("lit_topk", library().lit_topk(_ptr(scores), ld, B, S, start_pos, ratio, index_topk,
                                          _ptr(idx), _ptr(ws), nbytes, _stream(stream)))
    return idx


def lit_candidate_blocks(scores, start_pos: int, ratio: int, topk_blocks: int, block_size: int,
                         blocks=None, ws=None, stream=None) -> torch.Tensor:
    """Level one of the two-level top-k: kept block numbers [B,S,kb] int32 (ascending,
    -1 padded), kb = min(topk_blocks, ceil(T / block_size))."""
    _need(scores, torch.float32, "scores")
    B, S, ld = scores.shape
    kb = library().lit_candidate_blocks_width(S, start_pos, ratio, topk_blocks, block_size)
    if blocks is None:
        blocks = torch.empty((B, S, kb), dtype=torch.int32, device=scores.device)
    _need(blocks, torch.int32, "blocks")
    need = library().lit_candidate_blocks_workspace_bytes(B, S, start_pos, ratio, block_size)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=scores.device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("lit_candidate_blocks", library().lit_candidate_blocks(
        _ptr(scores), ld, B, S, start_pos, ratio, topk_blocks, block_size, _ptr(blocks), _ptr(ws),
        nbytes, _stream(stream)))
    return blocks


def lit_topk_candidates(scores, start_pos: int, ratio: int, index_topk: int, blocks,
                        block_size: int, idx=None, stream=None) -> torch.Tensor:
    """Level two: top-k [B,S,k_eff] over the scores with rows outside ``blocks`` at -inf."""
    _need(scores, torch.float32, "scores")
    _need(blocks, torch.int32, "blocks")
    B, S, ld = scores.shape
    keff = topk_width(S, start_pos, ratio, index_topk)
    if idx is None:
        idx = torch.empty((B, S, keff), dtype=torch.int32, device=scores.device)
    _need(idx, torch.int32, "idx")
    _check("lit_topk_candidates", library().lit_topk_candidates(
        _ptr(scores), ld, B, S, start_pos, ratio, index_topk, _ptr(blocks), blocks.shape[-1],
        block_size, _ptr(idx), None, 0, _stream(stream)))
    return idx


def lit_window_indices(B: int, S: int, start_pos: int, W: int, R: int, win_idx=None,
                       device="cuda", stream=None) -> torch.Tensor:
    width = lit_window_width(S, start_pos, W)
    if win_idx is None:
        win_idx = torch.empty((B, S, width), dtype=torch.int32, device=device)
    _need(win_idx, torch.int32, "win_idx")
    _check("lit_window_indices", library().lit_window_indices(B, S, start_pos, W, R, _ptr(win_idx),
                                                              _stream(stream)))
    return win_idx


def lit_sparse_attn_workspace_bytes(B, S, H, dv, W, K) -> int:
    return library().lit_sparse_attn_workspace_bytes(B, S, H, dv, W, K)


def lit_sparse_attn(q, win_kv, win_idx, comp_kv, comp_idx, sink, scale: float, dv=None,
                    out=None, ws=None, stream=None) -> torch.Tensor:
    """Attention [B,S,H,dv] bf16 over the window slots in win_idx and the compressed rows in
    comp_idx (either source may be None)."""
    _need(q, torch.bfloat16, "q")
    B, S, H, D = q.shape
    dv = D if dv is None else dv
    W = 0 if win_idx is None else win_idx.shape[-1]
    K = 0 if comp_idx is None else comp_idx.shape[-1]
    R = 0 if win_kv is None else win_kv.shape[1]
    T_cap = 0 if comp_kv is None else comp_kv.shape[1]
    for t, dt, n in ((win_kv, torch.bfloat16, "win_kv"), (comp_kv, torch.bfloat16, "comp_kv"),
                     (win_idx, torch.int32, "win_idx"), (comp_idx, torch.int32, "comp_idx"),
                     (sink, torch.float32, "sink")):
        if t is not None:
            _need(t, dt, n)
    if out is None:
        out = torch.empty((B, S, H, dv), dtype=torch.bfloat16, device=q.device)
    _need(out, torch.bfloat16, "out")
    need = lit_sparse_attn_workspace_bytes(B, S, H, dv, W, K)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("lit_sparse_attn", library().lit_sparse_attn(
        _ptr(q), B, S, H, D, dv, _ptr(win_kv), R, _ptr(win_idx), W, _ptr(comp_kv), T_cap,
        _ptr(comp_idx), K, _ptr(sink), float(scale), _ptr(out), _ptr(ws), nbytes, _stream(stream)))
    return out


def lit_sparse_attn_fmt(q, win_kv, win_idx, comp_kv, comp_idx, sink, scale: float, dv=None,
                        win_fmt: str = "bf16", win_sc=None, comp_fmt: str = "bf16", comp_sc=None,
                        out=None, ws=None, stream=None) -> torch.Tensor:
    """lit_sparse_attn with quantised sources: win_kv e4m3 codes uint8 [B,R,D] + win_sc
    [B,R,D/32], comp_kv e2m1 codes uint8 [B,T_cap,D/2] + comp_sc [B,T_cap,D/16] (or bf16)."""
    _need(q, torch.bfloat16, "q")
    B, S, H, D = q.shape
    dv = D if dv is None else dv
    W = 0 if win_idx is None else win_idx.shape[-1]
    K = 0 if comp_idx is None else comp_idx.shape[-1]
    R = 0 if win_kv is None else win_kv.shape[1]
    T_cap = 0 if comp_kv is None else comp_kv.shape[1]
    for t, fmt, n in ((win_kv, win_fmt, "win_kv"), (comp_kv, comp_fmt, "comp_kv")):
        if t is not None:
            _need(t, torch.bfloat16 if fmt == "bf16" else torch.uint8, n)
    for t, dt, n in ((win_sc, torch.uint8, "win_sc"), (comp_sc, torch.uint8, "comp_sc"),
                     (win_idx, torch.int32, "win_idx"), (comp_idx, torch.int32, "comp_idx"),
                     (sink, torch.float32, "sink")):
        if t is not None:
            _need(t, dt, n)
    if out is None:
        out = torch.empty((B, S, H, dv), dtype=torch.bfloat16, device=q.device)
    _need(out, torch.bfloat16, "out")
    need = lit_sparse_attn_workspace_bytes(B, S, H, dv, W, K)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("lit_sparse_attn_fmt", library().lit_sparse_attn_fmt(
        _ptr(q), B, S, H, D, dv, KV_FORMATS[win_fmt], _ptr(win_kv), _ptr(win_sc), R, _ptr(win_idx), W,
        KV_FORMATS[comp_fmt], _ptr(comp_kv), _ptr(comp_sc), T_cap, _ptr(comp_idx), K, _ptr(sink),
        float(scale), _ptr(out), _ptr(ws), nbytes, _stream(stream)))
    return out


def lit_sparse_attn_layers(q, win_kv, win_idx, comp_kv, comp_idx, sink, scale: float, dv=None,
                           out=None, ws=None, stream=None, window: int = 0,
                           start_pos: int = 0) -> torch.Tensor:
    """Attention [L,B,S,H,dv] bf16 for L layers sharing the row lists and comp_kv:
    q [L,B,S,H,D], win_kv [L,B,R,D] (or None), sink [L,H] (or None).  With win_idx None
    and ``window`` > 0 the window list is derived from ``start_pos`` in the kernel."""
    _need(q, torch.bfloat16, "q")
    L, B, S, H, D = q.shape
    dv = D if dv is None else dv
    W = window if win_idx is None else win_idx.shape[-1]
    K = 0 if comp_idx is None else comp_idx.shape[-1]
    R = 0 if win_kv is None else win_kv.shape[2]
    T_cap = 0 if comp_kv is None else comp_kv.shape[1]
    for t, dt, n in ((win_kv, torch.bfloat16, "win_kv"), (comp_kv, torch.bfloat16, "comp_kv"),
                     (win_idx, torch.int32, "win_idx"), (comp_idx, torch.int32, "comp_idx"),
                     (sink, torch.float32, "sink")):
        if t is not None:
            _need(t, dt, n)
    if out is None:
        out = torch.empty((L, B, S, H, dv), dtype=torch.bfloat16, device=q.device)
    _need(out, torch.bfloat16, "out")
    nwin = W if win_idx is not None else lit_window_width(S, start_pos, W)
    need = library().lit_sparse_attn_layers_workspace_bytes(L, B, S, H, dv, nwin, K)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("lit_sparse_attn_layers", library().lit_sparse_attn_layers(
        L, _ptr(q), B, S, H, D, dv, _ptr(win_kv), R, _ptr(win_idx), W, start_pos, _ptr(comp_kv), T_cap,
        _ptr(comp_idx), K, _ptr(sink), float(scale), _ptr(out), _ptr(ws), nbytes, _stream(stream)))
    return out


def lit_compress_append(kv, score, kv_state, score_state, norm_w, eps: float, freqs, rd: int,
                        codes, scales, start_pos: int, ratio: int, latent=None, stream=None) -> bool:
    """One decode token per sequence into the compressor (state and cache updated in
    place); returns whether the group completed and a cache row was written."""
    _need(kv, torch.float32, "kv")
    B, D = kv.shape
    for t, dt, n in ((score, torch.float32, "score"), (norm_w, torch.float32, "norm_w"),
                     (freqs, torch.float32, "freqs"), (codes, torch.uint8, "codes"),
                     (scales, torch.uint8, "scales")):
        _need(t, dt, n)
    for t, n in ((kv_state, "kv_state"), (score_state, "score_state")):
        if t is not None:
            _need(t, torch.float32, n)
    if latent is not None:
        _need(latent, torch.bfloat16, "latent")
    _check("lit_compress_append", library().lit_compress_append(
        B, D, ratio, start_pos, _ptr(kv), _ptr(score), _ptr(kv_state), _ptr(score_state),
        _ptr(norm_w), float(eps), _ptr(freqs), freqs.shape[0], rd, _ptr(codes), _ptr(scales),
        codes.shape[1], _ptr(latent), _stream(stream)))
    return bool(library().lit_compress_writes_row(start_pos, ratio))


def lit_window_append(kv, freqs, rd: int, codes, scales, start_pos: int, stream=None) -> None:
    """One decode token per sequence into the window ring (codes [B,R,D] e4m3, scales)."""
    _need(kv, torch.bfloat16, "kv")
    B, D = kv.shape
    for t, dt, n in ((freqs, torch.float32, "freqs"), (codes, torch.uint8, "codes"),
                     (scales, torch.uint8, "scales")):
        _need(t, dt, n)
    _check("lit_window_append", library().lit_window_append(
        B, D, start_pos, _ptr(kv), _ptr(freqs), freqs.shape[0], rd, _ptr(codes), _ptr(scales),
        codes.shape[1], _stream(stream)))


def lit_compress_chunk(kv, score, kv_state, score_state, norm_w, eps: float, freqs, rd: int,
                       codes, scales, start_pos: int, ratio: int, latent=None, stream=None) -> int:
    """A chunk of S tokens per sequence (kv, score [B, S, D]) into the compressor; returns
    the number of compressed rows written (latent, if given: [B, rows, D] bf16)."""
    _need(kv, torch.float32, "kv")
    B, S, D = kv.shape
    for t, dt, n in ((score, torch.float32, "score"), (norm_w, torch.float32, "norm_w"),
                     (freqs, torch.float32, "freqs"), (codes, torch.uint8, "codes"),
                     (scales, torch.uint8, "scales")):
        _need(t, dt, n)
    for t, n in ((kv_state, "kv_state"), (score_state, "score_state")):
        if t is not None:
            _need(t, torch.float32, n)
    if latent is not None:
        _need(latent, torch.bfloat16, "latent")
    _check("lit_compress_chunk", library().lit_compress_chunk(
        B, S, D, ratio, start_pos, _ptr(kv), _ptr(score), _ptr(kv_state), _ptr(score_state),
        _ptr(norm_w), float(eps), _ptr(freqs), freqs.shape[0], rd, _ptr(codes), _ptr(scales),
        codes.shape[1], _ptr(latent), _stream(stream)))
    return int(library().lit_compress_chunk_rows(start_pos, S, ratio))


def lit_window_chunk(kv, freqs, rd: int, codes, scales, start_pos: int, stream=None) -> None:
    """A chunk of S window rows per sequence (kv [B, S, D] bf16) into the ring."""
    _need(kv, torch.bfloat16, "kv")
    B, S, D = kv.shape
    for t, dt, n in ((freqs, torch.float32, "freqs"), (codes, torch.uint8, "codes"),
                     (scales, torch.uint8, "scales")):
        _need(t, dt, n)
    _check("lit_window_chunk", library().lit_window_chunk(
        B, S, D, start_pos, _ptr(kv), _ptr(freqs), freqs.shape[0], rd, _ptr(codes), _ptr(scales),
        codes.shape[1], _stream(stream)))


def make_step_args(*, q8, q_sc, w, k8, k_sc, q, win_kv, comp_kv, start_pos: int, ratio: int,
                   index_topk: int, W: int, scale: float, dv=None, sink=None, topk_idx=None,
                   out=None, stage_events=None, flags: int = 0, fmt: str = "e4m3",
                   cand_in=None, cand_out=None, cand_topk_blocks: int = 0,
                   cand_block_size: int = 0, win_fmt: str = "bf16", win_sc=None,
                   comp_fmt: str = "bf16", comp_sc=None) -> tuple:
    """Build the lit_step_args struct (and allocate outputs the caller did not pass).
    ``fmt`` is the index-code format ("e4m3" or "e2m1"); Di comes from q_sc.  For the
    two-level top-k, ``cand_in`` [B,S,cand_k] int32 makes this a level-two layer and
    ``cand_out`` [B,S,kb] int32 the candidate source (blocks of ``cand_block_size``).
    Quantised attention KV: ``win_fmt="e4m3"`` (win_kv uint8 codes, win_sc scales) and
    ``comp_fmt="e2m1"`` (comp_kv uint8 codes, comp_sc scales).  Layers sharing the top-k:
    a 5-D ``q`` [L,B,S,H,D] with win_kv [L,B,R,*] (and sink [L,H]) makes L layers attend
    over the one list; ``out`` is then [L,B,S,H,dv]."""
    B, S, Hi, _ = q8.shape
    Di = 32 * q_sc.shape[-1]
    layers = q.shape[0] if q.dim() == 5 else 1
    H, D = q.shape[-2], q.shape[-1]
    R = win_kv.shape[-2]
    dv = D if dv is None else dv
    keff = topk_width(S, start_pos, ratio, index_topk)
    if topk_idx is None:
        topk_idx = torch.empty((B, S, keff), dtype=torch.int32, device=q.device)
    if out is None:
        shape = (layers, B, S, H, dv) if layers > 1 else (B, S, H, dv)
        out = torch.empty(shape, dtype=torch.bfloat16, device=q.device)
    a = lit_step_args(B=B, S=S, start_pos=start_pos, ratio=ratio, Hi=Hi, Di=Di,
                      index_topk=index_topk, T_cap=k8.shape[1], q8=q8.data_ptr(),
                      q_sc=q_sc.data_ptr(), w=w.data_ptr(), k8=k8.data_ptr(), k_sc=k_sc.data_ptr(),
                      H=H, D=D, dv=dv, W=W, R=R, q=q.data_ptr(),
                      win_kv=win_kv.data_ptr(), comp_kv=comp_kv.data_ptr(),
                      sink=0 if sink is None else sink.data_ptr(), scale=scale,
                      topk_idx=topk_idx.data_ptr(), out=out.data_ptr(), flags=flags,
                      index_format=INDEX_FORMATS[fmt],
                      cand_in=0 if cand_in is None else cand_in.data_ptr(),
                      cand_k=0 if cand_in is None else cand_in.shape[-1],
                      cand_out=0 if cand_out is None else cand_out.data_ptr(),
                      cand_topk_blocks=cand_topk_blocks, cand_block_size=cand_block_size,
                      win_kv_format=KV_FORMATS[win_fmt],
                      win_kv_scales=0 if win_sc is None else win_sc.data_ptr(),
                      comp_kv_format=KV_FORMATS[comp_fmt],
                      comp_kv_scales=0 if comp_sc is None else comp_sc.data_ptr(),
                      layers=layers)
    for t, n in ((cand_in, "cand_in"), (cand_out, "cand_out")):
        if t is not None:
            _need(t, torch.int32, n)
    if stage_events is not None:
        # hipEvent_t handles (e.g. torch.cuda.Event(...).cuda_event after one record)
        for k, ev in enumerate(stage_events):
            a.stage_events[k] = ev or None
    # the struct holds raw addresses: keep the tensors behind them alive with it, or a
    # caller passing temporaries would have their memory reused by the next allocation
    a._keep = (q8, q_sc, w, k8, k_sc, q, win_kv, comp_kv, sink, topk_idx, out, cand_in, cand_out,
               win_sc, comp_sc)
    return a, topk_idx, out


def lit_sparse_step_workspace_bytes(args: lit_step_args) -> int:
    return library().lit_sparse_step_workspace_bytes(ctypes.byref(args))


def step_workspace(args: lit_step_args, device="cuda") -> torch.Tensor:
    """Scratch workspace of the size the step needs."""
    return torch.empty(max(256, lit_sparse_step_workspace_bytes(args)), dtype=torch.uint8,
                       device=device)


def lit_sparse_step_state_bytes(args: lit_step_args) -> int:
    return library().lit_sparse_step_state_bytes(ctypes.byref(args))


def attach_state(args: lit_step_args, state: Optional[torch.Tensor] = None, device="cuda"):
    """Give the step a zero-filled fused-form state (allocated when not passed); returns
    it, or None when the fused form does not apply to these sizes."""
    need = lit_sparse_step_state_bytes(args)
    if need == 0:
        args.state, args.state_bytes = None, 0
        return None
    if state is None:
        state = torch.zeros(need, dtype=torch.uint8, device=device)
    args.state = state.data_ptr()
    args.state_bytes = state.numel() * state.element_size()
    args._state = state  # kept alive with the struct that points at it
    return state


def state_error(state: Optional[torch.Tensor]) -> int:
    """The sticky error word of a fused-form state (0 = no team timed out)."""
    return 0 if state is None else int(state[:4].view(torch.int32).item())


def lit_sparse_step(args: lit_step_args, ws: torch.Tensor, stream=None) -> None:
    """Run indexer -> top-k -> attention for one layer on the stream."""
    nbytes = ws.numel() * ws.element_size()
    _check("lit_sparse_step", library().lit_sparse_step(ctypes.byref(args), _ptr(ws), nbytes,
                                                        _stream(stream)))


def lit_sparse_step_noalloc(args: lit_step_args, err: Optional[torch.Tensor] = None, stream=None) -> None:
    """The step on the library's own scratch (no workspace or state from the caller);
    err: an optional zero-filled int32 device word that receives a team timeout."""
    if err is not None:
        _need(err, torch.int32, "err")
    _check("lit_sparse_step_noalloc", library().lit_sparse_step_noalloc(ctypes.byref(args), _ptr(err),
                                                                         _stream(stream)))
