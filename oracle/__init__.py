"""Plain fp64 CPU oracle for the sparse-attention step (indexer -> top-k -> attention).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU-baseline leg
are the only callers.  The product path (``lightning_indexer_top_amd``) never imports
this package, and this package never imports the product path: the two share nothing
but the seeded input generator.

The arithmetic lives in ``lit_oracle.c`` (plain C, double precision, OpenMP over
queries); this module only marshals numpy arrays into it and composes the steps.
Sources are cited per function there:

* DeepSeek-V4.1-Flash-NVFP4 ``inference/model.py``: module globals (e4m3 with one
  ue8m0 scale per 32 values; fp4 e2m1 with the same scales for the indexer),
  ``get_window_topk_idxs``, ``Indexer.forward``,
  ``Attention.forward``.
* DeepSeek-V3.2-Exp ``inference/model.py``: ``Indexer.forward`` (``fp8_index``) and
  ``MLA.forward`` (dense scores, index mask, softmax).

Parity status: every function here is pinned by ``tests/test_oracle_*.py`` (closed
forms, library routines on special cases, invariants, derived integer cases); the
composed step has no end-to-end expected values on the pages and is pinned only
through its parts.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lit_oracle.c")
_LIB = os.path.join(_HERE, "liblit_oracle.so")

ORC_E_ARG = -1
ORC_E_CODE = -2
ORC_E_INDEX = -3


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, no FMA contraction, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _bind(path: str):
    """Open a compiled oracle library and declare its signatures."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.orc_e4m3.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3.restype = ctypes.c_double
    lib.orc_e8m0.argtypes = [ctypes.c_uint8]
    lib.orc_e8m0.restype = ctypes.c_double
    lib.orc_bf16.argtypes = [ctypes.c_uint16]
    lib.orc_bf16.restype = ctypes.c_double
    lib.orc_n_visible.argtypes = [I, I, I]
    lib.orc_n_visible.restype = I
    lib.orc_e2m1.argtypes = [ctypes.c_uint8]
    lib.orc_e2m1.restype = ctypes.c_double
    lib.orc_index_scores.argtypes = [I, P, P, P, P, P, I, I, I, I, I, I, I, P]
    lib.orc_index_scores.restype = I
    lib.orc_topk_width.argtypes = [I, I, I, I]
    lib.orc_topk_width.restype = I
    lib.orc_topk.argtypes = [P, I, I, I, I, I, I, P]
    lib.orc_topk.restype = I
    lib.orc_candidate_blocks_width.argtypes = [I, I, I, I, I]
    lib.orc_candidate_blocks_width.restype = I
    lib.orc_candidate_blocks.argtypes = [P, I, I, I, I, I, I, I, P]
    lib.orc_candidate_blocks.restype = I
    lib.orc_window_width.argtypes = [I, I, I]
    lib.orc_window_width.restype = I
    lib.orc_window_indices.argtypes = [I, I, I, I, I, P]
    lib.orc_window_indices.restype = I
    lib.orc_sparse_attn.argtypes = [P, I, I, I, I, I, P, I, P, I, P, I, P, I, P,
                                    ctypes.c_double, P]
    lib.orc_sparse_attn.restype = I
    lib.orc_sparse_attn_fmt.argtypes = [P, I, I, I, I, I, I, P, P, I, P, I, I, P, P, I, P, I, P,
                                        ctypes.c_double, P]
    lib.orc_sparse_attn_fmt.restype = I
    lib.orc_round_bf16.argtypes = [ctypes.c_double]
    lib.orc_round_bf16.restype = ctypes.c_double
    lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_quant_e4m3.argtypes = [P, I, P, P]
    lib.orc_quant_e4m3.restype = None
    lib.orc_quant_e2m1.argtypes = [P, I, P, P]
    lib.orc_quant_e2m1.restype = None
    lib.orc_compress_append.argtypes = [I, I, I, I, P, P, P, P, P, ctypes.c_double, P, I, P, P, I, P, P, P]
    lib.orc_compress_write.argtypes = [I, P, P, I, I, P, P]
    lib.orc_compress_write.restype = I
    lib.orc_compress_append.restype = I
    lib.orc_window_append.argtypes = [I, I, I, P, P, I, I, P, P]
    lib.orc_window_append.restype = I
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = I
    lib.orc_set_num_threads.argtypes = [I]
    lib.orc_set_num_threads.restype = None
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = _bind(_LIB)
    return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Run the wrappers against another build of the oracle source (used by the
    mutation tests, which compile deliberately broken copies on the CPU)."""
    global _lib
    saved = _load()
    _lib = _bind(path)
    try:
        yield
    finally:
        _lib = saved


class OracleError(RuntimeError):
    pass


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} refused its arguments (code {rc})")


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# -- byte formats -----------------------------------------------------------

def e4m3_value(code: int) -> float:
    return _load().orc_e4m3(code)


def e8m0_value(code: int) -> float:
    return _load().orc_e8m0(code)


def e2m1_value(code: int) -> float:
    """Value of one 4-bit e2m1 code (0..15)."""
    return _load().orc_e2m1(code)


def bf16_value(bits: int) -> float:
    return _load().orc_bf16(bits)


def decode_e4m3(codes) -> np.ndarray:
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.orc_e4m3(int(c)) for c in codes.ravel()]).reshape(codes.shape)


# -- steps --------------------------------------------------------------------

def n_visible(start_pos: int, i: int, ratio: int) -> int:
    return _load().orc_n_visible(start_pos, i, ratio)


def topk_width(S: int, start_pos: int, ratio: int, index_topk: int) -> int:
    return _load().orc_topk_width(S, start_pos, ratio, index_topk)


def window_width(S: int, start_pos: int, W: int) -> int:
    return _load().orc_window_width(S, start_pos, W)


# index-code formats: one e4m3 byte per element, or two e2m1 codes per byte
INDEX_FORMATS = {"e4m3": 0, "e2m1": 1}


def index_scores(q8, q_sc, w, k8, k_sc, start_pos: int, ratio: int,
                 fmt: str = "e4m3") -> np.ndarray:
    """Scores [B,S,T] (float64, -inf where invisible), T = (start_pos+S)//ratio.

    ``fmt`` names the code format of ``q8`` / ``k8``: "e4m3" ([..., Di] bytes) or
    "e2m1" ([..., Di/2] bytes, element 2j in the low nibble of byte j).  Di is taken
    from the scale arrays (one byte per 32 elements)."""
    q8 = _c(q8, np.uint8)
    q_sc = _c(q_sc, np.uint8)
    w = _c(w, np.float32)
    k8 = _c(k8, np.uint8)
    k_sc = _c(k_sc, np.uint8)
    B, S, Hi, _ = q8.shape
    Di = 32 * q_sc.shape[-1]
    per_byte = 2 if fmt == "e2m1" else 1
    if q8.shape[-1] * per_byte != Di or k8.shape[-1] * per_byte != Di:
        raise OracleError(f"code rows do not hold {Di} {fmt} elements")
    T_cap = k8.shape[1]
    T = (start_pos + S) // ratio
    out = np.empty((B, S, T), dtype=np.float64)
    rc = _load().orc_index_scores(INDEX_FORMATS[fmt], _ptr(q8), _ptr(q_sc), _ptr(w), _ptr(k8),
                                  _ptr(k_sc), B, S, Hi, Di, T_cap, start_pos, ratio, _ptr(out))
    _check(rc, "orc_index_scores")
    return out


def topk(scores, start_pos: int, ratio: int, index_topk: int) -> np.ndarray:
    """Top-k row lists [B,S,k_eff] int32: ascending, -1 padded."""
    scores = _c(scores, np.float64)
    B, S, ld = scores.shape
    keff = topk_width(S, start_pos, ratio, index_topk)
    out = np.empty((B, S, keff), dtype=np.int32)
    rc = _load().orc_topk(_ptr(scores), ld, B, S, start_pos, ratio, index_topk, _ptr(out))
    _check(rc, "orc_topk")
    return out


def candidate_blocks_width(S: int, start_pos: int, ratio: int, topk_blocks: int,
                           block_size: int) -> int:
    return _load().orc_candidate_blocks_width(S, start_pos, ratio, topk_blocks, block_size)


def candidate_blocks(scores, start_pos: int, ratio: int, topk_blocks: int,
                     block_size: int) -> np.ndarray:
    """Level one of the two-level top-k: kept block numbers [B,S,kb] int32, ascending,
    -1 padded (kb = min(topk_blocks, ceil(T / block_size)))."""
    scores = _c(scores, np.float64)
    B, S, ld = scores.shape
    kb = candidate_blocks_width(S, start_pos, ratio, topk_blocks, block_size)
    out = np.empty((B, S, kb), dtype=np.int32)
    rc = _load().orc_candidate_blocks(_ptr(scores), ld, B, S, start_pos, ratio, topk_blocks,
                                      block_size, _ptr(out))
    _check(rc, "orc_candidate_blocks")
    return out


def apply_candidates(scores, blocks, block_size: int) -> np.ndarray:
    """Level two's mask (DeepSeek-V4.1-Flash-NVFP4 model.py, Indexer.forward): every
    score outside the listed blocks becomes -inf.  scores [B,S,T], blocks [B,S,kb]."""
    scores = np.array(scores, dtype=np.float64)
    B, S, T = scores.shape
    keep = np.zeros((B, S, T), dtype=bool)
    for b in range(B):
        for i in range(S):
            for j in blocks[b, i]:
                if j >= 0:
                    keep[b, i, j * block_size:(j + 1) * block_size] = True
    scores[~keep] = -np.inf
    return scores


def window_indices(B: int, S: int, start_pos: int, W: int, R: int) -> np.ndarray:
    width = window_width(S, start_pos, W)
    out = np.empty((B, S, width), dtype=np.int32)
    rc = _load().orc_window_indices(B, S, start_pos, W, R, _ptr(out))
    _check(rc, "orc_window_indices")
    return out


# KV row formats: bf16, e4m3 with ue8m0 per 32 (window), fp4 e2m1 with e4m3 per 16
# (compressed)
KV_FORMATS = {"bf16": 0, "e4m3": 1, "e2m1": 2}


def sparse_attn(q, win_kv, win_idx, comp_kv, comp_idx, sink, scale: float,
                dv: int | None = None, win_fmt: str = "bf16", win_sc=None,
                comp_fmt: str = "bf16", comp_sc=None) -> np.ndarray:
    """Attention output [B,S,H,dv] float64.  q is bf16 bits; each KV source is bf16 bits
    (uint16) or, with its format "e4m3" / "e2m1", uint8 codes plus uint8 scales."""
    q = _c(q, np.uint16)
    B, S, H, D = q.shape
    dv = D if dv is None else dv

    def src(kv, sc, fmt):
        if fmt == "bf16":
            return _c(kv, np.uint16), None
        return _c(kv, np.uint8), _c(sc, np.uint8)
    if win_idx is None or win_idx.shape[-1] == 0:
        W, R, win_kv_c, win_sc_c, win_idx_c = 0, 0, None, None, None
    else:
        win_kv_c, win_sc_c = src(win_kv, win_sc, win_fmt)
        win_idx_c = _c(win_idx, np.int32)
        W, R = win_idx_c.shape[-1], win_kv_c.shape[1]
    if comp_idx is None or comp_idx.shape[-1] == 0:
        K, T_cap, comp_kv_c, comp_sc_c, comp_idx_c = 0, 0, None, None, None
    else:
        comp_kv_c, comp_sc_c = src(comp_kv, comp_sc, comp_fmt)
        comp_idx_c = _c(comp_idx, np.int32)
        K, T_cap = comp_idx_c.shape[-1], comp_kv_c.shape[1]
    sink_c = None if sink is None else _c(sink, np.float32)
    out = np.empty((B, S, H, dv), dtype=np.float64)
    rc = _load().orc_sparse_attn_fmt(_ptr(q), B, S, H, D, dv, KV_FORMATS[win_fmt], _ptr(win_kv_c),
                                     _ptr(win_sc_c), R, _ptr(win_idx_c), W, KV_FORMATS[comp_fmt],
                                     _ptr(comp_kv_c), _ptr(comp_sc_c), T_cap, _ptr(comp_idx_c), K,
                                     _ptr(sink_c), float(scale), _ptr(out))
    _check(rc, "orc_sparse_attn_fmt")
    return out


def sparse_attn_layers(q, win_kv, win_idx, comp_kv, comp_idx, sink, scale: float,
                       dv: int | None = None) -> np.ndarray:
    """Several layers over one shared row list (DeepSeek-V4.1-Flash-NVFP4 model.py: layers
    between index sources reuse the source's top-k and compressed KV): layer l is
    sparse_attn with its own q[l], win_kv[l] and sink[l].  Returns [L,B,S,H,dv]."""
    L = q.shape[0]
    return np.stack([sparse_attn(q[l], None if win_kv is None else win_kv[l], win_idx, comp_kv,
                                 comp_idx, None if sink is None else sink[l], scale, dv)
                     for l in range(L)])


def step(inp, fp32_scores: bool = True, cand_in=None, cand_topk_blocks: int = 0,
         cand_block_size: int = 0) -> dict:
    """The whole step: index scores -> top-k -> window rows -> attention.

    ``inp`` is a ``lightning_indexer_top_amd.synth.StepInputs``-like object (numpy
    arrays plus sizes).  With ``fp32_scores`` the scores are rounded to float32 before
    selection, so the oracle takes its top-k decision in the precision the kernel keeps
    its scores in; the scores themselves are still the exact fp64 values.

    Two-level top-k: ``cand_topk_blocks`` > 0 makes this layer the candidate source (its
    kept blocks are returned as "cand"); ``cand_in`` (blocks [B,S,kb]) makes it a level-two
    layer whose top-k runs over the scores masked to those blocks ("scores" stay unmasked).
    """
    s = index_scores(inp.q8, inp.q_sc, inp.w, inp.k8, inp.k_sc, inp.start_pos, inp.ratio,
                     getattr(inp, "index_fmt", "e4m3"))
    sel = s.astype(np.float32).astype(np.float64) if fp32_scores else s
    res = {"scores": s}
    if cand_topk_blocks > 0:
        res["cand"] = candidate_blocks(sel, inp.start_pos, inp.ratio, cand_topk_blocks,
                                       cand_block_size)
    if cand_in is not None:
        sel = apply_candidates(sel, cand_in, cand_block_size)
        res["masked"] = sel
    idx = topk(sel, inp.start_pos, inp.ratio, inp.index_topk)
    win = window_indices(inp.B, inp.S, inp.start_pos, inp.W, inp.R)
    o = sparse_attn(inp.q, inp.win_kv, win, inp.comp_kv, idx, inp.sink, inp.scale, inp.dv,
                    getattr(inp, "win_kv_fmt", "bf16"), getattr(inp, "win_sc", None),
                    getattr(inp, "comp_kv_fmt", "bf16"), getattr(inp, "comp_sc", None))
    res.update({"idx": idx, "win_idx": win, "out": o})
    return res


# -- producer side: the cache writes of one decode step --------------------------

def round_bf16(x: float) -> float:
    return _load().orc_round_bf16(float(x))


def e4m3_encode(y: float) -> int:
    return int(_load().orc_e4m3_encode(float(y)))


def quant_e4m3(x) -> tuple:
    """e4m3 codes [..., D] and ue8m0 scales [..., D/32] of float64 rows."""
    x = _c(x, np.float64)
    D = x.shape[-1]
    rows = x.reshape(-1, D)
    codes = np.empty(rows.shape, dtype=np.uint8)
    scales = np.empty((rows.shape[0], D // 32), dtype=np.uint8)
    for r in range(rows.shape[0]):
        _load().orc_quant_e4m3(_ptr(rows[r]), D, _ptr(codes[r]), _ptr(scales[r]))
    return codes.reshape(x.shape), scales.reshape(*x.shape[:-1], D // 32)


def quant_e2m1(x) -> tuple:
    """Packed e2m1 codes [..., D/2] and e4m3 scales [..., D/16] of float64 rows."""
    x = _c(x, np.float64)
    D = x.shape[-1]
    rows = x.reshape(-1, D)
    codes = np.empty((rows.shape[0], D // 2), dtype=np.uint8)
    scales = np.empty((rows.shape[0], D // 16), dtype=np.uint8)
    for r in range(rows.shape[0]):
        _load().orc_quant_e2m1(_ptr(np.ascontiguousarray(rows[r])), D, _ptr(codes[r]), _ptr(scales[r]))
    return codes.reshape(*x.shape[:-1], D // 2), scales.reshape(*x.shape[:-1], D // 16)


def compress_append(kv, score, kv_state, score_state, norm_w, eps: float, freqs, rd: int,
                    codes, scales, start_pos: int, ratio: int, raw: bool = False):
    """One decode step of the compressor and the compressed-cache write (in place on
    kv_state / score_state / codes / scales).  Returns (row written?, latent [B, D]),
    and with raw=True also the pooled kv and the norm's result before their bf16
    roundings ([B, D] each)."""
    kv = _c(kv, np.float32)
    score = _c(score, np.float32)
    B, D = kv.shape
    for a, n in ((kv_state, "kv_state"), (score_state, "score_state")):
        if ratio > 1 and (a.dtype != np.float32 or not a.flags.c_contiguous):
            raise OracleError(f"{n} must be contiguous float32 (updated in place)")
    for a in (codes, scales):
        if a.dtype != np.uint8 or not a.flags.c_contiguous:
            raise OracleError("codes / scales must be contiguous uint8 (updated in place)")
    latent = np.zeros((B, D), dtype=np.float64)
    pooled = np.zeros((B, D), dtype=np.float64)
    normed = np.zeros((B, D), dtype=np.float64)
    rc = _load().orc_compress_append(B, D, ratio, start_pos, _ptr(kv), _ptr(score),
                                     _ptr(kv_state) if ratio > 1 else None,
                                     _ptr(score_state) if ratio > 1 else None,
                                     _ptr(_c(norm_w, np.float32)), float(eps),
                                     _ptr(_c(freqs, np.float32)), rd, _ptr(codes), _ptr(scales),
                                     codes.shape[1], _ptr(latent), _ptr(pooled), _ptr(normed))
    if rc < 0:
        _check(rc, "orc_compress_append")
    if raw:
        return bool(rc), latent, pooled, normed
    return bool(rc), latent


def compress_write(latent, freqs, rd: int, pos: int) -> tuple:
    """The compressed-cache row of one pre-rotation latent [D] (bf16 values): rotated at
    `pos`, quantised; returns (codes [D/2], scales [D/16])."""
    lat = _c(latent, np.float64)
    D = lat.shape[-1]
    codes = np.zeros(D // 2, np.uint8)
    scales = np.zeros(D // 16, np.uint8)
    _check(_load().orc_compress_write(D, _ptr(lat), _ptr(_c(freqs, np.float32)), rd, pos, _ptr(codes),
                                      _ptr(scales)), "orc_compress_write")
    return codes, scales


def compress_chunk(kv, score, kv_state, score_state, norm_w, eps: float, freqs, rd: int,
                   codes, scales, start_pos: int, ratio: int):
    """A chunk of S tokens per sequence into the compressor: by definition the S decode
    steps start_pos, start_pos + 1, ... in order (at start_pos 0 this is the pages'
    prefill branch: whole groups pooled, the remainder left in the state).  kv, score
    [B, S, D].  Returns (rows written, latents [B, rows, D], pooled_raw, norm_raw)."""
    kv = _c(kv, np.float32)
    score = _c(score, np.float32)
    B, S, D = kv.shape
    lat, pooled, normed = [], [], []
    for t in range(S):
        w, l, pr, nr = compress_append(kv[:, t], score[:, t], kv_state, score_state, norm_w, eps, freqs, rd,
                                       codes, scales, start_pos + t, ratio, raw=True)
        if w:
            lat.append(l)
            pooled.append(pr)
            normed.append(nr)
    stack = lambda xs: np.stack(xs, axis=1) if xs else np.zeros((B, 0, D))  # noqa: E731
    return len(lat), stack(lat), stack(pooled), stack(normed)


def window_chunk(kv_bits, freqs, rd: int, codes, scales, start_pos: int):
    """A chunk of S bf16 window rows per sequence ([B, S, D]) into the ring: by definition
    the S decode-step writes in order (a later position takes a slot an earlier one held;
    at start_pos 0 this is the pages' prefill seeding of the ring)."""
    kv_bits = _c(kv_bits, np.uint16)
    for t in range(kv_bits.shape[1]):
        window_append(kv_bits[:, t], freqs, rd, codes, scales, start_pos + t)


def window_append(kv_bits, freqs, rd: int, codes, scales, start_pos: int):
    """One decode step's window-cache write (in place on codes [B,R,D] / scales)."""
    kv_bits = _c(kv_bits, np.uint16)
    B, D = kv_bits.shape
    for a in (codes, scales):
        if a.dtype != np.uint8 or not a.flags.c_contiguous:
            raise OracleError("codes / scales must be contiguous uint8 (updated in place)")
    rc = _load().orc_window_append(B, D, start_pos, _ptr(kv_bits), _ptr(_c(freqs, np.float32)), rd,
                                   codes.shape[1], _ptr(codes), _ptr(scales))
    _check(rc, "orc_window_append")


def num_threads() -> int:
    return _load().orc_num_threads()


def set_num_threads(n: int) -> None:
    _load().orc_set_num_threads(n)
