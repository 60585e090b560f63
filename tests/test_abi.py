"""CPU checks of the C ABI: liblit.so loads, exports every entry point include/lit.h
declares, and refuses bad arguments on the host before anything is launched.  No call
here reaches a kernel launch (no GPU is needed)."""
import ctypes
import os
import re

import pytest

import lightning_indexer_top_amd as L
from lightning_indexer_top_amd import lit as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lit.h")
A = 0x10000      # a 16-byte aligned stand-in address; never dereferenced on refusal
MIS = 0x10001    # misaligned stand-in


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from lightning_indexer_top_amd import build as bld
        bld.build()
    return L.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lit_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
        assert n in B.SIGNATURES, f"binding lacks {n}"
    assert set(B.SIGNATURES) == set(names)


def test_version_and_status_strings(lib):
    assert lib.lit_abi_version() == 2
    for code, name in B.STATUS_NAMES.items():
        assert lib.lit_status_str(code).decode().startswith(name)
    assert b"unknown" in lib.lit_status_str(99)


def test_topk_width_matches_oracle(lib, orc):
    """k_eff from the library equals the oracle's rule on a grid of shapes."""
    for S in (0, 1, 5, 4096):
        for start_pos in (0, 1, 7, 1023, 12288, 131071):
            for ratio in (1, 2, 3, 4):
                for k in (0, 1, 64, 2048):
                    assert lib.lit_topk_width(S, start_pos, ratio, k) == \
                        orc.topk_width(S, start_pos, ratio, k), (S, start_pos, ratio, k)
    assert lib.lit_topk_width(1, 100, 0, 64) == 0
    assert lib.lit_topk_width(-1, 100, 2, 64) == 0


def test_compress_writes_row_matches_oracle(lib, orc):
    """The library's group-completion answer equals whether the oracle's compressor
    writes a cache row at that position (one sequence, D = 32, no rotation)."""
    import numpy as np
    for ratio in (1, 2, 3, 4):
        ks = np.zeros((1, ratio, 32), np.float32)
        gs = np.full((1, ratio, 32), -np.inf, np.float32)
        codes = np.zeros((1, 8, 16), np.uint8)
        scales = np.zeros((1, 8, 2), np.uint8)
        kv = np.ones((1, 32), np.float32)
        for pos in range(2 * ratio + 1):
            wrote, _ = orc.compress_append(kv, kv, ks if ratio > 1 else None, gs if ratio > 1 else None,
                                           np.ones(32, np.float32), 1e-6, np.zeros((16, 0, 2), np.float32),
                                           0, codes, scales, pos, ratio)
            assert lib.lit_compress_writes_row(pos, ratio) == int(wrote), (pos, ratio)
    assert lib.lit_compress_writes_row(5, 0) == 0
    assert lib.lit_compress_writes_row(-1, 2) == 0


def test_step_sizing_of_an_empty_batch(lib):
    """B = 0 or S = 0: nothing to size (the attention plan once divided by the query count)."""
    args = B.lit_step_args()
    args.B, args.S, args.start_pos, args.ratio, args.Hi, args.Di = 0, 1, 1023, 2, 16, 64
    args.index_topk, args.T_cap, args.H, args.D, args.dv, args.W, args.R = 64, 512, 16, 128, 128, 128, 128
    for f in ("q8", "q_sc", "w", "k8", "k_sc", "q", "win_kv", "comp_kv", "topk_idx", "out"):
        setattr(args, f, A)
    lib.lit_sparse_step_workspace_bytes(ctypes.byref(args))
    args.B, args.S = 1, 0
    lib.lit_sparse_step_workspace_bytes(ctypes.byref(args))
    assert lib.lit_sparse_step(ctypes.byref(args), None, 0, None) == 0


def test_noalloc_refusals(lib):
    """The no-allocation step refuses a workspace beyond its scratch before any launch, and
    does nothing for an empty batch."""
    args = B.lit_step_args()
    args.B, args.S, args.start_pos, args.ratio, args.Hi, args.Di = 1, 4096, 12288, 2, 16, 64
    args.index_topk, args.T_cap, args.H, args.D, args.dv, args.W, args.R = 512, 8192, 16, 128, 128, 128, 4223
    for f in ("q8", "q_sc", "w", "k8", "k_sc", "q", "win_kv", "comp_kv", "topk_idx", "out"):
        setattr(args, f, A)
    assert lib.lit_sparse_step_noalloc(ctypes.byref(args), None, None) == 5   # LIT_E_WORKSPACE
    args.B = 0
    assert lib.lit_sparse_step_noalloc(ctypes.byref(args), None, None) == 0
    args.B, args.Di = 1, 48
    assert lib.lit_sparse_step_noalloc(ctypes.byref(args), None, None) == 2


def scores_call(lib, **kw):
    a = dict(q8=A, q_sc=A, w=A, k8=A, k_sc=A, B=1, S=1, Hi=16, Di=64, T_cap=512, start_pos=1023,
             ratio=2, scores=A, ld=512)
    a.update(kw)
    return lib.lit_indexer_scores(a["q8"], a["q_sc"], a["w"], a["k8"], a["k_sc"], a["B"], a["S"],
                                  a["Hi"], a["Di"], a["T_cap"], a["start_pos"], a["ratio"],
                                  a["scores"], a["ld"], None)


def test_indexer_refusals(lib):
    assert scores_call(lib, Di=48) == 2
    assert scores_call(lib, Di=96) == 4
    assert scores_call(lib, Hi=8) == 4
    assert scores_call(lib, Hi=80) == 4
    assert scores_call(lib, Hi=0) == 2
    assert scores_call(lib, T_cap=511) == 2          # T = 512 rows visible
    assert scores_call(lib, ld=510) == 2
    assert scores_call(lib, ld=514) == 3
    assert scores_call(lib, ratio=0) == 2
    assert scores_call(lib, k8=None) == 1
    assert scores_call(lib, scores=None) == 1
    assert scores_call(lib, k8=MIS) == 3
    assert scores_call(lib, B=0) == 0                 # nothing to do
    assert scores_call(lib, start_pos=0, S=1, ratio=2) == 0   # T = 0


def test_indexer_format_refusals(lib):
    def fmt_call(fmt, **kw):
        a = dict(q8=A, q_sc=A, w=A, k8=A, k_sc=A, B=1, S=1, Hi=16, Di=64, T_cap=512,
                 start_pos=1023, ratio=2, scores=A, ld=512)
        a.update(kw)
        return lib.lit_indexer_scores_fmt(fmt, a["q8"], a["q_sc"], a["w"], a["k8"], a["k_sc"],
                                          a["B"], a["S"], a["Hi"], a["Di"], a["T_cap"],
                                          a["start_pos"], a["ratio"], a["scores"], a["ld"], None)
    assert fmt_call(2) == 4 and fmt_call(-1) == 4       # unknown format
    assert fmt_call(1, Di=96) == 4 and fmt_call(1, Di=48) == 2
    assert fmt_call(1, k8=None) == 1 and fmt_call(1, q8=MIS) == 3
    assert fmt_call(1, B=0) == 0
    assert B.INDEX_FORMATS == {"e4m3": 0, "e2m1": 1}


def test_candidate_refusals(lib):
    f, g = lib.lit_candidate_blocks, lib.lit_topk_candidates
    need = lib.lit_candidate_blocks_workspace_bytes(2, 1, 65535, 2, 8)
    assert need >= 2 * 4096 * 4 and need % 256 == 0
    assert lib.lit_candidate_blocks_width(1, 65535, 2, 2048, 8) == 2048
    assert lib.lit_candidate_blocks_width(1, 1023, 2, 2048, 8) == 64
    assert lib.lit_candidate_blocks_width(1, 1023, 2, 2048, 0) == 0
    assert f(A, 32768, 2, 1, 65535, 2, 2048, 0, A, A, need, None) == 2      # block size 0
    assert f(A, 32768, 2, 1, 65535, 2, 2048, 8, A, None, 0, None) == 5      # no workspace
    assert f(A, 32768, 2, 1, 65535, 2, 2048, 8, A, A, need - 1, None) == 5
    assert f(A, 32770, 2, 1, 65535, 2, 2048, 8, A, A, need, None) == 3      # ld not a multiple of 4
    assert f(A, 32764, 2, 1, 65535, 2, 2048, 8, A, A, need, None) == 2      # ld < T
    assert f(A, 32768, 2, 1, 65535, 2, 2048, 8, None, A, need, None) == 1
    assert f(A, 32768, 0, 1, 65535, 2, 2048, 8, None, None, 0, None) == 0   # nothing to do
    assert g(A, 32768, 2, 1, 65535, 2, 2048, A, 2048, 0, A, None, 0, None) == 2
    assert g(A, 32768, 2, 1, 65535, 2, 2048, None, 2048, 8, A, None, 0, None) == 1
    assert g(A, 1 << 20, 1, 1, (1 << 20) - 1, 1, 64, A, 8, 1, A, None, 0, None) == 4  # bitmap too big


def test_topk_refusals(lib):
    f = lib.lit_topk
    assert f(A, 8, 1, 1, 1023, 2, 64, A, None, 0, None) == 2        # ld < T
    assert f(A, 514, 1, 1, 1023, 2, 64, A, None, 0, None) == 3      # ld not a multiple of 4
    assert f(None, 512, 1, 1, 1023, 2, 64, A, None, 0, None) == 1
    assert f(A, 512, 1, 1, 1023, 2, 64, None, None, 0, None) == 1
    assert f(A, 512, 1, 1, 1023, 2, -1, A, None, 0, None) == 2
    assert f(A, 512, 1, 1, 1023, 2, 0, None, None, 0, None) == 0    # k = 0: nothing
    assert lib.lit_topk_workspace_bytes(8, 1, 16383, 2, 2048) == 0


def attn_call(lib, **kw):
    a = dict(q=A, B=1, S=1, H=16, D=128, dv=128, win_kv=A, R=128, win_idx=A, W=128, comp_kv=A,
             T_cap=512, comp_idx=A, K=64, sink=None, scale=0.1, out=A, ws=A, ws_bytes=1 << 30)
    a.update(kw)
    return lib.lit_sparse_attn(a["q"], a["B"], a["S"], a["H"], a["D"], a["dv"], a["win_kv"], a["R"],
                               a["win_idx"], a["W"], a["comp_kv"], a["T_cap"], a["comp_idx"], a["K"],
                               a["sink"], a["scale"], a["out"], a["ws"], a["ws_bytes"], None)


def test_attention_refusals(lib):
    assert attn_call(lib, H=32) == 4
    assert attn_call(lib, D=96, dv=96) == 4
    assert attn_call(lib, dv=256) == 2
    assert attn_call(lib, dv=40) == 4
    assert attn_call(lib, R=0) == 2
    assert attn_call(lib, q=None) == 1
    assert attn_call(lib, comp_idx=None) == 1
    assert attn_call(lib, win_kv=None) == 1
    assert attn_call(lib, comp_kv=MIS) == 3
    need = lib.lit_sparse_attn_workspace_bytes(1, 1, 16, 128, 128, 2048)
    assert need > 0
    assert attn_call(lib, K=2048, T_cap=4096, ws=None, ws_bytes=0) == 5
    assert attn_call(lib, K=2048, T_cap=4096, ws_bytes=need - 1) == 5
    assert attn_call(lib, B=0) == 0
    # one sequence's source must stay below 2 GiB (rows are addressed by 32-bit offsets)
    assert attn_call(lib, T_cap=(1 << 23)) == 4      # 8M rows x 128 dims x 2 bytes = 2 GiB
    assert attn_call(lib, R=(1 << 23)) == 4
    assert attn_call(lib, T_cap=(1 << 23) - 1, B=0) == 0


def test_attention_layers_refusals(lib):
    f = lib.lit_sparse_attn_layers

    def call(L=3, B=8, S=1, W=128, start_pos=16383, R=128, ws_bytes=1 << 30, win_idx=None, **kw):
        a = dict(q=A, H=16, D=192, dv=192, win_kv=A, comp_kv=A, T_cap=8192, comp_idx=A, K=2048,
                 sink=None, out=A, ws=A)
        a.update(kw)
        return f(L, a["q"], B, S, a["H"], a["D"], a["dv"], a["win_kv"], R, win_idx, W, start_pos,
                 a["comp_kv"], a["T_cap"], a["comp_idx"], a["K"], a["sink"], 0.07, a["out"], a["ws"],
                 ws_bytes, None)
    assert call(L=0) == 2
    assert call(L=5000, B=8, S=2, R=129) == 4           # L*B*S > 65535
    assert call(R=64) == 2                               # derived window needs 128 slots
    assert call(win_kv=None) == 1
    assert call(H=32) == 4
    assert call(start_pos=-1) == 2
    need = lib.lit_sparse_attn_layers_workspace_bytes(3, 8, 1, 16, 192, 128, 2048)
    assert need > lib.lit_sparse_attn_workspace_bytes(8, 1, 16, 192, 128, 2048)
    assert call(ws=None, ws_bytes=0) == 5
    assert call(ws_bytes=need - 1) == 5
    assert call(B=0) == 0
    assert lib.lit_sparse_attn_layers_workspace_bytes(0, 8, 1, 16, 192, 128, 2048) == 0


def test_quantised_kv_refusals(lib):
    f = lib.lit_sparse_attn_fmt

    def call(wf=1, cf=2, wsc=A, csc=A, **kw):
        a = dict(q=A, B=1, S=1, H=16, D=128, dv=128, win_kv=A, R=128, win_idx=A, W=128, comp_kv=A,
                 T_cap=512, comp_idx=A, K=64, ws=A, ws_bytes=1 << 30)
        a.update(kw)
        return f(a["q"], a["B"], a["S"], a["H"], a["D"], a["dv"], wf, a["win_kv"], wsc, a["R"],
                 a["win_idx"], a["W"], cf, a["comp_kv"], csc, a["T_cap"], a["comp_idx"], a["K"], None,
                 0.1, A, a["ws"], a["ws_bytes"], None)
    assert call(wf=2) == 4 and call(cf=1) == 4 and call(wf=7) == 4   # formats per source
    assert call(wsc=None) == 1 and call(csc=None) == 1
    assert call(B=0) == 0


def test_producer_refusals(lib):
    f, g = lib.lit_compress_append, lib.lit_window_append
    def call(**kw):
        a = dict(B=2, D=192, ratio=4, sp=7, kv=A, sc=A, ks=A, gs=A, w=A, eps=1e-20, fr=A, n=64,
                 rd=64, c=A, s=A, T=2, lat=None, st=None)
        a.update(kw)
        return f(*[a[k] for k in ("B", "D", "ratio", "sp", "kv", "sc", "ks", "gs", "w", "eps",
                                  "fr", "n", "rd", "c", "s", "T", "lat", "st")])
    assert call(D=80) == 2 and call(D=288) == 4 and call(rd=63) == 2 and call(rd=224) == 2
    assert call(T=1) == 2                       # row 7/4 = 1 needs two rows
    assert call(n=4) == 2                       # rotation position 4 is outside the table
    assert call(ks=None) == 1 and call(c=None) == 1
    assert call(ratio=0) == 2 and call(B=0) == 0
    assert g(2, 192, 70, A, A, 64, 64, A, A, 128, None) == 2   # position 70 outside the table
    assert g(2, 192, 7, None, A, 64, 64, A, A, 128, None) == 1
    assert g(2, 192, 7, A, A, 64, 64, A, A, 0, None) == 2
    assert g(0, 192, 7, A, A, 64, 64, A, A, 128, None) == 0


def test_window_refusals(lib):
    assert lib.lit_window_indices(1, 8, 100, 16, 16, A, None) == 2   # needs 23 slots
    assert lib.lit_window_indices(1, 8, 100, 16, 23, None, None) == 1
    assert lib.lit_window_indices(-1, 8, 100, 16, 23, A, None) == 2
    assert lib.lit_window_indices(0, 8, 100, 16, 23, None, None) == 0
    assert lib.lit_window_width(5, 0, 128) == 5
    assert lib.lit_window_width(1, 1023, 128) == 128


def test_step_refusals(lib):
    args = B.lit_step_args(B=8, S=1, start_pos=16383, ratio=2, Hi=64, Di=128, index_topk=2048,
                           T_cap=8192, q8=A, q_sc=A, w=A, k8=A, k_sc=A, H=16, D=192, dv=192, W=128,
                           R=128, q=A, win_kv=A, comp_kv=A, sink=0, scale=0.07, topk_idx=A, out=A)
    need = lib.lit_sparse_step_workspace_bytes(ctypes.byref(args))
    assert need >= 8 * 8192 * 4
    assert lib.lit_sparse_step(None, A, need, None) == 1
    assert lib.lit_sparse_step(ctypes.byref(args), A, 100, None) == 5
    assert lib.lit_sparse_step(ctypes.byref(args), None, 0, None) == 5
    assert lib.lit_sparse_step(ctypes.byref(args), A + 16, need, None) == 3   # not 256-aligned
    args.T_cap = 4000
    assert lib.lit_sparse_step(ctypes.byref(args), A, need, None) == 2
    args.T_cap = 8192
    args.R = 64                                                             # window ring too small
    assert lib.lit_sparse_step(ctypes.byref(args), A, need, None) == 2
    args.R = 128
    args.topk_idx = 0
    assert lib.lit_sparse_step(ctypes.byref(args), A, need, None) == 1
    assert lib.lit_sparse_step_workspace_bytes(None) == 0
    assert lib.lit_sparse_step_state_bytes(None) == 0
    args.topk_idx = A
    args.index_format = 3                                                   # unknown format
    assert lib.lit_sparse_step(ctypes.byref(args), A, need, None) == 4
    assert lib.lit_sparse_step_workspace_bytes(ctypes.byref(args)) == 0
    args.index_format = 1
    assert lib.lit_sparse_step_workspace_bytes(ctypes.byref(args)) >= need


def test_step_state_sizes(lib):
    """The fused form's state size is queried without a GPU only when the device can be
    asked; here (no GPU) the plan cannot size the teams and reports 0 (multi-kernel)."""
    args = B.lit_step_args(B=8, S=1, start_pos=16383, ratio=2, Hi=64, Di=128, index_topk=2048,
                           T_cap=8192, q8=A, q_sc=A, w=A, k8=A, k_sc=A, H=16, D=192, dv=192, W=128,
                           R=128, q=A, win_kv=A, comp_kv=A, sink=0, scale=0.07, topk_idx=A, out=A)
    n = lib.lit_sparse_step_state_bytes(ctypes.byref(args))
    assert n == 0 or n >= 256 + 8 * (32 + 4096 * 4)
    args.flags = 1
    assert lib.lit_sparse_step_state_bytes(ctypes.byref(args)) == 0


def test_step_args_keep_their_tensors_alive():
    """make_step_args stores raw addresses; the struct must keep the tensors behind them
    alive, or temporaries passed by a caller would be freed and their memory reused."""
    import gc
    import weakref
    import torch
    t = lambda *shape, dt=torch.uint8: torch.zeros(*shape, dtype=dt)  # noqa: E731
    q8 = t(1, 1, 16, 64)
    ref = weakref.ref(q8)
    args, idx, out = B.make_step_args(
        q8=q8, q_sc=t(1, 1, 16, 2), w=t(1, 1, 16, dt=torch.float32), k8=t(1, 512, 64),
        k_sc=t(1, 512, 2), q=t(1, 1, 16, 128, dt=torch.bfloat16),
        win_kv=t(1, 128, 128, dt=torch.bfloat16), comp_kv=t(1, 512, 128, dt=torch.bfloat16),
        start_pos=1023, ratio=2, index_topk=64, W=128, scale=0.088)
    del q8
    gc.collect()
    assert ref() is not None and args.q8 == ref().data_ptr()
    del args
    gc.collect()
    assert ref() is None


def test_compress_chunk_rows_matches_oracle(lib, orc):
    """The rows a chunk writes (lit_compress_chunk_rows) equal the rows the oracle's chunk
    writes, for chunks starting on and inside groups, and none for bad arguments."""
    import numpy as np
    for ratio in (1, 2, 4):
        for start_pos in (0, 1, 3, 6):
            for S in (0, 1, 3, 4, 9):
                ks = np.zeros((1, ratio, 32), np.float32)
                gs = np.full((1, ratio, 32), -np.inf, np.float32)
                codes = np.zeros((1, 32, 16), np.uint8)
                scales = np.zeros((1, 32, 2), np.uint8)
                kv = np.ones((1, S, 32), np.float32)
                n, _, _, _ = orc.compress_chunk(kv, kv, ks if ratio > 1 else None, gs if ratio > 1 else None,
                                                np.ones(32, np.float32), 1e-6, np.zeros((32, 0, 2), np.float32),
                                                0, codes, scales, start_pos, ratio) if S else (0, None, None, None)
                assert lib.lit_compress_chunk_rows(start_pos, S, ratio) == n, (start_pos, S, ratio)
    assert lib.lit_compress_chunk_rows(0, 8, 0) == 0
    assert lib.lit_compress_chunk_rows(-1, 8, 2) == 0


def test_chunk_producers_refuse_bad_arguments(lib):
    """Refusals happen on the host, before any launch (no GPU is touched here)."""
    import ctypes
    P = ctypes.c_void_p
    fake = P(256)  # never dereferenced: every call below is refused first
    # ratio 0, negative start, D not a multiple of 32, D > 256, row past T_cap, rotation past n_pos
    cases = [
        dict(ratio=0), dict(start_pos=-1), dict(D=48), dict(D=288), dict(T_cap=1), dict(n_pos=4),
    ]
    for over in cases:
        a = dict(B=1, S=8, D=64, ratio=2, start_pos=0, n_pos=64, rd=16, T_cap=16)
        a.update(over)
        st = lib.lit_compress_chunk(a["B"], a["S"], a["D"], a["ratio"], a["start_pos"], fake, fake, fake, fake,
                                    fake, ctypes.c_float(1e-6), fake, a["n_pos"], a["rd"], fake, fake, a["T_cap"],
                                    None, None)
        assert st != 0, over
    st = lib.lit_window_chunk(1, 8, 64, 0, fake, fake, 64, 16, fake, fake, 0, None)   # R = 0
    assert st != 0
    st = lib.lit_window_chunk(1, 8, 64, 60, fake, fake, 64, 16, fake, fake, 128, None)  # position 67 >= n_pos
    assert st != 0
    assert lib.lit_window_chunk(0, 8, 64, 0, None, None, 64, 16, None, None, 128, None) == 0  # empty batch
