"""GPU parity: every entry point of liblit.so against the fp64 oracle, through the C ABI.

Acceptance rules (the tolerances of the sparse-attention step):
* window lists and top-k of identical fp32 scores: bit-exact;
* indexer scores (e4m3 and fp4 e2m1 codes): |gpu - oracle| <= 1e-4 * sum_h w_h sum_d
  |q_hd k_td| + 1e-6 |s| (the MX-scaled MFMA's accumulation error, bounded by the
  magnitudes it sums), and -inf exactly where the oracle has -inf;
* top-k from the full pipeline: sets identical, except rows within 1e-3 relative of the
  oracle's k-th score;
* attention: max |gpu - oracle| <= 2e-2 (bf16 output) given the same selected set.
"""
import numpy as np
import pytest
import torch

import lightning_indexer_top_amd as L
from lightning_indexer_top_amd import synth
from tests.gpu_util import (bf16_dev, bf16_host, dev, score_tolerance, step_inputs_dev,
                            topk_sets_agree)

pytestmark = pytest.mark.gpu

ATTN_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.library()


# ---------------------------------------------------------------------------------
# indexer scores
# ---------------------------------------------------------------------------------
INDEXER_CASES = [
    # B, S, start_pos, ratio, Hi, Di
    (2, 1, 999, 2, 16, 64),      # ragged tail: 500 rows
    (1, 1, 1023, 2, 16, 64),     # the 1K decode shape
    (3, 1, 2047, 1, 32, 128),
    (2, 1, 4095, 2, 64, 128),
    (1, 70, 0, 2, 16, 64),       # prefill from 0, causal rows
    (2, 37, 100, 3, 32, 64),     # chunk after cached tokens, groups of 2 queries
    (1, 45, 300, 4, 64, 128),
    (1, 9, 20, 1, 48, 128),      # three head tiles
    (1, 33, 500, 2, 16, 64),     # 16 heads x 64 in query pairs: a last block of one query
    (2, 19, 1000, 1, 16, 64),    # two sequences, an odd last block, a ragged key tail
]


FORMATS = ["e4m3", "e2m1"]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("B,S,start_pos,ratio,Hi,Di", INDEXER_CASES)
def test_indexer_scores(orc, B, S, start_pos, ratio, Hi, Di, fmt):
    inp = synth.make_step(B=B, S=S, start_pos=start_pos, ratio=ratio, Hi=Hi, Di=Di, H=16, D=64,
                          W=8, index_topk=16, seed=1000 + B * 7 + S + Hi + Di, index_fmt=fmt)
    d = step_inputs_dev(inp)
    got = L.lit_indexer_scores(d["q8"], d["q_sc"], d["w"], d["k8"], d["k_sc"], start_pos, ratio,
                               fmt=fmt)
    torch.cuda.synchronize()
    got = got.cpu().numpy().astype(np.float64)[..., :inp.T]
    want = orc.index_scores(inp.q8, inp.q_sc, inp.w, inp.k8, inp.k_sc, start_pos, ratio, fmt)
    inf = np.isneginf(want)
    assert np.array_equal(np.isneginf(got), inf)
    tol = 1e-4 * score_tolerance(inp) + 1e-6 * np.abs(np.where(inf, 0, want))
    err = np.abs(np.where(inf, 0.0, got) - np.where(inf, 0.0, want))
    assert np.all(err <= tol), f"max err {err.max()} (tol at argmax {tol.flat[err.argmax()]})"


@pytest.mark.parametrize("fmt", FORMATS)
def test_indexer_keys_scaled_by_four(orc, fmt):
    """The decode-4k shape whose boosted key rows (x4: +2 on every scale byte) stand out."""
    inp = synth.workload("decode-4k-r2", index_fmt=fmt)
    d = step_inputs_dev(inp)
    got = L.lit_indexer_scores(d["q8"], d["q_sc"], d["w"], d["k8"], d["k_sc"], inp.start_pos,
                               inp.ratio, fmt=fmt).cpu().numpy().astype(np.float64)[..., :inp.T]
    want = orc.index_scores(inp.q8, inp.q_sc, inp.w, inp.k8, inp.k_sc, inp.start_pos, inp.ratio,
                            fmt)
    tol = 1e-4 * score_tolerance(inp) + 1e-6 * np.abs(want)
    assert np.all(np.abs(got - want) <= tol)


# ---------------------------------------------------------------------------------
# top-k on identical fp32 scores: bit-exact
# ---------------------------------------------------------------------------------
TOPK_CASES = [
    # B, S, start_pos, ratio, k, ties
    (1, 1, 1023, 2, 64, False),
    (4, 1, 4095, 1, 64, False),
    (8, 1, 16383, 2, 2048, False),
    (2, 1, 131071, 4, 2048, False),
    (3, 1, 4095, 2, 300, True),          # many equal scores at the threshold
    (1, 1, 79999, 2, 1000, False),       # 40000 rows: segmented path
    (1, 64, 0, 2, 16, False),            # prefill from 0: short rows padded with -1
    (2, 33, 500, 3, 100, True),
    (1, 1, 9, 1, 64, False),             # k larger than the rows: all of them
]


@pytest.mark.parametrize("B,S,start_pos,ratio,k,ties", TOPK_CASES)
def test_topk_exact(orc, B, S, start_pos, ratio, k, ties):
    T = (start_pos + S) // ratio
    ld = (T + 3) // 4 * 4
    sc = synth.random_scores(B, S, ld, seed=B * 131 + S + k, ties=ties)
    got = L.lit_topk(dev(sc), start_pos, ratio, k)
    torch.cuda.synchronize()
    want = orc.topk(sc.astype(np.float64), start_pos, ratio, k)
    assert np.array_equal(got.cpu().numpy(), want)


def test_topk_all_equal_and_signed_zero(orc):
    sc = np.zeros((2, 1, 1024), np.float32)
    sc[1, 0, ::3] = -0.0
    got = L.lit_topk(dev(sc), 1023, 1, 100)
    want = orc.topk(sc.astype(np.float64), 1023, 1, 100)
    assert np.array_equal(got.cpu().numpy(), want)
    assert np.array_equal(want[0, 0], np.arange(100))


# Rows whose score arrays hold 1025..8192 positions take the row kernel (one workgroup a
# row, whatever the row count); its clustered forms are the candidate refinement (9
# distinct values) and the radix levels (2 distinct values: thousands of scores in the
# cut's bin).  Shorter arrays take the radix kernel.
ROWS_CASES = [
    # B, S, start_pos, ratio, k, kind
    (1, 256, 0, 2, 16, "normal"),        # prefill from 0, 128 positions: the radix kernel
    (2, 160, 16000, 2, 512, "normal"),   # rows of 8000..8079 positions
    (1, 300, 4000, 2, 512, "ties"),
    (1, 256, 9000, 2, 700, "two"),
    (1, 2100, 0, 2, 512, "normal"),      # 1050 positions from 0: rows of fewer than k padded
    (2, 3, 6000, 2, 300, "inf"),         # +inf and -inf among finite visible scores
    (1, 16, 16000, 2, 512, "levels9"),   # ~890 equal scores in the cut's bin: the refinement
                                         # near its 1024-candidate capacity
    (1, 16, 16000, 2, 512, "levels5"),   # ~1600: past that capacity, the radix levels
    (1, 1100, 14000, 2, 512, "levels9"), # the same over 1100 rows
    (1, 1100, 14000, 2, 512, "levels5"),
]


@pytest.mark.parametrize("B,S,start_pos,ratio,k,kind", ROWS_CASES)
def test_topk_many_rows_exact(orc, B, S, start_pos, ratio, k, kind):
    T = (start_pos + S) // ratio
    ld = (T + 3) // 4 * 4
    if kind == "two" or kind.startswith("levels"):
        rng = np.random.Generator(np.random.PCG64(B * 7 + S))
        sc = rng.integers(0, 2 if kind == "two" else int(kind[6:]), size=(B, S, ld)).astype(np.float32)
    elif kind == "inf":
        sc = synth.random_scores(B, S, ld, seed=B * 131 + S + k, ties=False)
        rng = np.random.Generator(np.random.PCG64(5))
        for b in range(B):
            for i in range(S):
                pos = rng.choice(T, 40, replace=False)
                sc[b, i, pos[:10]] = np.inf
                sc[b, i, pos[10:]] = -np.inf
    else:
        sc = synth.random_scores(B, S, ld, seed=B * 131 + S + k, ties=kind == "ties")
    got = L.lit_topk(dev(sc), start_pos, ratio, k)
    torch.cuda.synchronize()
    want = orc.topk(sc.astype(np.float64), start_pos, ratio, k)
    assert np.array_equal(got.cpu().numpy(), want)


# ---------------------------------------------------------------------------------
# window lists
# ---------------------------------------------------------------------------------
@pytest.mark.parametrize("B,S,start_pos,W,R", [(2, 1, 2, 4, 4), (1, 5, 0, 3, 5), (2, 1, 1023, 128, 128),
                                               (1, 4096, 12288, 128, 4223), (1, 300, 0, 128, 300),
                                               (3, 7, 100, 4, 10)])
def test_window_indices(orc, B, S, start_pos, W, R):
    got = L.lit_window_indices(B, S, start_pos, W, R)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), orc.window_indices(B, S, start_pos, W, R))


# ---------------------------------------------------------------------------------
# sparse attention on oracle-chosen index lists
# ---------------------------------------------------------------------------------
def _attn_case(orc, B, S, start_pos, ratio, D, dv, W, k, seed, sink=None, minus_ones=0,
               repeat=False, R=None):
    inp = synth.make_step(B=B, S=S, start_pos=start_pos, ratio=ratio, Hi=16, Di=64, H=16, D=D,
                          W=W, index_topk=k, seed=seed, dv=dv, R=R, sink=sink)
    rng = np.random.default_rng(seed)
    T = inp.T
    keff = inp.k_eff
    comp_idx = np.stack([np.stack([np.sort(rng.choice(T, keff, replace=False)) for _ in range(S)])
                         for _ in range(B)]).astype(np.int32) if keff > 0 else np.zeros((B, S, 0), np.int32)
    if minus_ones and keff > 0:
        comp_idx[..., -minus_ones:] = -1
    if repeat and keff > 1:
        comp_idx[..., 1] = comp_idx[..., 0]
    win_idx = orc.window_indices(B, S, start_pos, W, inp.R) if W > 0 else None
    return inp, win_idx, comp_idx


ATTN_CASES = [
    # B, S, start_pos, ratio, D, dv, W, k, extra
    (1, 1, 1023, 2, 128, 128, 128, 64, {}),
    (4, 1, 4095, 1, 128, 128, 128, 64, {}),
    (2, 1, 16383, 2, 192, 192, 128, 2048, {}),
    (2, 1, 16383, 2, 192, 128, 128, 300, {}),               # dv < D
    (1, 1, 600, 2, 256, 256, 128, 100, {"minus_ones": 7}),
    (2, 1, 4000, 2, 64, 64, 0, 77, {}),                     # compressed rows only
    (2, 1, 300, 2, 128, 128, 128, 0, {}),                   # window only (k = 0)
    (1, 200, 1000, 2, 128, 128, 128, 50, {}),               # many queries: one split each
    (1, 40, 0, 2, 128, 64, 16, 8, {"repeat": True}),        # prefill from 0, repeated rows
    (2, 1, 5000, 2, 128, 128, 128, 500, {"sink": "mixed"}),
    (3, 1, 2000, 2, 128, 128, 45, 333, {"minus_ones": 5}),  # 45 window rows padded to 64; 4 splits
]


@pytest.mark.parametrize("B,S,start_pos,ratio,D,dv,W,k,extra", ATTN_CASES)
def test_sparse_attn(orc, B, S, start_pos, ratio, D, dv, W, k, extra):
    extra = dict(extra)
    sink = None
    if extra.pop("sink", None) == "mixed":
        sink = np.linspace(-3.0, 6.0, 16).astype(np.float32)
    inp, win_idx, comp_idx = _attn_case(orc, B, S, start_pos, ratio, D, dv, W, k,
                                        seed=77 + B + S + D + k, sink=sink, **extra)
    d = step_inputs_dev(inp)
    got = L.lit_sparse_attn(d["q"], d["win_kv"] if W else None,
                            dev(win_idx) if win_idx is not None else None,
                            d["comp_kv"], dev(comp_idx) if comp_idx.shape[-1] else None,
                            d["sink"], inp.scale, dv=dv)
    torch.cuda.synchronize()
    want = orc.sparse_attn(inp.q, inp.win_kv, win_idx, inp.comp_kv,
                           comp_idx if comp_idx.shape[-1] else None, inp.sink, inp.scale, dv)
    err = np.abs(bf16_host(got) - want).max()
    assert err <= ATTN_TOL, err


def test_sparse_attn_empty_lists_and_huge_sink(orc):
    inp, win_idx, comp_idx = _attn_case(orc, 2, 3, 0, 2, 128, 128, 0, 4, seed=5)
    comp_idx[:] = -1
    d = step_inputs_dev(inp)
    got = L.lit_sparse_attn(d["q"], None, None, d["comp_kv"], dev(comp_idx), None, inp.scale)
    assert torch.count_nonzero(got.float()).item() == 0
    comp_idx[..., 0] = 0
    big = torch.full((16,), 1e4, dtype=torch.float32, device="cuda")
    got = L.lit_sparse_attn(d["q"], None, None, d["comp_kv"], dev(comp_idx), big, inp.scale)
    assert got.float().abs().max().item() == 0.0


# ---------------------------------------------------------------------------------
# the fused step
# ---------------------------------------------------------------------------------
def _run_step(d, inp, flags=0, state=None, expect_fused=None):
    args, idx, out = L.make_step_args(q8=d["q8"], q_sc=d["q_sc"], w=d["w"], k8=d["k8"],
                                      k_sc=d["k_sc"], q=d["q"], win_kv=d["win_kv"],
                                      comp_kv=d["comp_kv"], start_pos=inp.start_pos,
                                      ratio=inp.ratio, index_topk=inp.index_topk, W=inp.W,
                                      scale=inp.scale, dv=inp.dv, sink=d["sink"], flags=flags,
                                      fmt=inp.index_fmt, win_fmt=inp.win_kv_fmt, win_sc=d["win_sc"],
                                      comp_fmt=inp.comp_kv_fmt, comp_sc=d["comp_sc"])
    state = L.attach_state(args, state)
    if expect_fused is not None:
        assert (state is not None) == expect_fused, "fused form expected" if expect_fused else "kernels expected"
    ws = L.step_workspace(args)
    L.lit_sparse_step(args, ws)
    torch.cuda.synchronize()
    assert L.state_error(state) == 0, "fused step reported a team timeout"
    return idx, out


def _check_step(orc, inp, idx, out, queries=None):
    """Compare a step's outputs with the oracle, query by query (b, i).

    The top-k set must equal the oracle's up to near-ties (rows within 1e-3 relative of
    the oracle's k-th score).  Attention is then checked for every query on the list the
    GPU itself selected: the oracle attends over the same window rows and the GPU's rows,
    and the output must agree within ATTN_TOL.  Returns the number of queries whose set
    differed by near-ties."""
    d_idx = idx.cpu().numpy()
    d_out = bf16_host(out)
    queries = queries or [(b, i) for b in range(inp.B) for i in range(inp.S)]
    swaps = 0
    for (b, i) in queries:
        sub = _one_query(inp, b, i)
        ref = orc.step(sub)
        keff_i = ref["idx"].shape[-1]
        g_idx = d_idx[b, i]
        assert np.all(g_idx[keff_i:] == -1)
        ok, why = topk_sets_agree(ref["scores"][0, 0], ref["idx"][0, 0], g_idx[:keff_i])
        assert ok, f"query {(b, i)}: {why}"
        if set(ref["idx"][0, 0]) == set(g_idx[:keff_i]):
            want = ref["out"][0, 0]
        else:
            swaps += 1
            want = _attn_on_list(orc, sub, ref["win_idx"], g_idx[None, None, :keff_i])[0, 0]
        err = np.abs(d_out[b, i] - want).max()
        assert err <= ATTN_TOL, f"query {(b, i)}: attention err {err}"
    return swaps


def _attn_on_list(orc, inp, win_idx, comp_idx):
    """The oracle's attention of `inp`'s queries over its window rows and a given list of
    compressed rows (the GPU's own picks)."""
    return orc.sparse_attn(inp.q, inp.win_kv, win_idx, inp.comp_kv, comp_idx, inp.sink, inp.scale,
                           inp.dv, getattr(inp, "win_kv_fmt", "bf16"), getattr(inp, "win_sc", None),
                           getattr(inp, "comp_kv_fmt", "bf16"), getattr(inp, "comp_sc", None))


def _one_query(inp, b, i):
    """The same query as a single-query decode at its own position (the oracle then
    computes exactly that query's scores, picks and output)."""
    import dataclasses
    P = inp.start_pos + i
    sub = dataclasses.replace(
        inp, B=1, S=1, start_pos=P, q8=inp.q8[b:b + 1, i:i + 1], q_sc=inp.q_sc[b:b + 1, i:i + 1],
        w=inp.w[b:b + 1, i:i + 1], q=inp.q[b:b + 1, i:i + 1], k8=inp.k8[b:b + 1],
        k_sc=inp.k_sc[b:b + 1], win_kv=inp.win_kv[b:b + 1], comp_kv=inp.comp_kv[b:b + 1],
        win_sc=None if inp.win_sc is None else inp.win_sc[b:b + 1],
        comp_sc=None if inp.comp_sc is None else inp.comp_sc[b:b + 1])
    return sub


STEP_SMALL = [
    dict(B=2, S=1, start_pos=700, ratio=2, Hi=16, Di=64, H=16, D=128, W=128, index_topk=64),
    dict(B=1, S=50, start_pos=2000, ratio=2, Hi=16, Di=64, H=16, D=128, W=128, index_topk=100),
    dict(B=2, S=1, start_pos=3000, ratio=4, Hi=64, Di=128, H=16, D=192, W=128, index_topk=300),
    dict(B=1, S=1, start_pos=2, ratio=4, Hi=16, Di=64, H=16, D=128, W=128, index_topk=64),  # T = 0
    # one-member teams: the merge covers more output words than a workgroup has threads
    dict(B=1, S=1, start_pos=400, ratio=2, Hi=16, Di=64, H=16, D=128, W=128, index_topk=64),
    dict(B=2, S=1, start_pos=450, ratio=2, Hi=32, Di=128, H=16, D=256, W=64, index_topk=100),
    # twelve 8192-row queries (three sequences of four): teams of 32 members of 256 rows would
    # exceed the device's co-resident workgroups, so the fused plan takes 512-row chunks (each
    # wave scores two 64-key groups) -- ragged visibility across each sequence's queries
    dict(B=3, S=4, start_pos=16380, ratio=2, Hi=16, Di=64, H=16, D=128, W=128, index_topk=512),
    # k_eff = 64 of T = 65: three of each sequence's four queries see at most k rows (all
    # picked, the list padded with -1), the fourth needs a cut
    dict(B=2, S=4, start_pos=126, ratio=2, Hi=16, Di=64, H=16, D=128, W=128, index_topk=64),
]


MODES = [pytest.param(0, id="fused"), pytest.param(L.LIT_STEP_UNFUSED, id="kernels")]


@pytest.mark.parametrize("flags", MODES)
@pytest.mark.parametrize("cfg", STEP_SMALL, ids=lambda c: f"B{c['B']}S{c['S']}p{c['start_pos']}r{c['ratio']}")
def test_step_small(orc, cfg, flags):
    inp = synth.make_step(seed=4242 + cfg["start_pos"], **cfg)
    idx, out = _run_step(step_inputs_dev(inp), inp, flags, expect_fused=(flags == 0) if inp.T > 0 else None)
    _check_step(orc, inp, idx, out)


@pytest.mark.parametrize("flags", MODES)
@pytest.mark.parametrize("cfg", STEP_SMALL[:3] + STEP_SMALL[4:],
                         ids=lambda c: f"B{c['B']}S{c['S']}p{c['start_pos']}r{c['ratio']}")
def test_step_small_fp4(orc, cfg, flags):
    """The small steps with fp4 (e2m1) index queries and keys."""
    inp = synth.make_step(seed=5252 + cfg["start_pos"], index_fmt="e2m1", **cfg)
    idx, out = _run_step(step_inputs_dev(inp), inp, flags)
    _check_step(orc, inp, idx, out)


@pytest.mark.parametrize("flags", MODES)
@pytest.mark.parametrize("cfg", [STEP_SMALL[0], STEP_SMALL[2], STEP_SMALL[4], STEP_SMALL[5]],
                         ids=lambda c: f"B{c['B']}S{c['S']}p{c['start_pos']}r{c['ratio']}")
def test_step_small_qkv(orc, cfg, flags):
    """The small steps with quantised attention KV (window e4m3, compressed e2m1), fused
    and as kernels."""
    inp = synth.make_step(seed=6262 + cfg["start_pos"], kv_fmt="quant", **cfg)
    idx, out = _run_step(step_inputs_dev(inp), inp, flags)
    _check_step(orc, inp, idx, out)


@pytest.mark.parametrize("flags", MODES)
@pytest.mark.parametrize("name", ["decode-1k", "decode-4k-r2", "decode-4k-r1", "decode-16k",
                                  "decode-128k", "decode-16k-fp4", "decode-128k-fp4",
                                  "decode-16k-qkv"])
def test_step_workloads(orc, name, flags):
    inp = synth.workload(name)
    idx, out = _run_step(step_inputs_dev(inp), inp, flags)
    _check_step(orc, inp, idx, out)


def test_step_fused_with_sink_ties_and_dv(orc):
    """Fused path with a sink, dv < D and many equal index scores (integer-valued keys).
    Equal scores go to the lower row: the fused list equals the multi-kernel list and the
    oracle's selection over the GPU's own fp32 scores, bit for bit."""
    inp = synth.make_step(B=3, S=2, start_pos=1500, ratio=2, Hi=32, Di=64, H=16, D=128, dv=64,
                          W=64, index_topk=120, seed=77, sink=np.linspace(-2, 3, 16).astype(np.float32))
    inp.k8[:] = np.where(inp.k8 & 0x40, 0x38, 0xB8).astype(np.uint8)   # keys are +-1 (scaled)
    d = step_inputs_dev(inp)
    idx, out = _run_step(d, inp, 0)
    _check_step(orc, inp, idx, out)
    idx_k, _ = _run_step(d, inp, L.LIT_STEP_UNFUSED)
    assert torch.equal(idx, idx_k)
    sc = L.lit_indexer_scores(d["q8"], d["q_sc"], d["w"], d["k8"], d["k_sc"], inp.start_pos, inp.ratio)
    torch.cuda.synchronize()
    want = orc.topk(sc.cpu().numpy().astype(np.float64), inp.start_pos, inp.ratio, inp.index_topk)
    assert np.array_equal(idx.cpu().numpy(), want)


@pytest.mark.parametrize("name", ["decode-16k", "decode-4k-r1", "decode-128k"])
def test_step_duplicated_keys_exact(orc, name):
    """Key rows repeated many times (bit-identical scores on both sides) so that the cut
    falls inside a group of equal scores: the fused list must be the oracle's exactly
    (equal scores taken lowest row first)."""
    inp = synth.workload(name)
    rng = np.random.default_rng(11)
    full = orc.index_scores(inp.q8, inp.q_sc, inp.w, inp.k8, inp.k_sc, inp.start_pos, inp.ratio)
    for b in range(inp.B):
        # 24 rows whose scores lie at least 2e-3 apart (relative), each repeated at random
        keep = []
        for t in rng.permutation(inp.T):
            v = full[b, 0, t]
            if all(abs(v - full[b, 0, u]) > 2e-3 * max(abs(v), abs(full[b, 0, u])) for u in keep):
                keep.append(t)
            if len(keep) == 24:
                break
        src = rng.choice(np.array(keep), size=inp.T_cap)
        inp.k8[b] = inp.k8[b, src]
        inp.k_sc[b] = inp.k_sc[b, src]
    ref = orc.step(inp)
    d = step_inputs_dev(inp)
    idx, out = _run_step(d, inp, 0)
    got = idx.cpu().numpy()
    assert np.array_equal(got, ref["idx"]), np.argwhere(got != ref["idx"])[:5]
    err = np.abs(bf16_host(out) - ref["out"]).max()
    assert err <= ATTN_TOL, err
    idx_k, _ = _run_step(d, inp, L.LIT_STEP_UNFUSED)
    assert torch.equal(idx, idx_k)


def test_step_prefill_full(orc):
    """The 4096-query chunk at full size.  Attention of every query is checked on the
    GPU's own lists; the top-k sets of 256 queries (16 at each position of a 16-query
    indexer block, the first and last queries among them) against the oracle."""
    inp = synth.workload("prefill-16k")
    idx, out = _run_step(step_inputs_dev(inp), inp, 0)
    g_idx = idx.cpu().numpy()
    win = orc.window_indices(inp.B, inp.S, inp.start_pos, inp.W, inp.R)
    want = _attn_on_list(orc, inp, win, g_idx)
    err = np.abs(bf16_host(out) - want).max()
    assert err <= ATTN_TOL, err
    rng = np.random.default_rng(1)
    sample = {0, inp.S - 1}
    for r in range(16):
        sample |= set(int(x) for x in rng.choice(np.arange(r, inp.S, 16), 16, replace=False))
    for i in sorted(sample):
        sub = _one_query(inp, 0, i)
        scores = orc.index_scores(sub.q8, sub.q_sc, sub.w, sub.k8, sub.k_sc, sub.start_pos, sub.ratio)
        ref_idx = orc.topk(scores.astype(np.float32).astype(np.float64), sub.start_pos, sub.ratio,
                           sub.index_topk)
        keff_i = ref_idx.shape[-1]
        assert np.all(g_idx[0, i, keff_i:] == -1)
        ok, why = topk_sets_agree(scores[0, 0], ref_idx[0, 0], g_idx[0, i, :keff_i])
        assert ok, f"query {i}: {why}"


@pytest.mark.parametrize("flags", MODES)
def test_step_deterministic(flags):
    inp = synth.workload("decode-16k")
    d = step_inputs_dev(inp)
    i1, o1 = _run_step(d, inp, flags)
    i2, o2 = _run_step(d, inp, flags)
    assert torch.equal(i1, i2) and torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_step_fused_matches_kernels():
    """Same scores and selection rule: identical top-k lists; outputs within bf16 rounding
    of each other (the merge order differs)."""
    for name in ["decode-16k", "decode-128k", "decode-4k-r1"]:
        inp = synth.workload(name)
        d = step_inputs_dev(inp)
        i1, o1 = _run_step(d, inp, 0)
        i2, o2 = _run_step(d, inp, L.LIT_STEP_UNFUSED)
        assert torch.equal(i1, i2), name
        assert (o1.float() - o2.float()).abs().max().item() <= 1.6e-2, name


def test_step_fused_state_reuse():
    """One state buffer for calls of several shapes: every fused call leaves it
    consistent for the next (per-query launch counts, exchange words tagged with the
    query and its count), so repeated calls in any shape order give identical results
    and the error word stays clear."""
    state = torch.zeros(16 << 20, dtype=torch.uint8, device="cuda")
    outs = {}
    for rep in range(3):
        for name in ["decode-16k", "decode-1k", "decode-128k", "prefill-16k"]:
            if name == "prefill-16k" and rep == 2:
                continue
            inp = synth.workload(name)
            d = step_inputs_dev(inp)
            idx, out = _run_step(d, inp, 0, state=state)
            if rep == 0:
                outs[name] = (idx, out)
            else:
                assert torch.equal(outs[name][0], idx), name
                assert torch.equal(outs[name][1].view(torch.int16), out.view(torch.int16)), name
    assert L.state_error(state) == 0


@pytest.mark.parametrize("flags", MODES)
def test_step_graph_replays(flags):
    """The step captured in a HIP graph, replayed with eager work in between; every
    replay equals the eager result."""
    inp = synth.workload("decode-16k")
    d = step_inputs_dev(inp)
    ref_idx, ref_out = _run_step(d, inp, flags)
    args, idx, out = L.make_step_args(q8=d["q8"], q_sc=d["q_sc"], w=d["w"], k8=d["k8"],
                                      k_sc=d["k_sc"], q=d["q"], win_kv=d["win_kv"],
                                      comp_kv=d["comp_kv"], start_pos=inp.start_pos,
                                      ratio=inp.ratio, index_topk=inp.index_topk, W=inp.W,
                                      scale=inp.scale, flags=flags)
    state = L.attach_state(args)
    ws = L.step_workspace(args)
    L.lit_sparse_step(args, ws)          # warm once outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.lit_sparse_step(args, ws)
    for rep in range(4):
        idx.fill_(-7)
        out.zero_()
        _ = (torch.randn(1000, device="cuda") * 2).sum().item()   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx), rep
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), rep
        assert L.state_error(state) == 0


def test_step_matches_separate_calls():
    """The multi-kernel step and the three separate entry points give identical results."""
    inp = synth.workload("decode-4k-r2")
    d = step_inputs_dev(inp)
    idx, out = _run_step(d, inp, L.LIT_STEP_UNFUSED)
    sc = L.lit_indexer_scores(d["q8"], d["q_sc"], d["w"], d["k8"], d["k_sc"], inp.start_pos, inp.ratio)
    idx2 = L.lit_topk(sc, inp.start_pos, inp.ratio, inp.index_topk)
    win = L.lit_window_indices(inp.B, inp.S, inp.start_pos, inp.W, inp.R)
    out2 = L.lit_sparse_attn(d["q"], d["win_kv"], win, d["comp_kv"], idx2, None, inp.scale)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


# ---------------------------------------------------------------------------------
# two-level top-k: candidate blocks (level one) and the masked top-k (level two); both
# are integer results of identical fp32 scores, so they are compared bit-exactly
# ---------------------------------------------------------------------------------
CAND_CASES = [
    # B, S, start_pos, ratio, topk_blocks, block_size, ties
    (2, 1, 16383, 2, 256, 8, False),      # 1024 blocks, keep 256
    (2, 1, 131071, 4, 2048, 8, False),    # the released shape at 128K: 4096 blocks, keep 2048
    (1, 1, 1000, 1, 40, 7, False),        # ragged last block
    (3, 1, 4095, 2, 64, 8, True),         # many equal block scores
    (1, 300, 0, 2, 16, 4, False),         # prefill from 0: per-query visibility, short queries
    (1, 70, 900, 3, 20, 8, False),        # a chunk after cached tokens
    (2, 1, 500, 2, 4096, 8, False),       # more blocks asked than exist
]


def _visible_scores(B, S, start_pos, ratio, seed, ties):
    from lightning_indexer_top_amd import synth as sy
    T = (start_pos + S) // ratio
    s = sy.random_scores(B, S, T, seed=seed, ties=ties)
    for i in range(S):
        s[:, i, min(T, (start_pos + i + 1) // ratio):] = -np.inf
    ld = max(4, (T + 3) // 4 * 4)
    buf = np.full((B, S, ld), np.nan, dtype=np.float32)   # columns past T are never read
    buf[..., :T] = s
    return s.astype(np.float64), buf


@pytest.mark.parametrize("B,S,start_pos,ratio,kb,bs,ties", CAND_CASES)
def test_candidate_blocks_exact(orc, B, S, start_pos, ratio, kb, bs, ties):
    s, buf = _visible_scores(B, S, start_pos, ratio, 900 + S + kb, ties)
    got = L.lit_candidate_blocks(dev(buf), start_pos, ratio, kb, bs).cpu().numpy()
    want = orc.candidate_blocks(s, start_pos, ratio, kb, bs)
    assert got.shape == want.shape
    bad = np.argwhere((got != want).any(-1))
    assert bad.size == 0, f"first mismatch at {bad[0]}: {got[tuple(bad[0])][:12]} vs {want[tuple(bad[0])][:12]}"


@pytest.mark.parametrize("B,S,start_pos,ratio,kb,bs,ties", CAND_CASES)
def test_topk_candidates_exact(orc, B, S, start_pos, ratio, kb, bs, ties):
    s, buf = _visible_scores(B, S, start_pos, ratio, 1900 + S + kb, ties)
    # candidates from another layer's scores (level one of a source layer)
    s2, buf2 = _visible_scores(B, S, start_pos, ratio, 2900 + S + kb, ties)
    blocks = orc.candidate_blocks(s2, start_pos, ratio, kb, bs)
    k = max(1, min(kb * bs // 2, 600))
    got = L.lit_topk_candidates(dev(buf), start_pos, ratio, k, dev(blocks), bs).cpu().numpy()
    want = orc.topk(orc.apply_candidates(s, blocks, bs), start_pos, ratio, k)
    assert np.array_equal(got, want)


def test_topk_candidates_short_and_empty_lists(orc):
    """Fewer rows inside the blocks than k (the rest are the lowest rows outside), and an
    empty candidate list (every row masked: the lowest visible rows)."""
    s, buf = _visible_scores(2, 1, 4095, 2, 77, False)
    blocks = np.full((2, 1, 6), -1, dtype=np.int32)
    blocks[0, 0, :3] = [5, 40, 255]
    blocks[1, 0, :1] = [100]
    got = L.lit_topk_candidates(dev(buf), 4095, 2, 64, dev(blocks), 8).cpu().numpy()
    want = orc.topk(orc.apply_candidates(s, blocks, 8), 4095, 2, 64)
    assert np.array_equal(got, want)
    assert set(range(40, 48)) <= set(got[0, 0]) and set(range(800, 808)) <= set(got[1, 0])
    empty = torch.empty((2, 1, 0), dtype=torch.int32, device="cuda")
    got = L.lit_topk_candidates(dev(buf), 4095, 2, 64, empty, 8).cpu().numpy()
    assert (got == np.arange(64)).all()


@pytest.mark.parametrize("flags", MODES)
@pytest.mark.parametrize("fmt", FORMATS)
def test_step_two_level(orc, fmt, flags):
    """A candidate-source layer and a level-two layer of the 128K decode shape (at 32K
    context): the source's blocks come out of its step, the second layer's picks lie in
    them, and both layers match the oracle.  Both layers run fused or as kernels."""
    kw = dict(B=2, S=1, start_pos=32767, ratio=4, Hi=64, Di=128, H=16, D=128, W=128,
              index_topk=512, keys="mixture", index_fmt=fmt)
    src = synth.make_step(seed=61, **kw)
    lvl2 = synth.make_step(seed=62, **kw)
    ds, d2 = step_inputs_dev(src), step_inputs_dev(lvl2)
    kb = orc.candidate_blocks_width(1, 32767, 4, 256, 8)
    cand = torch.empty((2, 1, kb), dtype=torch.int32, device="cuda")
    a1, idx1, out1 = L.make_step_args(q8=ds["q8"], q_sc=ds["q_sc"], w=ds["w"], k8=ds["k8"],
                                      k_sc=ds["k_sc"], q=ds["q"], win_kv=ds["win_kv"],
                                      comp_kv=ds["comp_kv"], start_pos=src.start_pos,
                                      ratio=src.ratio, index_topk=src.index_topk, W=src.W,
                                      scale=src.scale, fmt=fmt, cand_out=cand,
                                      cand_topk_blocks=256, cand_block_size=8, flags=flags)
    st1 = L.attach_state(a1)
    assert (st1 is not None) == (flags == 0)
    L.lit_sparse_step(a1, L.step_workspace(a1))
    a2, idx2, out2 = L.make_step_args(q8=d2["q8"], q_sc=d2["q_sc"], w=d2["w"], k8=d2["k8"],
                                      k_sc=d2["k_sc"], q=d2["q"], win_kv=d2["win_kv"],
                                      comp_kv=d2["comp_kv"], start_pos=lvl2.start_pos,
                                      ratio=lvl2.ratio, index_topk=lvl2.index_topk, W=lvl2.W,
                                      scale=lvl2.scale, fmt=fmt, cand_in=cand, cand_block_size=8,
                                      flags=flags)
    st2 = L.attach_state(a2)
    assert (st2 is not None) == (flags == 0)
    L.lit_sparse_step(a2, L.step_workspace(a2))
    torch.cuda.synchronize()
    assert L.state_error(st1) == 0 and L.state_error(st2) == 0
    ref1 = orc.step(src, cand_topk_blocks=256, cand_block_size=8)
    g_cand = cand.cpu().numpy()
    # level one decides on the kernel's fp32 scores; near-equal block maxima may swap
    for b in range(2):
        bmax = ref1["scores"][b, 0].reshape(1024, 8).max(-1)
        bmax[-1] = np.inf                              # the newest block is pinned
        ok, why = topk_sets_agree(bmax, ref1["cand"][b, 0], g_cand[b, 0])
        assert ok, f"candidate blocks of sequence {b}: {why}"
        assert 1023 in g_cand[b, 0]
    _check_step(orc, src, idx1, out1)
    ref2 = orc.step(lvl2, cand_in=g_cand, cand_block_size=8)
    d_idx2, d_out2 = idx2.cpu().numpy(), bf16_host(out2)
    for b in range(2):
        assert set(d_idx2[b, 0] // 8) <= set(g_cand[b, 0])
        ok, why = topk_sets_agree(ref2["masked"][b, 0], ref2["idx"][b, 0], d_idx2[b, 0])
        assert ok, f"level-two picks of sequence {b}: {why}"
    want2 = _attn_on_list(orc, lvl2, ref2["win_idx"], d_idx2)
    assert np.abs(d_out2 - want2).max() <= ATTN_TOL


SRC_STEP_CASES = [
    # B, S, start_pos, ratio, Hi, Di, index_topk, topk_blocks, block_size, runs fused
    (2, 1, 32767, 4, 64, 128, 512, 256, 8, True),     # the 128K decode shape at 32K context
    (3, 1, 5001, 2, 32, 64, 256, 64, 16, True),       # 2501 rows: a short last block
    (2, 1, 700, 4, 16, 64, 256, 512, 8, True),        # every row picked; more blocks asked than exist
    (2, 3, 9001, 2, 64, 128, 512, 128, 4, True),      # three queries per sequence
    (2, 1, 8191, 2, 64, 128, 512, 256, 3, False),     # blocks of 3 do not divide the chunks
]


@pytest.mark.parametrize("B,S,start_pos,ratio,Hi,Di,topk,kb,bs,fused", SRC_STEP_CASES)
def test_candidate_source_step_exact(orc, B, S, start_pos, ratio, Hi, Di, topk, kb, bs, fused):
    """A candidate-source step, fused where its blocks divide the members' score chunks.
    Its block list is the oracle's level one over the GPU's own fp32 scores, exactly (the
    fused kernel scores a decode query with the indexer kernel's arithmetic); its top-k
    equals the kernels form's, and both forms meet the oracle's step rules."""
    inp = synth.make_step(B=B, S=S, start_pos=start_pos, ratio=ratio, Hi=Hi, Di=Di, H=16, D=128,
                          W=128, index_topk=topk, seed=500 + S + start_pos % 97)
    d = step_inputs_dev(inp)
    nb = orc.candidate_blocks_width(S, start_pos, ratio, kb, bs)
    got = {}
    for flags in (0, L.LIT_STEP_UNFUSED):
        cand = torch.full((B, S, nb), -7, dtype=torch.int32, device="cuda")
        a, idx, out = L.make_step_args(q8=d["q8"], q_sc=d["q_sc"], w=d["w"], k8=d["k8"],
                                       k_sc=d["k_sc"], q=d["q"], win_kv=d["win_kv"],
                                       comp_kv=d["comp_kv"], start_pos=start_pos, ratio=ratio,
                                       index_topk=topk, W=inp.W, scale=inp.scale, fmt=inp.index_fmt,
                                       cand_out=cand, cand_topk_blocks=kb, cand_block_size=bs,
                                       flags=flags)
        st = L.attach_state(a)
        assert (st is not None) == (flags == 0 and fused)
        L.lit_sparse_step(a, L.step_workspace(a))
        torch.cuda.synchronize()
        assert L.state_error(st) == 0
        _check_step(orc, inp, idx, out)
        got[flags] = (cand.cpu().numpy(), idx)
    sc = L.lit_indexer_scores(d["q8"], d["q_sc"], d["w"], d["k8"], d["k_sc"], start_pos, ratio,
                              fmt=inp.index_fmt).cpu().numpy().astype(np.float64)
    for i in range(S):
        sc[:, i, min(inp.T, (start_pos + i + 1) // ratio):] = -np.inf
    want = orc.candidate_blocks(sc, start_pos, ratio, kb, bs)
    for flags, (cand, _) in got.items():
        bad = np.argwhere((cand != want).any(-1))
        assert bad.size == 0, (flags, bad[:3], cand[tuple(bad[0])][:12], want[tuple(bad[0])][:12])
    assert torch.equal(got[0][1], got[L.LIT_STEP_UNFUSED][1])


@pytest.mark.parametrize("flags", MODES)
def test_step_level_two_short_candidate_list(orc, flags):
    """Fewer rows inside the candidate blocks than k: the remaining picks are the lowest
    rows outside them (all at -inf), in both step forms; a second sequence lists one block
    twice and one out of range."""
    inp = synth.make_step(B=2, S=1, start_pos=4095, ratio=2, Hi=16, Di=64, H=16, D=128, W=128,
                          index_topk=64, seed=73)
    d = step_inputs_dev(inp)
    blocks = np.array([[[3, 17, 200, 255]], [[9, 9, 4000, -1]]], dtype=np.int32)
    cand = dev(blocks)
    args, idx, out = L.make_step_args(q8=d["q8"], q_sc=d["q_sc"], w=d["w"], k8=d["k8"],
                                      k_sc=d["k_sc"], q=d["q"], win_kv=d["win_kv"],
                                      comp_kv=d["comp_kv"], start_pos=inp.start_pos,
                                      ratio=inp.ratio, index_topk=inp.index_topk, W=inp.W,
                                      scale=inp.scale, cand_in=cand, cand_block_size=8,
                                      flags=flags)
    state = L.attach_state(args)
    L.lit_sparse_step(args, L.step_workspace(args))
    torch.cuda.synchronize()
    assert L.state_error(state) == 0
    ref = orc.step(inp, cand_in=blocks, cand_block_size=8)
    got = idx.cpu().numpy()
    assert np.array_equal(got, ref["idx"]), (got[:, 0, :40], ref["idx"][:, 0, :40])
    err = np.abs(bf16_host(out) - ref["out"]).max()
    assert err <= ATTN_TOL, err


# ---------------------------------------------------------------------------------
# cross-layer reuse: several layers over one shared list and compressed KV
# ---------------------------------------------------------------------------------
LAYER_CASES = [
    # layers, B, S, start_pos, D, dv, W, K, derived window, sink
    (2, 2, 1, 4095, 128, 128, 128, 64, True, False),
    (3, 8, 1, 16383, 192, 192, 128, 2048, True, True),   # decode-16k's attention shape
    (4, 1, 5, 300, 64, 32, 16, 40, False, True),         # explicit lists, dv < D, chunk
    (1, 2, 1, 1023, 256, 256, 128, 64, True, False),
]


@pytest.mark.parametrize("NL,B,S,start_pos,D,dv,W,K,derived,with_sink", LAYER_CASES)
def test_sparse_attn_layers(orc, NL, B, S, start_pos, D, dv, W, K, derived, with_sink):
    rng = np.random.default_rng(4000 + NL * 10 + D)
    R = max(1, S if start_pos == 0 else W + S - 1)
    T = (start_pos + S) // 2
    bits = lambda shape: synth.to_bf16_bits(rng.standard_normal(shape).astype(np.float32))  # noqa: E731
    q, win_kv, comp_kv = bits((NL, B, S, 16, D)), bits((NL, B, R, D)), bits((B, T, D))
    comp_idx = np.sort(rng.choice(T, size=(B, S, K), replace=True), axis=-1).astype(np.int32)
    comp_idx[:, :, -3:] = -1
    sink = rng.standard_normal((NL, 16)).astype(np.float32) if with_sink else None
    win_idx = orc.window_indices(B, S, start_pos, W, R)
    scale = D ** -0.5
    out = L.lit_sparse_attn_layers(bf16_dev(q), bf16_dev(win_kv), None if derived else dev(win_idx),
                                    bf16_dev(comp_kv), dev(comp_idx),
                                    None if sink is None else dev(sink), scale, dv=dv,
                                    window=W, start_pos=start_pos)
    torch.cuda.synchronize()
    got = bf16_host(out)
    want = orc.sparse_attn_layers(q, win_kv, win_idx, comp_kv, comp_idx, sink, scale, dv)
    err = np.abs(got - want).max()
    assert err <= ATTN_TOL, f"max err {err}"
    # layer l alone through lit_sparse_attn agrees to the same bar
    one = L.lit_sparse_attn(bf16_dev(q[-1]), bf16_dev(win_kv[-1]), dev(win_idx), bf16_dev(comp_kv),
                             dev(comp_idx), None if sink is None else dev(sink[-1]), scale, dv=dv)
    assert np.abs(bf16_host(one) - got[-1]).max() <= ATTN_TOL



# ---------------------------------------------------------------------------------
# quantised attention KV (window e4m3 / ue8m0-32, compressed e2m1 / e4m3-16)
# ---------------------------------------------------------------------------------
QKV_CASES = [
    # B, S, start_pos, D, dv, W, K, window format, compressed format
    (2, 1, 16383, 192, 192, 128, 2048, "e4m3", "e2m1"),
    (1, 70, 0, 128, 128, 128, 30, "e4m3", "e2m1"),      # 70 window rows: padded tiles
    (2, 3, 500, 64, 32, 40, 50, "e4m3", "bf16"),
    (2, 1, 4095, 256, 256, 128, 64, "bf16", "e2m1"),
]


@pytest.mark.parametrize("B,S,start_pos,D,dv,W,K,wf,cf", QKV_CASES)
def test_sparse_attn_quantised_kv(orc, B, S, start_pos, D, dv, W, K, wf, cf):
    inp = synth.make_step(B=B, S=S, start_pos=start_pos, ratio=2, Hi=16, Di=64, H=16, D=D, dv=dv,
                          W=W, index_topk=K, seed=6000 + D + S, kv_fmt="quant",
                          sink=np.linspace(-3, 1, 16).astype(np.float32))
    rng = np.random.default_rng(D + S)
    win = orc.window_indices(B, S, start_pos, W, inp.R)
    idx = rng.integers(-1, inp.T_cap, size=(B, S, K)).astype(np.int32)
    wkv, wsc = (inp.win_kv, inp.win_sc)
    ckv, csc = (inp.comp_kv, inp.comp_sc)
    if wf == "bf16":  # the same rows, decoded, as bf16
        from tests.test_oracle_attention import _exact_bf16_bits, _lib_rows_e4m3
        wkv, wsc = _exact_bf16_bits(_lib_rows_e4m3(inp.win_kv, inp.win_sc)), None
    if cf == "bf16":
        from tests.test_oracle_attention import _exact_bf16_bits, _table_rows_e2m1
        ckv, csc = _exact_bf16_bits(_table_rows_e2m1(inp.comp_kv, inp.comp_sc)), None
    to = lambda a, f: bf16_dev(a) if f == "bf16" else dev(a)  # noqa: E731
    got = L.lit_sparse_attn_fmt(bf16_dev(inp.q), to(wkv, wf), dev(win), to(ckv, cf), dev(idx),
                                dev(inp.sink), inp.scale, dv=dv, win_fmt=wf,
                                win_sc=None if wsc is None else dev(wsc), comp_fmt=cf,
                                comp_sc=None if csc is None else dev(csc))
    torch.cuda.synchronize()
    want = orc.sparse_attn(inp.q, wkv, win, ckv, idx, inp.sink, inp.scale, dv, wf, wsc, cf, csc)
    err = np.abs(bf16_host(got) - want).max()
    assert err <= ATTN_TOL, f"max err {err}"



# ---------------------------------------------------------------------------------
# producer side: the cache writes of decode steps and chunks (compressor pooling, norm,
# rotation, quantised rows).  The window rows and every cache row computed from a given
# latent are exact; the latents themselves may differ from the oracle's only by one bf16 step
# at a rounding midpoint (the pages' fp32 pooling and norm are not bit-reproducible across exp
# and rsqrt implementations and summation orders).
# ---------------------------------------------------------------------------------
def _dequant_fp4_rows(codes, scales):
    from tests.test_oracle_attention import _table_rows_e2m1
    return _table_rows_e2m1(codes, scales)  # codes x e4m3 scale per 16, exact


def _bf16_flip_possible(raw, rel=3e-5):
    """True where a value lies within `rel` (relative; broadcast) of a bf16 rounding
    midpoint: there fp32 arithmetic in another order or with another exp / rsqrt may round
    the other way."""
    raw = np.asarray(raw, np.float64)
    lo = torch.from_numpy(raw * (1 - rel)).to(torch.bfloat16).to(torch.float64).numpy()
    hi = torch.from_numpy(raw * (1 + rel)).to(torch.bfloat16).to(torch.float64).numpy()
    return lo != hi


def _pool_magnitude(kv, score, ratio):
    """Per pooled value, the sum of softmax(score)_r |kv_r| over the group's slots (kv,
    score [..., ratio, D]): the scale of the fp32 rounding error of the pooling, which
    cancellation can make far larger than the result itself."""
    g = np.asarray(score, np.float64)
    p = np.exp(g - g.max(axis=-2, keepdims=True))
    return (p / p.sum(axis=-2, keepdims=True) * np.abs(np.asarray(kv, np.float64))).sum(axis=-2)


def _check_latents(lat_g, lat_o, pooled_raw, norm_raw, pool_mag):
    """The GPU's bf16 latents against the oracle's.  The pages pool and normalise in fp32
    (the oracle: exactly, then bf16).  A latent may differ from the oracle's only where the
    exact pooled value lies within fp32 noise of a bf16 rounding midpoint (16 fp32 ulps of
    its group's magnitude, pool_mag; None: no pooling) -- by up to two bf16 steps -- or
    where the exact normalised value does -- by one step; the latter within 3e-5 (relative)
    plus what the pooled values of its row that may round the other way can move the row's
    norm (each by one bf16 step: the sum of squares by at most 2 x^2 2^-7 per such value)."""
    diff = lat_g != lat_o
    if not diff.any():
        return 0
    pooled_raw = np.asarray(pooled_raw, np.float64)
    bf = lambda v: torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()  # noqa: E731
    if pool_mag is None:
        near_pool = np.zeros(pooled_raw.shape, bool)
    else:
        tol = 16 * 2.0 ** -24 * np.asarray(pool_mag, np.float64)
        near_pool = bf(pooled_raw - tol) != bf(pooled_raw + tol)
    x = bf(pooled_raw)
    ss = (x * x).sum(-1, keepdims=True)
    dss = (2.0 * x * x * 2.0 ** -7 * near_pool).sum(-1, keepdims=True)
    rel = 3e-5 + 0.6 * dss / np.maximum(ss, 1e-300)
    # a pooled value one step off moves its latent by about one step, which may then round
    # one step further: two steps there, one elsewhere
    steps = np.abs(lat_g - lat_o) / np.maximum(2.0 ** -7 * np.abs(lat_o), 1e-300)
    ok = (near_pool & (steps <= 2.0001)) | (_bf16_flip_possible(norm_raw, rel) & (steps <= 1.0001))
    bad = diff & ~ok
    assert not bad.any(), (f"{int(bad.sum())} latent(s) differ away from a rounding midpoint: "
                           f"norm {np.asarray(norm_raw)[bad][:4]}, pooled {pooled_raw[bad][:4]}, "
                           f"gpu {lat_g[bad][:4]}, oracle {lat_o[bad][:4]}")
    return int(diff.sum())


def _check_rows_from_latents(orc, lat_g, codes_g, scales_g, freqs, rd, positions):
    """Rotation and quantisation of the GPU's own latents (the oracle's fp32 reading of the
    rotation): the GPU's cache rows must match exactly."""
    for b in range(lat_g.shape[0]):
        for j, pos in enumerate(positions):
            c, s = orc.compress_write(lat_g[b, j], freqs, rd, pos)
            assert np.array_equal(codes_g[b, j], c) and np.array_equal(scales_g[b, j], s), (b, j, pos)


@pytest.mark.parametrize("ratio,D,rd,B", [(4, 192, 64, 3), (2, 128, 32, 2), (1, 64, 16, 2),
                                          (4, 256, 64, 1)])
def test_compress_append_steps(orc, ratio, D, rd, B):
    """Decode steps of the compressor: state exact; latents per _check_latents; every cache
    row equal to the oracle's rotation and quantisation of the GPU's latent."""
    steps = 3 * ratio + 1
    a = synth.make_append(B=B, D=D, rd=rd, ratio=ratio, steps=steps, positions=64, seed=70 + D)
    T_cap = steps // ratio + 1
    ks = np.zeros((B, ratio, D), np.float32)
    gs = np.full((B, ratio, D), -np.inf, np.float32)
    oc = np.zeros((B, T_cap, D // 2), np.uint8)
    osc = np.zeros((B, T_cap, D // 16), np.uint8)
    dks, dgs = dev(ks.copy()), dev(gs.copy())
    dc, dsc = dev(oc.copy()), dev(osc.copy())
    dw, dfr = dev(a.norm_w), dev(a.freqs)
    lat = torch.zeros((B, D), dtype=torch.bfloat16, device="cuda")
    for t in range(steps):
        w_o, lat_o, pr, nr = orc.compress_append(a.kv[t], a.score[t], ks if ratio > 1 else None,
                                                 gs if ratio > 1 else None, a.norm_w, a.eps, a.freqs, rd,
                                                 oc, osc, t, ratio, raw=True)
        w_g = L.lit_compress_append(dev(a.kv[t]), dev(a.score[t]), dks if ratio > 1 else None,
                                    dgs if ratio > 1 else None, dw, a.eps, dfr, rd, dc, dsc, t,
                                    ratio, latent=lat)
        torch.cuda.synchronize()
        assert w_g == w_o
        if ratio > 1:
            assert np.array_equal(dks.cpu().numpy(), ks) and np.array_equal(dgs.cpu().numpy(), gs)
        if w_o:
            lg = bf16_host(lat)
            grp = slice(t + 1 - ratio, t + 1)
            mag = _pool_magnitude(a.kv[grp].transpose(1, 0, 2), a.score[grp].transpose(1, 0, 2), ratio) \
                if ratio > 1 else None
            _check_latents(lg, lat_o, pr, nr, mag)
            row = t // ratio
            _check_rows_from_latents(orc, lg[:, None], dc.cpu().numpy()[:, row:row + 1],
                                     dsc.cpu().numpy()[:, row:row + 1], a.freqs, rd, [t + 1 - ratio])


def test_window_append_steps(orc):
    """Decode-step window writes: codes and scales equal the oracle's exactly (the rotation
    in the pages' fp32, the quantiser's decisions exact)."""
    B, D, rd, R = 3, 192, 64, 128
    a = synth.make_append(B=B, D=D, rd=rd, ratio=1, steps=5, positions=300, seed=81)
    oc = np.zeros((B, R, D), np.uint8)
    osc = np.zeros((B, R, D // 32), np.uint8)
    dc, dsc, dfr = dev(oc.copy()), dev(osc.copy()), dev(a.freqs)
    for t, pos in enumerate([0, 1, 127, 128, 290]):
        orc.window_append(a.win[t], a.freqs, rd, oc, osc, pos)
        L.lit_window_append(bf16_dev(a.win[t]), dfr, rd, dc, dsc, pos)
    torch.cuda.synchronize()
    assert np.array_equal(dsc.cpu().numpy(), osc)
    assert np.array_equal(dc.cpu().numpy(), oc)


@pytest.mark.parametrize("ratio,S,start_pos,D,rd,B", [
    (4, 4096, 0, 128, 64, 1),    # a prefill chunk of whole groups
    (4, 1030, 0, 192, 64, 2),    # remainder 2 left in the state
    (2, 301, 0, 128, 32, 2),     # odd chunk at ratio 2
    (4, 37, 6, 128, 64, 2),      # a chunk starting inside a group (slots 0-1 from the state)
    (4, 3, 5, 64, 16, 2),        # no group completes: every token to the state
    (1, 90, 17, 64, 16, 2),      # ratio 1: a row per token
])
def test_compress_chunk(orc, ratio, S, start_pos, D, rd, B):
    """A chunk into the compressor (lit_compress_chunk) against the oracle's chunk (the S
    decode steps): rows written, the state exactly, latents per _check_latents, cache rows
    exactly from the GPU's latents.  Earlier tokens (start_pos > 0) are fed first through
    the same chunk call on both sides."""
    a = synth.make_append(B=B, D=D, rd=rd, ratio=ratio, steps=start_pos + S, positions=start_pos + S + 1,
                          seed=120 + S)
    kv, sc = a.kv.transpose(1, 0, 2).copy(), a.score.transpose(1, 0, 2).copy()
    T_cap = (start_pos + S) // ratio + 1
    ks = np.zeros((B, ratio, D), np.float32)
    gs = np.full((B, ratio, D), -np.inf, np.float32)
    oc = np.zeros((B, T_cap, D // 2), np.uint8)
    osc = np.zeros((B, T_cap, D // 16), np.uint8)
    dks, dgs = dev(ks.copy()), dev(gs.copy())
    dc, dsc = dev(oc.copy()), dev(osc.copy())
    dw, dfr = dev(a.norm_w), dev(a.freqs)
    if start_pos > 0:  # the tokens before the chunk, on both sides
        orc.compress_chunk(kv[:, :start_pos], sc[:, :start_pos], ks, gs, a.norm_w, a.eps, a.freqs, rd, oc, osc, 0,
                           ratio)
        L.lit_compress_chunk(dev(kv[:, :start_pos]), dev(sc[:, :start_pos]), dks if ratio > 1 else None,
                             dgs if ratio > 1 else None, dw, a.eps, dfr, rd, dc, dsc, 0, ratio)
        torch.cuda.synchronize()
        if ratio > 1:
            assert np.array_equal(dks.cpu().numpy(), ks) and np.array_equal(dgs.cpu().numpy(), gs)
        dc.copy_(torch.from_numpy(oc).cuda())    # continue from the oracle's rows (compared below)
        dsc.copy_(torch.from_numpy(osc).cuda())
    n_o, lat_o, pr, nr = orc.compress_chunk(kv[:, start_pos:], sc[:, start_pos:], ks, gs, a.norm_w, a.eps,
                                            a.freqs, rd, oc, osc, start_pos, ratio)
    lat = torch.zeros((B, max(n_o, 1), D), dtype=torch.bfloat16, device="cuda")
    n_g = L.lit_compress_chunk(dev(kv[:, start_pos:]), dev(sc[:, start_pos:]), dks if ratio > 1 else None,
                               dgs if ratio > 1 else None, dw, a.eps, dfr, rd, dc, dsc, start_pos, ratio,
                               latent=lat)
    torch.cuda.synchronize()
    assert n_g == n_o == (start_pos + S) // ratio - start_pos // ratio
    if ratio > 1:
        assert np.array_equal(dks.cpu().numpy(), ks) and np.array_equal(dgs.cpu().numpy(), gs)
    if n_o == 0:
        assert np.array_equal(dc.cpu().numpy(), oc)
        return
    lg = bf16_host(lat)[:, :n_o]
    r0 = start_pos // ratio
    mag = None
    if ratio > 1:
        pos = (r0 + np.arange(n_o))[:, None] * ratio + np.arange(ratio)[None, :]   # [rows, ratio]
        mag = _pool_magnitude(kv[:, pos], sc[:, pos], ratio)
    _check_latents(lg, lat_o, pr, nr, mag)
    _check_rows_from_latents(orc, lg, dc.cpu().numpy()[:, r0:r0 + n_o], dsc.cpu().numpy()[:, r0:r0 + n_o],
                             a.freqs, rd, [(r0 + j) * ratio for j in range(n_o)])


@pytest.mark.parametrize("S,start_pos,R", [(4096, 0, 128), (100, 0, 128), (300, 12288, 4223), (257, 40, 64)])
def test_window_chunk(orc, S, start_pos, R):
    """A chunk's window rows into the ring (lit_window_chunk) against the oracle's S
    decode-step writes: codes and scales exactly, untouched slots unchanged."""
    B, D, rd = 2, 128, 64
    a = synth.make_append(B=B, D=D, rd=rd, ratio=1, steps=S, positions=start_pos + S + 1, seed=S + R)
    win_bits = a.win.transpose(1, 0, 2).copy()
    rng = np.random.default_rng(5)
    oc = rng.integers(0, 256, size=(B, R, D), dtype=np.uint8)   # stale ring contents
    osc = rng.integers(0, 256, size=(B, R, D // 32), dtype=np.uint8)
    dc, dsc, dfr = dev(oc.copy()), dev(osc.copy()), dev(a.freqs)
    orc.window_chunk(win_bits, a.freqs, rd, oc, osc, start_pos)
    L.lit_window_chunk(bf16_dev(win_bits), dfr, rd, dc, dsc, start_pos)
    torch.cuda.synchronize()
    assert np.array_equal(dsc.cpu().numpy(), osc)
    assert np.array_equal(dc.cpu().numpy(), oc)


# ---------------------------------------------------------------------------------
# the fused kernel's re-reading selection form (more than 8192 visible rows) with level-two
# masking and with quantised KV
# ---------------------------------------------------------------------------------
def test_step_level_two_rereading_form(orc):
    """16384 rows per query (the re-reading form) as a level-two layer, fused, against
    the oracle; the candidates keep 1024 of 2048 blocks."""
    kw = dict(B=2, S=1, start_pos=65535, ratio=4, Hi=64, Di=128, H=16, D=128, W=128,
              index_topk=1024, keys="mixture")
    src = synth.make_step(seed=91, **kw)
    inp = synth.make_step(seed=92, **kw)
    ref_src = orc.step(src, cand_topk_blocks=1024, cand_block_size=8)
    blocks = ref_src["cand"]
    d = step_inputs_dev(inp)
    args, idx, out = L.make_step_args(q8=d["q8"], q_sc=d["q_sc"], w=d["w"], k8=d["k8"],
                                      k_sc=d["k_sc"], q=d["q"], win_kv=d["win_kv"],
                                      comp_kv=d["comp_kv"], start_pos=inp.start_pos,
                                      ratio=inp.ratio, index_topk=inp.index_topk, W=inp.W,
                                      scale=inp.scale, cand_in=dev(blocks), cand_block_size=8)
    state = L.attach_state(args)
    assert state is not None, "expected the fused form"
    L.lit_sparse_step(args, L.step_workspace(args))
    torch.cuda.synchronize()
    assert L.state_error(state) == 0
    ref = orc.step(inp, cand_in=blocks, cand_block_size=8)
    g_idx, g_out = idx.cpu().numpy(), bf16_host(out)
    for b in range(2):
        assert set(g_idx[b, 0] // 8) <= set(blocks[b, 0])
        ok, why = topk_sets_agree(ref["masked"][b, 0], ref["idx"][b, 0], g_idx[b, 0])
        assert ok, f"sequence {b}: {why}"
    want = _attn_on_list(orc, inp, ref["win_idx"], g_idx)
    assert np.abs(g_out - want).max() <= ATTN_TOL


@pytest.mark.parametrize("fmt", FORMATS)
def test_step_qkv_rereading_form(orc, fmt):
    """Quantised attention KV with 16384 rows per query (the re-reading selection form),
    fused, against the oracle."""
    inp = synth.make_step(B=2, S=1, start_pos=65535, ratio=4, Hi=64, Di=128, H=16, D=128, W=128,
                          index_topk=1024, seed=93, kv_fmt="quant", index_fmt=fmt)
    d = step_inputs_dev(inp)
    args, idx, out = L.make_step_args(q8=d["q8"], q_sc=d["q_sc"], w=d["w"], k8=d["k8"],
                                      k_sc=d["k_sc"], q=d["q"], win_kv=d["win_kv"],
                                      comp_kv=d["comp_kv"], start_pos=inp.start_pos,
                                      ratio=inp.ratio, index_topk=inp.index_topk, W=inp.W,
                                      scale=inp.scale, fmt=fmt, win_fmt="e4m3", win_sc=d["win_sc"],
                                      comp_fmt="e2m1", comp_sc=d["comp_sc"])
    state = L.attach_state(args)
    assert state is not None, "expected the fused form"
    L.lit_sparse_step(args, L.step_workspace(args))
    torch.cuda.synchronize()
    assert L.state_error(state) == 0
    _check_step(orc, inp, idx, out)


# ---------------------------------------------------------------------------------
# layers sharing one top-k inside the step (fused: one launch for every layer)
# ---------------------------------------------------------------------------------
@pytest.mark.parametrize("flags", MODES)
@pytest.mark.parametrize("kv", ["bf16", "quant"])
def test_step_shared_topk_layers(orc, flags, kv):
    NL = 3
    inp = synth.make_step(B=2, S=1, start_pos=4095, ratio=2, Hi=32, Di=128, H=16, D=192, W=128,
                          index_topk=512, seed=95, kv_fmt=kv,
                          sink=np.linspace(-1, 2, 16).astype(np.float32))
    rng = np.random.default_rng(96)
    bits = lambda shape: synth.to_bf16_bits(rng.standard_normal(shape).astype(np.float32))  # noqa: E731
    qs = np.concatenate([inp.q[None], bits((NL - 1,) + inp.q.shape)])
    sinks = np.stack([inp.sink] + [rng.standard_normal(16).astype(np.float32) for _ in range(NL - 1)])
    if kv == "quant":
        wq = [synth._quant_np(rng.standard_normal(inp.win_kv.shape).astype(np.float32), "e4m3")
              for _ in range(NL - 1)]
        wins = np.concatenate([inp.win_kv[None]] + [w[0][None] for w in wq])
        win_sc = np.concatenate([inp.win_sc[None]] + [w[1][None] for w in wq])
    else:
        wins = np.concatenate([inp.win_kv[None], bits((NL - 1,) + inp.win_kv.shape)])
        win_sc = None
    d = step_inputs_dev(inp)
    q_dev = bf16_dev(qs)
    win_dev = bf16_dev(wins) if kv == "bf16" else dev(wins)
    args, idx, out = L.make_step_args(q8=d["q8"], q_sc=d["q_sc"], w=d["w"], k8=d["k8"],
                                      k_sc=d["k_sc"], q=q_dev, win_kv=win_dev, comp_kv=d["comp_kv"],
                                      start_pos=inp.start_pos, ratio=inp.ratio,
                                      index_topk=inp.index_topk, W=inp.W, scale=inp.scale,
                                      sink=dev(sinks), flags=flags,
                                      win_fmt="e4m3" if kv == "quant" else "bf16",
                                      win_sc=None if win_sc is None else dev(win_sc),
                                      comp_fmt="e2m1" if kv == "quant" else "bf16",
                                      comp_sc=d["comp_sc"])
    state = L.attach_state(args)
    assert (state is not None) == (flags == 0)
    L.lit_sparse_step(args, L.step_workspace(args))
    torch.cuda.synchronize()
    assert L.state_error(state) == 0
    assert out.shape == (NL, 2, 1, 16, 192)
    g_idx, g_out = idx.cpu().numpy(), bf16_host(out)
    ref = orc.step(inp)
    win = orc.window_indices(inp.B, inp.S, inp.start_pos, inp.W, inp.R)
    for b in range(2):
        ok, why = topk_sets_agree(ref["scores"][b, 0], ref["idx"][b, 0], g_idx[b, 0])
        assert ok, why
    wf, cf = ("e4m3", "e2m1") if kv == "quant" else ("bf16", "bf16")
    for ly in range(NL):  # every layer over the kernel's own list
        want = orc.sparse_attn(qs[ly], wins[ly], win, inp.comp_kv, g_idx, sinks[ly], inp.scale, None,
                               wf, None if win_sc is None else win_sc[ly], cf, inp.comp_sc)
        err = np.abs(g_out[ly] - want).max()
        assert err <= ATTN_TOL, f"layer {ly}: {err}"


# ---------------------------------------------------------------------------------
# the fused kernel's combined forms: level two with quantised KV and / or several layers
# ---------------------------------------------------------------------------------
@pytest.mark.parametrize("flags", MODES)
@pytest.mark.parametrize("kv,NL,start_pos", [("quant", 1, 16383), ("bf16", 3, 16383), ("quant", 3, 16383),
                                             ("quant", 1, 65535), ("quant", 2, 65535)])
def test_step_level_two_combined_forms(orc, kv, NL, start_pos, flags):
    """A level-two layer (candidate blocks of a source layer) with quantised KV, several
    layers over its top-k, or both: one fused launch (the cached selection at 4096 rows,
    the re-reading one at 16384) or kernels, against the oracle on every layer."""
    kw = dict(B=2, S=1, start_pos=start_pos, ratio=4, Hi=64, Di=128, H=16, D=128, W=128,
              index_topk=512, keys="mixture")
    nblk = (start_pos + 1) // 4 // 8
    src = synth.make_step(seed=101, **kw)
    inp = synth.make_step(seed=102, kv_fmt=kv, sink=np.linspace(-1, 1, 16).astype(np.float32), **kw)
    blocks = orc.step(src, cand_topk_blocks=nblk // 4, cand_block_size=8)["cand"]
    rng = np.random.default_rng(103)
    bits = lambda shape: synth.to_bf16_bits(rng.standard_normal(shape).astype(np.float32))  # noqa: E731
    qs = np.concatenate([inp.q[None], bits((NL - 1,) + inp.q.shape)])
    sinks = np.stack([inp.sink] + [rng.standard_normal(16).astype(np.float32) for _ in range(NL - 1)])
    if kv == "quant":
        wq = [synth._quant_np(rng.standard_normal(inp.win_kv.shape).astype(np.float32), "e4m3")
              for _ in range(NL - 1)]
        wins = np.concatenate([inp.win_kv[None]] + [w[0][None] for w in wq])
        win_sc = np.concatenate([inp.win_sc[None]] + [w[1][None] for w in wq])
    else:
        wins = np.concatenate([inp.win_kv[None], bits((NL - 1,) + inp.win_kv.shape)])
        win_sc = None
    d = step_inputs_dev(inp)
    args, idx, out = L.make_step_args(q8=d["q8"], q_sc=d["q_sc"], w=d["w"], k8=d["k8"],
                                      k_sc=d["k_sc"], q=bf16_dev(qs) if NL > 1 else d["q"],
                                      win_kv=(bf16_dev(wins) if kv == "bf16" else dev(wins)) if NL > 1
                                      else d["win_kv"],
                                      comp_kv=d["comp_kv"], start_pos=inp.start_pos, ratio=inp.ratio,
                                      index_topk=inp.index_topk, W=inp.W, scale=inp.scale,
                                      sink=dev(sinks) if NL > 1 else d["sink"], flags=flags,
                                      win_fmt="e4m3" if kv == "quant" else "bf16",
                                      win_sc=None if win_sc is None else dev(win_sc),
                                      comp_fmt="e2m1" if kv == "quant" else "bf16",
                                      comp_sc=d["comp_sc"], cand_in=dev(blocks), cand_block_size=8)
    state = L.attach_state(args)
    assert (state is not None) == (flags == 0), "expected the fused form"
    L.lit_sparse_step(args, L.step_workspace(args))
    torch.cuda.synchronize()
    assert L.state_error(state) == 0
    g_idx = idx.cpu().numpy()
    g_out = bf16_host(out).reshape((NL,) + inp.q.shape[:3] + (inp.q.shape[3],))
    ref = orc.step(inp, cand_in=blocks, cand_block_size=8)
    for b in range(2):
        assert set(g_idx[b, 0] // 8) <= set(blocks[b, 0])
        ok, why = topk_sets_agree(ref["masked"][b, 0], ref["idx"][b, 0], g_idx[b, 0])
        assert ok, f"sequence {b}: {why}"
    wf, cf = ("e4m3", "e2m1") if kv == "quant" else ("bf16", "bf16")
    for ly in range(NL):  # every layer over the kernel's own list
        want = orc.sparse_attn(qs[ly], wins[ly], ref["win_idx"], inp.comp_kv, g_idx, sinks[ly], inp.scale,
                               None, wf, None if win_sc is None else win_sc[ly], cf, inp.comp_sc)
        err = np.abs(g_out[ly] - want).max()
        assert err <= ATTN_TOL, f"layer {ly}: {err}"


# ---------------------------------------------------------------------------------
# chunked prefill steps (16 index heads of 64 e4m3 dims): exact against the separate calls
# ---------------------------------------------------------------------------------
PS_CASES = [
    # B, S, start_pos, ratio, k, keys, oracle sample (None: every query)
    (1, 4096, 12288, 2, 512, "normal", 24),   # prefill-16k's shape
    (2, 301, 0, 2, 64, "normal", None),       # from position 0 (early rows: fewer than k), ragged S
    (1, 1030, 7000, 4, 300, "mixture", 64),   # clustered scores: several narrowing levels
    (1, 64, 8128, 1, 2048, "normal", 16),     # T = 8192 rows at ratio 1, large k
    (2, 96, 4000, 2, 128, "dup", None),       # every key row twice: exactly equal scores
    (1, 40, 2000, 2, 64, "const", None),      # one key for every row: all scores equal
]


@pytest.mark.parametrize("B,S,start_pos,ratio,k,keys,sample", PS_CASES)
def test_prefill_step_exact(orc, B, S, start_pos, ratio, k, keys, sample):
    """Chunked-prefill steps: the step's picks equal lit_indexer_scores followed by lit_topk
    bit for bit (equal scores lowest row first: duplicated and constant keys), and match the
    oracle (sets up to near-ties, attention on the GPU's own lists)."""
    inp = synth.make_step(B=B, S=S, start_pos=start_pos, ratio=ratio, Hi=16, Di=64, H=16, D=128, W=128,
                          index_topk=k, seed=110 + S, keys="mixture" if keys == "mixture" else "normal")
    if keys == "dup":
        n_odd = inp.k8[:, 1::2].shape[1]
        inp.k8[:, 1::2] = inp.k8[:, 0::2][:, :n_odd]
        inp.k_sc[:, 1::2] = inp.k_sc[:, 0::2][:, :n_odd]
    elif keys == "const":
        inp.k8[:] = inp.k8[:, :1]
        inp.k_sc[:] = inp.k_sc[:, :1]
    d = step_inputs_dev(inp)
    idx, out = _run_step(d, inp, L.LIT_STEP_UNFUSED)
    sc = L.lit_indexer_scores(d["q8"], d["q_sc"], d["w"], d["k8"], d["k_sc"], inp.start_pos, inp.ratio)
    idx2 = L.lit_topk(sc, inp.start_pos, inp.ratio, inp.index_topk)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2), torch.nonzero(idx != idx2)[:5].tolist()
    queries = [(b, i) for b in range(B) for i in range(S)]
    if sample is not None:
        rng = np.random.default_rng(7)
        pick = rng.choice(len(queries), size=sample, replace=False)
        queries = sorted({queries[j] for j in pick} | {queries[0], queries[-1]})
    _check_step(orc, inp, idx, out, queries)
