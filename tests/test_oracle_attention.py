"""Pins for the oracle's sparse attention.

Definition: DeepSeek-V4.1-Flash-NVFP4 model.py, Attention.forward (sparse_attn over the
window KV and the compressed KV, one shared row as key and value, an attention sink
per head); DeepSeek-V3.2-Exp model.py, MLA.forward (dense scores, -inf outside the
index set, softmax, weighted values).

Pins:
* index set = every compressed row, no window, no sink: torch's
  scaled_dot_product_attention in float64 (library routine);
* arbitrary sets over both sources with dv < D: the dense masked softmax form of the
  V3.2 page evaluated with torch.softmax over the concatenated KV (library routine);
* a single row gives that row (closed form); q = 0 with a sink gives
  sum(rows) / (n + e^sink) (closed form); sink = -inf is no sink; a huge sink gives 0;
* invariance under reordering of the list, under a permutation of the KV rows, and
  under listing every row twice; an empty set gives 0.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from lightning_indexer_top_amd import synth


def bf(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(torch.float64)


def rand_case(B=2, S=3, H=4, D=64, R=10, T=24, seed=0):
    rng = np.random.default_rng(seed)
    q = synth.to_bf16_bits(rng.standard_normal((B, S, H, D)))
    win = synth.to_bf16_bits(rng.standard_normal((B, R, D)))
    comp = synth.to_bf16_bits(rng.standard_normal((B, T, D)))
    return q, win, comp


def test_all_rows_equals_library_sdpa(orc):
    B, S, H, D, T = 2, 3, 4, 64, 24
    q, _, comp = rand_case(B, S, H, D, 1, T, seed=1)
    idx = np.broadcast_to(np.arange(T, dtype=np.int32), (B, S, T)).copy()
    scale = D ** -0.5
    got = orc.sparse_attn(q, None, None, comp, idx, None, scale)
    qt = bf(q).reshape(B * S, H, 1, D)
    kv = bf(comp).unsqueeze(1).expand(B, S, T, D).reshape(B * S, 1, T, D).expand(B * S, H, T, D)
    want = F.scaled_dot_product_attention(qt, kv, kv, scale=scale).reshape(B, S, H, D)
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-12)


def test_dense_masked_softmax_two_sources(orc):
    B, S, H, D, dv, R, T, W, K = 2, 3, 4, 64, 48, 10, 24, 5, 7
    q, win, comp = rand_case(B, S, H, D, R, T, seed=2)
    rng = np.random.default_rng(3)
    win_idx = np.full((B, S, W), -1, np.int32)
    comp_idx = np.full((B, S, K), -1, np.int32)
    for b in range(B):
        for i in range(S):
            ws = rng.choice(R, size=W - 1 - i % 2, replace=False)
            win_idx[b, i, :len(ws)] = ws
            cs = rng.choice(T, size=K - i, replace=False)
            comp_idx[b, i, :len(cs)] = np.sort(cs)
    scale = 0.125
    got = orc.sparse_attn(q, win, win_idx, comp, comp_idx, None, scale, dv)
    kv = torch.cat([bf(win), bf(comp)], dim=1)           # [B, R+T, D]
    for b in range(B):
        for i in range(S):
            mask = torch.full((R + T,), -math.inf, dtype=torch.float64)
            for s in win_idx[b, i]:
                if s >= 0:
                    mask[s] = 0
            for t in comp_idx[b, i]:
                if t >= 0:
                    mask[R + t] = 0
            scores = bf(q)[b, i] @ kv[b].T * scale + mask   # [H, R+T]
            want = torch.softmax(scores, dim=-1) @ kv[b, :, :dv]
            np.testing.assert_allclose(got[b, i], want.numpy(), rtol=1e-12, atol=1e-12)


def test_single_row_and_empty_set(orc):
    q, win, comp = rand_case(seed=4)
    idx = np.full((2, 3, 3), -1, np.int32)
    idx[:, :, 1] = 7
    got = orc.sparse_attn(q, None, None, comp, idx, None, 0.3, 32)
    for b in range(2):
        for i in range(3):
            for h in range(4):
                assert np.array_equal(got[b, i, h], bf(comp)[b, 7, :32].numpy())
    empty = np.full((2, 3, 4), -1, np.int32)
    got = orc.sparse_attn(q, win, empty, comp, empty, None, 0.3)
    assert np.array_equal(got, np.zeros_like(got))
    sink = np.zeros(4, np.float32)
    got = orc.sparse_attn(q, win, empty, comp, empty, sink, 0.3)
    assert np.array_equal(got, np.zeros_like(got))


def test_sink_closed_forms(orc):
    B, S, H, D, T = 1, 2, 4, 64, 9
    _, _, comp = rand_case(B, S, H, D, 1, T, seed=5)
    q0 = np.zeros((B, S, H, D), np.uint16)                # all logits 0
    idx = np.broadcast_to(np.arange(T, dtype=np.int32), (B, S, T)).copy()
    sink = np.array([0.0, 1.5, -2.0, 4.0], np.float32)
    got = orc.sparse_attn(q0, None, None, comp, idx, sink, 0.5)
    rows = bf(comp)[0].numpy()
    for h in range(H):
        want = rows.sum(0) / (T + math.exp(float(sink[h])))
        np.testing.assert_allclose(got[0, 0, h], want, rtol=1e-13, atol=1e-14)
    q, _, _ = rand_case(B, S, H, D, 1, T, seed=6)
    none = orc.sparse_attn(q, None, None, comp, idx, None, 0.2)
    ninf = orc.sparse_attn(q, None, None, comp, idx, np.full(H, -np.inf, np.float32), 0.2)
    assert np.array_equal(none, ninf)
    huge = orc.sparse_attn(q, None, None, comp, idx, np.full(H, 1e4, np.float32), 0.2)
    assert np.abs(huge).max() < 1e-300


def test_order_permutation_and_duplication_invariance(orc):
    B, S, H, D, R, T, W, K = 1, 2, 4, 64, 8, 30, 8, 10
    q, win, comp = rand_case(B, S, H, D, R, T, seed=7)
    rng = np.random.default_rng(8)
    win_idx = np.broadcast_to(np.arange(W, dtype=np.int32), (B, S, W)).copy()
    comp_idx = np.stack([np.sort(rng.choice(T, K, replace=False)) for _ in range(S)])[None].astype(np.int32)
    base = orc.sparse_attn(q, win, win_idx, comp, comp_idx, None, 0.15)
    # list order
    shuf = comp_idx[..., rng.permutation(K)]
    np.testing.assert_allclose(orc.sparse_attn(q, win, win_idx[..., ::-1], comp, shuf, None, 0.15),
                               base, rtol=1e-13, atol=1e-14)
    # KV row permutation with the index lists remapped
    perm = rng.permutation(T)
    inv = np.argsort(perm)
    comp_p = comp[:, perm]
    np.testing.assert_allclose(orc.sparse_attn(q, win, win_idx, comp_p, inv[comp_idx].astype(np.int32),
                                               None, 0.15), base, rtol=1e-13, atol=1e-14)
    # every row listed twice
    dup = np.concatenate([comp_idx, comp_idx], -1)
    wdup = np.concatenate([win_idx, win_idx], -1)
    np.testing.assert_allclose(orc.sparse_attn(q, win, wdup, comp, dup, None, 0.15),
                               base, rtol=1e-13, atol=1e-14)


def test_refuses_out_of_range_rows(orc):
    q, win, comp = rand_case(seed=9)
    bad = np.full((2, 3, 2), 24, np.int32)
    with pytest.raises(orc.OracleError):
        orc.sparse_attn(q, None, None, comp, bad, None, 0.1)


def test_layers_are_independent_single_layer_calls(orc):
    """The multi-layer form is the single-layer attention per layer over the shared lists
    (cross-layer reuse shares the lists and compressed KV, nothing else)."""
    rng = np.random.default_rng(8)
    L, B, S, H, D, R, T = 3, 2, 1, 16, 64, 8, 20
    bits = lambda shape: synth.to_bf16_bits(rng.standard_normal(shape).astype(np.float32))  # noqa: E731
    q, win_kv, comp_kv = bits((L, B, S, H, D)), bits((L, B, R, D)), bits((B, T, D))
    win_idx = np.tile(np.arange(R, dtype=np.int32), (B, S, 1))
    comp_idx = rng.integers(0, T, size=(B, S, 5)).astype(np.int32)
    sink = rng.standard_normal((L, H)).astype(np.float32)
    out = orc.sparse_attn_layers(q, win_kv, win_idx, comp_kv, comp_idx, sink, 0.125)
    assert out.shape == (L, B, S, H, D)
    for l in range(L):
        one = orc.sparse_attn(q[l], win_kv[l], win_idx, comp_kv, comp_idx, sink[l], 0.125)
        assert np.array_equal(out[l], one)
    # swapping two layers' inputs swaps their outputs
    sw = orc.sparse_attn_layers(q[[1, 0, 2]], win_kv[[1, 0, 2]], win_idx, comp_kv, comp_idx,
                                sink[[1, 0, 2]], 0.125)
    assert np.array_equal(sw, out[[1, 0, 2]])


# -- quantised KV sources: DeepSeek-V4.1-Flash-NVFP4 model.py, Attention._window_kv
# (e4m3, ue8m0 per 32) and Attention._compress_kv (fp4 e2m1, e4m3 scales per 16) ---------

def _lib_rows_e4m3(codes, scales):
    c = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64)
    s = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e8m0fnu).to(torch.float64)
    return (c.unflatten(-1, (-1, 32)) * s.unsqueeze(-1)).flatten(-2).numpy()


def _table_rows_e2m1(packed, scales):
    from tests.test_oracle_formats import E2M1_TABLE
    p = np.ascontiguousarray(packed)
    lut = np.array(E2M1_TABLE + [-v for v in E2M1_TABLE])
    vals = np.stack([lut[p & 15], lut[p >> 4]], axis=-1).reshape(*p.shape[:-1], 2 * p.shape[-1])
    s = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return (vals.reshape(*vals.shape[:-1], -1, 16) * s[..., None]).reshape(vals.shape)


def _exact_bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    b = t.to(torch.bfloat16)
    assert torch.equal(b.to(torch.float64), t), "decoded KV value not exact in bf16"
    return b.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("D", [64, 192])
def test_quantised_kv_equals_library_decoded_rows(orc, D):
    """Rows decoded by torch's fp8 casts (window) and the MX e2m1 table with torch's e4m3
    cast (compressed) are exact in bf16; the bf16 attention over them is bit-identical to
    the oracle's quantised-source attention."""
    inp = synth.make_step(B=2, S=3, start_pos=200, ratio=2, Hi=16, Di=64, H=16, D=D, W=40,
                          index_topk=30, seed=31 + D, kv_fmt="quant",
                          sink=np.linspace(-1, 1, 16).astype(np.float32))
    assert inp.win_kv.shape[-1] == D and inp.comp_kv.shape[-1] == D // 2
    win = orc.window_indices(inp.B, inp.S, inp.start_pos, inp.W, inp.R)
    rng = np.random.default_rng(D)
    idx = rng.integers(-1, inp.T_cap, size=(inp.B, inp.S, 30)).astype(np.int32)
    got = orc.sparse_attn(inp.q, inp.win_kv, win, inp.comp_kv, idx, inp.sink, inp.scale, D,
                          "e4m3", inp.win_sc, "e2m1", inp.comp_sc)
    wb = _exact_bf16_bits(_lib_rows_e4m3(inp.win_kv, inp.win_sc))
    cb = _exact_bf16_bits(_table_rows_e2m1(inp.comp_kv, inp.comp_sc))
    want = orc.sparse_attn(inp.q, wb, win, cb, idx, inp.sink, inp.scale, D)
    assert np.array_equal(got, want)
    # one source quantised, the other bf16
    mixed = orc.sparse_attn(inp.q, wb, win, inp.comp_kv, idx, inp.sink, inp.scale, D,
                            "bf16", None, "e2m1", inp.comp_sc)
    assert np.array_equal(mixed, want)
