"""Pins for the oracle's indexer score and visibility rule.

Definition (DeepSeek-V4.1-Flash-NVFP4 model.py, Indexer.forward; DeepSeek-V3.2-Exp
model.py, fp8_index): score[t] = sum_h w_h * relu(qhat_h . khat_t) over block-scaled
e4m3 operands, and rows a query cannot see yet are -inf.

Pins, none of which re-runs the oracle's own loops:
* a closed form with constant codes and distinct per-block scales (catches a dropped
  scale, a block/scale index mix-up, a missing ReLU or a head-weight mix-up);
* one-hot head weights reduce the score to relu of a library matmul of operands
  decoded by torch's fp8 casts;
* relu(x) - relu(-x) = x turns s(q) - s(-q) into a plain linear form (catches a wrong
  ReLU sign);
* exact linearity in w and equivariance under key-row permutation;
* the visibility counts of the pages' prefill and decode forms.
"""
import numpy as np
import pytest
import torch

from lightning_indexer_top_amd import synth


def lib_dequant(codes, scales):
    c = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64)
    s = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e8m0fnu).to(torch.float64)
    return (c.unflatten(-1, (-1, 32)) * s.unsqueeze(-1)).flatten(-2).numpy()


def test_closed_form_constant_blocks(orc):
    Hi, Di, T = 4, 128, 3
    q_codes = [0x38, 0x40, 0xB8, 0x44]          # 1, 2, -1, 3
    q_vals = [1.0, 2.0, -1.0, 3.0]
    k_codes = [0x38, 0x30, 0x3C]                # 1, 0.5, 1.5
    k_vals = [1.0, 0.5, 1.5]
    a = np.array([[127, 128, 125, 130], [120, 127, 131, 126],
                  [129, 129, 127, 124], [126, 122, 128, 133]], dtype=np.uint8)
    b = np.array([[127, 126, 130, 121], [132, 127, 127, 127], [125, 129, 122, 128]],
                 dtype=np.uint8)
    w = np.array([0.5, 0.25, 1.0, 0.125], dtype=np.float32)
    q8 = np.array(q_codes, dtype=np.uint8)[:, None].repeat(Di, 1).reshape(1, 1, Hi, Di)
    k8 = np.array(k_codes, dtype=np.uint8)[:, None].repeat(Di, 1).reshape(1, T, Di)
    got = orc.index_scores(q8, a.reshape(1, 1, Hi, 4), w.reshape(1, 1, Hi), k8,
                           b.reshape(1, T, 4), start_pos=T - 1, ratio=1)
    want = np.zeros(T)
    for t in range(T):
        for h in range(Hi):
            dot = 32 * q_vals[h] * k_vals[t] * sum(
                2.0 ** ((int(a[h, c]) - 127) + (int(b[t, c]) - 127)) for c in range(4))
            want[t] += float(w[h]) * max(0.0, dot)
    assert np.array_equal(got[0, 0], want)


@pytest.mark.parametrize("Di", [64, 128])
def test_one_hot_weights_reduce_to_library_matmul(orc, Di):
    inp = synth.make_step(B=2, S=1, start_pos=39, ratio=2, Hi=16, Di=Di, H=16, D=64, W=8,
                          index_topk=8, seed=11 + Di)
    qd = lib_dequant(inp.q8, inp.q_sc)          # [B,1,Hi,Di]
    kd = lib_dequant(inp.k8, inp.k_sc)          # [B,T,Di]
    for h in (0, 5, 15):
        w = np.zeros_like(inp.w)
        w[..., h] = 1.0
        got = orc.index_scores(inp.q8, inp.q_sc, w, inp.k8, inp.k_sc, inp.start_pos, inp.ratio)
        for bb in range(inp.B):
            want = np.maximum(kd[bb] @ qd[bb, 0, h], 0.0)
            np.testing.assert_allclose(got[bb, 0], want, rtol=1e-12, atol=1e-12)


def test_relu_identity_gives_linear_form(orc):
    inp = synth.make_step(B=1, S=3, start_pos=60, ratio=4, Hi=32, Di=128, H=16, D=64, W=8,
                          index_topk=8, seed=5)
    neg = inp.q8 ^ np.uint8(0x80)               # exact negation of every e4m3 code
    sp = orc.index_scores(inp.q8, inp.q_sc, inp.w, inp.k8, inp.k_sc, inp.start_pos, inp.ratio)
    sn = orc.index_scores(neg, inp.q_sc, inp.w, inp.k8, inp.k_sc, inp.start_pos, inp.ratio)
    qd = lib_dequant(inp.q8, inp.q_sc)[0]       # [S,Hi,Di]
    kd = lib_dequant(inp.k8, inp.k_sc)[0]       # [T,Di]
    lin = np.einsum("sh,shd->sd", inp.w[0].astype(np.float64), qd) @ kd.T
    for i in range(inp.S):
        nvis = (inp.start_pos + i + 1) // inp.ratio
        diff = sp[0, i, :nvis] - sn[0, i, :nvis]
        scale = np.abs(lin[i, :nvis]).max()
        np.testing.assert_allclose(diff, lin[i, :nvis], rtol=0, atol=1e-12 * scale)


def test_linear_in_weights_and_permutation_equivariant(orc):
    inp = synth.make_step(B=1, S=1, start_pos=63, ratio=1, Hi=16, Di=64, H=16, D=64, W=8,
                          index_topk=8, seed=3)
    s = orc.index_scores(inp.q8, inp.q_sc, inp.w, inp.k8, inp.k_sc, inp.start_pos, 1)
    s2 = orc.index_scores(inp.q8, inp.q_sc, inp.w * 2, inp.k8, inp.k_sc, inp.start_pos, 1)
    assert np.array_equal(s2, 2 * s)
    perm = np.random.default_rng(0).permutation(inp.T_cap)
    sp = orc.index_scores(inp.q8, inp.q_sc, inp.w, inp.k8[:, perm], inp.k_sc[:, perm],
                          inp.start_pos, 1)
    assert np.array_equal(sp[0, 0], s[0, 0, perm])


def test_visibility_prefill_decode_and_chunk(orc):
    # prefill from position 0: the pages' count arange(1, S+1) // ratio
    S, r = 9, 2
    assert [orc.n_visible(0, i, r) for i in range(S)] == list(np.arange(1, S + 1) // r)
    # decode: one query, end_pos // ratio
    assert orc.n_visible(1023, 0, 2) == 1024 // 2
    assert orc.n_visible(131071, 0, 4) == 32768
    # a chunk appended to cached tokens: 4096 queries after 12288 tokens, ratio 2
    counts = [orc.n_visible(12288, i, 2) for i in range(4096)]
    assert counts[0] == 6144 and counts[-1] == 8192 and sum(counts) == 29360128
    inp = synth.make_step(B=1, S=S, start_pos=0, ratio=r, Hi=16, Di=64, H=16, D=64, W=8,
                          index_topk=8, seed=9, T_cap=S // r)
    s = orc.index_scores(inp.q8, inp.q_sc, inp.w, inp.k8, inp.k_sc, 0, r)
    assert s.shape == (1, S, S // r)
    for i in range(S):
        nv = (i + 1) // r
        assert np.all(np.isneginf(s[0, i, nv:]))
        assert np.all(np.isfinite(s[0, i, :nv]))


def test_refuses_bad_sizes(orc):
    inp = synth.make_step(B=1, S=1, start_pos=15, ratio=1, Hi=16, Di=64, H=16, D=64, W=8,
                          index_topk=8, seed=1)
    with pytest.raises(orc.OracleError):
        # T = 16 visible rows but a cache of only 8
        orc.index_scores(inp.q8, inp.q_sc, inp.w, inp.k8[:, :8], inp.k_sc[:, :8], 15, 1)


# -- fp4 (e2m1) index codes: DeepSeek-V4.1-Flash-NVFP4 model.py, Indexer.forward
# quantises queries and keys to fp4 with one ue8m0 scale per 32 elements --------------

from tests.test_oracle_formats import E2M1_TABLE  # noqa: E402


def fp4_table_decode(packed, scales):
    """Test-local decoder: table lookup of both nibbles (element 2j low), then the
    block scale from torch's e8m0 cast."""
    p = np.asarray(packed, dtype=np.uint8)
    lut = np.array(E2M1_TABLE + [-v for v in E2M1_TABLE])
    vals = np.stack([lut[p & 15], lut[p >> 4]], axis=-1).reshape(*p.shape[:-1], 2 * p.shape[-1])
    s = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e8m0fnu)
    s = s.to(torch.float64).numpy()
    return (vals.reshape(*vals.shape[:-1], -1, 32) * s[..., None]).reshape(vals.shape)


def fp4_table_encode(codes):
    """Pack 4-bit codes [..., Di] two per byte (element 2j in the low nibble)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


@pytest.mark.parametrize("Di", [64, 128])
def test_fp4_one_hot_weights_reduce_to_library_matmul(orc, Di):
    inp = synth.make_step(B=2, S=1, start_pos=39, ratio=2, Hi=16, Di=Di, H=16, D=64, W=8,
                          index_topk=8, seed=21 + Di, index_fmt="e2m1")
    assert inp.q8.shape[-1] == Di // 2 and inp.k8.shape[-1] == Di // 2
    qd = fp4_table_decode(inp.q8, inp.q_sc)     # [B,1,Hi,Di]
    kd = fp4_table_decode(inp.k8, inp.k_sc)     # [B,T,Di]
    for h in (0, 7, 15):
        w = np.zeros_like(inp.w)
        w[..., h] = 1.0
        got = orc.index_scores(inp.q8, inp.q_sc, w, inp.k8, inp.k_sc, inp.start_pos, inp.ratio,
                               "e2m1")
        for bb in range(inp.B):
            want = np.maximum((torch.from_numpy(kd[bb]) @ torch.from_numpy(qd[bb, 0, h])).numpy(), 0.0)
            np.testing.assert_allclose(got[bb, 0], want, rtol=1e-12, atol=1e-12)


def test_fp4_closed_form_constant_blocks(orc):
    # constant codes per head / key, a distinct scale per (row, block): the closed form
    # needs every element matched with its own block's scale
    Hi, Di, T = 4, 128, 3
    q_codes, q_vals = [2, 4, 10, 5], [1.0, 2.0, -1.0, 3.0]
    k_codes, k_vals = [2, 1, 3], [1.0, 0.5, 1.5]
    a = np.array([[127, 128, 125, 130], [120, 127, 131, 126],
                  [129, 129, 127, 124], [126, 122, 128, 133]], dtype=np.uint8)
    b = np.array([[127, 126, 130, 121], [132, 127, 127, 127], [125, 129, 122, 128]],
                 dtype=np.uint8)
    w = np.array([0.5, 0.25, 1.0, 0.125], dtype=np.float32)
    q4 = fp4_table_encode(np.array(q_codes)[:, None].repeat(Di, 1)).reshape(1, 1, Hi, Di // 2)
    k4 = fp4_table_encode(np.array(k_codes)[:, None].repeat(Di, 1)).reshape(1, T, Di // 2)
    got = orc.index_scores(q4, a.reshape(1, 1, Hi, 4), w.reshape(1, 1, Hi), k4,
                           b.reshape(1, T, 4), start_pos=T - 1, ratio=1, fmt="e2m1")
    want = np.zeros(T)
    for t in range(T):
        for h in range(Hi):
            dot = 32 * q_vals[h] * k_vals[t] * sum(
                2.0 ** ((int(a[h, c]) - 127) + (int(b[t, c]) - 127)) for c in range(4))
            want[t] += float(w[h]) * max(0.0, dot)
    assert np.array_equal(got[0, 0], want)


def test_fp4_equals_e4m3_on_shared_values(orc):
    # the same values written as fp4 codes and as e4m3 bytes (torch's cast) give
    # bit-identical scores: the two formats differ only in how codes are stored
    rng = np.random.default_rng(17)
    B, S, Hi, Di, T = 2, 3, 32, 128, 40
    start_pos = T - S
    qc = rng.integers(0, 16, size=(B, S, Hi, Di))
    kc = rng.integers(0, 16, size=(B, T, Di))
    q_sc = rng.integers(120, 135, size=(B, S, Hi, Di // 32)).astype(np.uint8)
    k_sc = rng.integers(120, 135, size=(B, T, Di // 32)).astype(np.uint8)
    w = rng.random((B, S, Hi), dtype=np.float32)
    lut = np.array(E2M1_TABLE + [-v for v in E2M1_TABLE])

    def e4m3(codes):
        return torch.from_numpy(lut[codes]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    s4 = orc.index_scores(fp4_table_encode(qc), q_sc, w, fp4_table_encode(kc), k_sc,
                          start_pos, 1, "e2m1")
    s8 = orc.index_scores(e4m3(qc), q_sc, w, e4m3(kc), k_sc, start_pos, 1, "e4m3")
    assert np.array_equal(s4, s8)
    assert np.isfinite(s4[:, -1]).all()


def test_fp4_nibble_order_does_not_change_scores(orc):
    # both nibbles of a byte share one scale block, so swapping them in q and k alike
    # permutes the terms of every dot product and leaves each score as it is
    inp = synth.make_step(B=1, S=2, start_pos=30, ratio=1, Hi=16, Di=64, H=16, D=64, W=8,
                          index_topk=8, seed=23, index_fmt="e2m1")
    swap = lambda p: ((p >> 4) | (p << 4)).astype(np.uint8)  # noqa: E731
    s = orc.index_scores(inp.q8, inp.q_sc, inp.w, inp.k8, inp.k_sc, 30, 1, "e2m1")
    t = orc.index_scores(swap(inp.q8), inp.q_sc, inp.w, swap(inp.k8), inp.k_sc, 30, 1, "e2m1")
    np.testing.assert_allclose(t, s, rtol=1e-13, atol=0)


def test_fp4_refuses_mismatched_rows(orc):
    inp = synth.make_step(B=1, S=1, start_pos=15, ratio=1, Hi=16, Di=64, H=16, D=64, W=8,
                          index_topk=8, seed=1)
    with pytest.raises(orc.OracleError):
        # e4m3 rows (Di bytes) passed as fp4 (Di/2 bytes expected)
        orc.index_scores(inp.q8, inp.q_sc, inp.w, inp.k8, inp.k_sc, 15, 1, "e2m1")
