"""Pins for the oracle's producer side: the cache writes of one decode step
(DeepSeek-V4.1-Flash-NVFP4 model.py: Compressor.forward, RMSNorm.forward,
apply_rotary_emb, Attention._compress_kv and _window_kv with their quantisers).

Pins: the bf16 rounding and the e4m3 encoder against torch's casts; both block
quantisers against brute force over every code (smallest admissible scale, nearest code,
ties to the even code); the compressor's group timing, softmax pooling (equal scores give
the mean, a dominant score gives its slot), the RMSNorm closed form for a constant row;
the rotation at angle 0 (identity) and a quarter turn; the window slot ring.
"""
import numpy as np
import pytest
import torch

from lightning_indexer_top_amd import synth
from tests.test_oracle_formats import E2M1_TABLE


def test_round_bf16_matches_torch(orc):
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(4000) * np.exp(rng.uniform(-20, 20, 4000))).astype(np.float32)
    # exact ties: bf16 value plus half an ulp
    b = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    ulp = np.abs(b) * 2.0 ** -7
    ties = (b + 0.5 * ulp * np.where(rng.random(4000) < 0.5, 1, -1)).astype(np.float32)
    for v in np.concatenate([x, ties]):
        want = float(torch.tensor(float(v), dtype=torch.float32).to(torch.bfloat16).to(torch.float64))
        assert orc.round_bf16(float(v)) == want, v


def test_e4m3_encoder_matches_torch(orc):
    rng = np.random.default_rng(1)
    vals = np.concatenate([rng.uniform(-448, 448, 3000), rng.uniform(-2 ** -5, 2 ** -5, 2000)])
    grid = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    fin = np.sort(np.unique(grid[np.isfinite(grid)]))
    mids = ((fin[1:] + fin[:-1]) / 2)                  # exact ties between neighbours
    vals = np.concatenate([vals, mids, -mids]).astype(np.float32)
    lib = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([orc.e4m3_encode(float(v)) for v in vals], dtype=np.uint8)
    nz = vals != 0
    assert np.array_equal(ours[nz], lib[nz])


def _brute_e4m3_block(x):
    amax = np.abs(x).max()
    e = -127
    if amax > 0:
        e = next(k for k in range(-140, 140) if amax <= 448.0 * 2.0 ** k)
    grid = torch.arange(128, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    codes = []
    for v in x / 2.0 ** e:
        d = np.abs(np.abs(v) - grid[:127])
        best = np.flatnonzero(d == d.min())
        c = best[0] if len(best) == 1 else [k for k in best if k % 2 == 0][0]
        codes.append(c | (0x80 if v < 0 else 0))
    return np.array(codes, dtype=np.uint8), e + 127


def test_quant_e4m3_brute_force(orc):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 64)) * np.array([[1e-3], [1.0], [300.0]])
    codes, scales = orc.quant_e4m3(x)
    for r in range(3):
        for blk in range(2):
            c, s = _brute_e4m3_block(x[r, 32 * blk:32 * blk + 32])
            assert scales[r, blk] == s
            assert np.array_equal(codes[r, 32 * blk:32 * blk + 32], c)


def test_quant_e2m1_brute_force(orc):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 32)) * np.array([[1e-3], [1.0], [7.0], [2000.0], [1.0]])
    x[1, :16] = 0.0
    # a block with amax 6 (scale 1) holding every midpoint between grid values: ties
    x[4, :16] = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75,
                 -2.5, -3.5, -5.0, 0.0]
    codes, scales = orc.quant_e2m1(x)
    e4 = torch.arange(127, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mags = np.array(E2M1_TABLE)
    for r in range(5):
        for blk in range(2):
            xb = x[r, 16 * blk:16 * blk + 16]
            amax = np.abs(xb).max()
            sc = next((k for k in range(1, 127) if 6 * e4[k] >= amax), 126)
            assert scales[r, blk] == sc
            s = e4[sc]
            for j, v in enumerate(xb):
                d = np.abs(np.abs(v) - mags * s)
                best = np.flatnonzero(d == d.min())
                c = best[0] if len(best) == 1 else [k for k in best if k % 2 == 0][0]
                c |= 8 if v < 0 else 0
                byte = codes[r, (16 * blk + j) // 2]
                got = (byte & 15) if j % 2 == 0 else (byte >> 4)
                assert got == c, (r, blk, j, v, s)


def _state(B, ratio, D):
    return (np.zeros((B, ratio, D), np.float32), np.full((B, ratio, D), -np.inf, np.float32))


def test_compressor_group_timing_and_pooling(orc):
    B, D, rd, ratio = 2, 64, 16, 4
    a = synth.make_append(B=B, D=D, rd=rd, ratio=ratio, steps=8, positions=16, seed=4)
    ks, gs = _state(B, ratio, D)
    codes = np.zeros((B, 4, D // 2), np.uint8)
    scales = np.zeros((B, 4, D // 16), np.uint8)
    kv = np.array(a.kv)
    score = np.zeros_like(a.score)               # equal scores: the pooled kv is the mean
    written = []
    for t in range(8):
        w, lat = orc.compress_append(kv[t], score[t], ks, gs, a.norm_w, a.eps, a.freqs, rd,
                                     codes, scales, t, ratio)
        written.append(w)
        assert np.array_equal(ks[:, t % ratio], kv[t]) and np.array_equal(gs[:, t % ratio], score[t])
        if w:
            mean = kv[t - 3:t + 1].astype(np.float64).mean(0)
            xb = np.array([[orc.round_bf16(v) for v in row] for row in mean])
            rms = np.sqrt((xb ** 2).mean(-1, keepdims=True) + a.eps)
            want = np.vectorize(orc.round_bf16)(a.norm_w.astype(np.float64) * (xb / rms))
            np.testing.assert_allclose(lat, want, rtol=0, atol=1e-12 * np.abs(want).max())
    assert written == [False, False, False, True] * 2
    assert codes[:, 2:].max() == 0 and scales[:, 2:].max() == 0   # rows 0 and 1 only
    # group 0 starts at position 0, whose rotation is the identity (angle 0)
    ks, gs = _state(B, ratio, D)
    for t in range(4):
        _, lat0 = orc.compress_append(kv[t], score[t], ks, gs, a.norm_w, a.eps, a.freqs, rd,
                                      codes, scales, t, ratio)
    c0, s0 = orc.quant_e2m1(lat0)
    assert np.array_equal(codes[:, 0], c0) and np.array_equal(scales[:, 0], s0)
    # a dominant gate score selects its slot's kv
    ks, gs = _state(B, ratio, D)
    sc2 = np.zeros((4, B, D), np.float32)
    sc2[2] = 1000.0
    for t in range(4):
        w, lat = orc.compress_append(kv[t], sc2[t], ks, gs, a.norm_w, a.eps, a.freqs, rd,
                                     codes, scales, t, ratio)
    xb = np.vectorize(orc.round_bf16)(kv[2].astype(np.float64))
    rms = np.sqrt((xb ** 2).mean(-1, keepdims=True) + a.eps)
    want = np.vectorize(orc.round_bf16)(a.norm_w.astype(np.float64) * (xb / rms))
    np.testing.assert_allclose(lat, want, rtol=0, atol=1e-12 * np.abs(want).max())


def test_rmsnorm_closed_form_and_rotation(orc):
    B, D, rd = 1, 32, 8
    w = np.linspace(0.5, 1.5, D).astype(np.float32)
    kv = np.full((1, B, D), -3.0, np.float32)     # constant row: norm = -w
    ident = np.zeros((4, rd // 2, 2), np.float32)
    ident[..., 0] = 1.0                           # cos 1, sin 0 at every position
    codes = np.zeros((B, 4, D // 2), np.uint8)
    scales = np.zeros((B, 4, D // 16), np.uint8)
    w_, lat = orc.compress_append(kv[0], kv[0], None, None, w, 1e-20, ident, rd, codes, scales, 0, 1)
    assert w_ and np.array_equal(lat[0], np.vectorize(orc.round_bf16)(-w.astype(np.float64)))
    c0, s0 = orc.quant_e2m1(lat)
    assert np.array_equal(codes[:, 0], c0) and np.array_equal(scales[:, 0], s0)
    # a quarter turn: (a, b) -> (-b, a) on the last rd dims
    quarter = np.zeros((4, rd // 2, 2), np.float32)
    quarter[..., 1] = 1.0
    x = np.random.default_rng(5).standard_normal((1, B, D)).astype(np.float32)
    _, lat = orc.compress_append(x[0], x[0], None, None, w, 1e-20, quarter, rd, codes, scales, 1, 1)
    rot = lat.copy()
    rot[0, D - rd::2], rot[0, D - rd + 1::2] = -lat[0, D - rd + 1::2], lat[0, D - rd::2]
    c1, s1 = orc.quant_e2m1(rot)
    assert np.array_equal(codes[:, 1], c1) and np.array_equal(scales[:, 1], s1)


def test_window_ring_and_identity_rotation(orc):
    B, D, rd, R = 2, 64, 16, 8
    a = synth.make_append(B=B, D=D, rd=rd, ratio=1, steps=3, positions=32, seed=6)
    codes = np.zeros((B, R, D), np.uint8)
    scales = np.zeros((B, R, D // 32), np.uint8)
    orc.window_append(a.win[0], a.freqs, rd, codes, scales, start_pos=0)
    x = np.array([[orc.bf16_value(int(b)) for b in row] for row in a.win[0]])
    c, s = orc.quant_e4m3(x)                     # position 0: cos 1, sin 0
    assert np.array_equal(codes[:, 0], c) and np.array_equal(scales[:, 0], s)
    orc.window_append(a.win[1], a.freqs, rd, codes, scales, start_pos=13)
    assert codes[:, 13 % R].any() and not codes[:, 1:5].any()


def test_producer_refuses_bad_arguments(orc):
    a = synth.make_append(B=1, D=64, rd=16, ratio=4, steps=1, positions=8, seed=7)
    ks, gs = _state(1, 4, 64)
    with pytest.raises(orc.OracleError):              # row 2 of a 2-row cache
        orc.compress_append(a.kv[0], a.score[0], ks, gs, a.norm_w, a.eps, a.freqs, 16,
                            np.zeros((1, 2, 32), np.uint8), np.zeros((1, 2, 4), np.uint8), 11, 4)


# -- chunks: the prefill seeding of the compressor state, the compressed rows and the ring --

@pytest.mark.parametrize("ratio,S", [(4, 14), (2, 9), (4, 4), (4, 3)])
def test_compress_chunk_is_the_pages_prefill(orc, ratio, S):
    """At start_pos 0 a chunk is the pages' prefill branch (Compressor.forward): the whole
    groups pooled at once -- kv times the softmax of the scores over each group's ratio
    tokens, summed -- the remaining S % ratio tokens left in state slots 0.., and group j's
    latent rotated at position j * ratio (Attention._compress_kv, freqs_cis[:cutoff:ratio]).
    The pooled values are recomputed here from that formula (numpy, fp64)."""
    B, D, rd = 2, 64, 16
    a = synth.make_append(B=B, D=D, rd=rd, ratio=ratio, steps=S, positions=64, seed=90 + S)
    kv, sc = a.kv.transpose(1, 0, 2).copy(), a.score.transpose(1, 0, 2).copy()
    ks = np.zeros((B, ratio, D), np.float32)
    gs = np.full((B, ratio, D), -np.inf, np.float32)
    codes = np.zeros((B, S // ratio + 1, D // 2), np.uint8)
    scales = np.zeros((B, S // ratio + 1, D // 16), np.uint8)
    n, lat, pooled, _ = orc.compress_chunk(kv, sc, ks, gs, a.norm_w, a.eps, a.freqs, rd, codes, scales, 0, ratio)
    cutoff = S - S % ratio
    assert n == S // ratio == cutoff // ratio
    g = sc[:, :cutoff].astype(np.float64).reshape(B, -1, ratio, D)
    p = np.exp(g - g.max(axis=2, keepdims=True))
    want = (kv[:, :cutoff].astype(np.float64).reshape(B, -1, ratio, D) * p / p.sum(axis=2, keepdims=True)).sum(axis=2)
    np.testing.assert_allclose(pooled, want, rtol=1e-12, atol=0)
    rem = S % ratio
    assert np.array_equal(ks[:, :rem], kv[:, cutoff:]) and np.array_equal(gs[:, :rem], sc[:, cutoff:])
    for b in range(B):
        for j in range(n):
            c, s = orc.compress_write(lat[b, j], a.freqs, rd, j * ratio)
            assert np.array_equal(codes[b, j], c) and np.array_equal(scales[b, j], s)


def test_compress_chunk_after_cached_tokens_continues_the_group(orc):
    """A chunk that starts inside a group (start_pos % ratio != 0) pools that group with the
    slots the earlier tokens left in the state; at every position the chunk equals the
    decode steps it stands for."""
    B, D, rd, ratio = 2, 64, 16, 4
    a = synth.make_append(B=B, D=D, rd=rd, ratio=ratio, steps=13, positions=64, seed=97)
    kv, sc = a.kv.transpose(1, 0, 2).copy(), a.score.transpose(1, 0, 2).copy()
    st = lambda: (np.zeros((B, ratio, D), np.float32), np.full((B, ratio, D), -np.inf, np.float32))  # noqa: E731
    cache = lambda: (np.zeros((B, 4, D // 2), np.uint8), np.zeros((B, 4, D // 16), np.uint8))  # noqa: E731
    ks1, gs1 = st()
    c1, s1 = cache()
    orc.compress_chunk(kv[:, :6], sc[:, :6], ks1, gs1, a.norm_w, a.eps, a.freqs, rd, c1, s1, 0, ratio)
    n, lat, _, _ = orc.compress_chunk(kv[:, 6:], sc[:, 6:], ks1, gs1, a.norm_w, a.eps, a.freqs, rd, c1, s1, 6, ratio)
    assert n == 13 // ratio - 6 // ratio == 2
    ks2, gs2 = st()
    c2, s2 = cache()
    lat2 = []
    for t in range(13):
        w, l2 = orc.compress_append(kv[:, t], sc[:, t], ks2, gs2, a.norm_w, a.eps, a.freqs, rd, c2, s2, t, ratio)
        if w and t >= 6:
            lat2.append(l2)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert np.array_equal(ks1, ks2) and np.array_equal(gs1, gs2)
    assert np.array_equal(lat, np.stack(lat2, axis=1))


@pytest.mark.parametrize("S,win", [(300, 128), (128, 128), (50, 128), (257, 64)])
def test_window_chunk_seeds_the_ring_like_the_pages(orc, S, win):
    """The pages' prefill seeding of the window ring (Attention._window_kv, start_pos 0):
    with S <= win the chunk's rows fill slots 0..S-1; else, with cutoff = S % win, the last
    win rows are split so that slots cutoff..win-1 take the first win - cutoff of them and
    slots 0..cutoff-1 the rest.  Each row is rotated at its own position and quantised."""
    B, D, rd = 2, 64, 16
    a = synth.make_append(B=B, D=D, rd=rd, ratio=1, steps=S, positions=S + 1, seed=S + win)
    win_bits = a.win.transpose(1, 0, 2).copy()
    codes = np.zeros((B, win, D), np.uint8)
    scales = np.zeros((B, win, D // 32), np.uint8)
    orc.window_chunk(win_bits, a.freqs, rd, codes, scales, 0)
    # the pages' split, as token positions per slot
    slot_tok = np.full(win, -1)
    if S <= win:
        slot_tok[:S] = np.arange(S)
    else:
        cutoff = S % win
        last = np.arange(S - win, S)
        slot_tok[cutoff:win], slot_tok[:cutoff] = last[:win - cutoff], last[win - cutoff:]
    for slot, t in enumerate(slot_tok):
        if t < 0:
            assert not codes[:, slot].any()
            continue
        one_c = np.zeros((B, 1, D), np.uint8)
        one_s = np.zeros((B, 1, D // 32), np.uint8)
        orc.window_append(win_bits[:, t], a.freqs, rd, one_c, one_s, int(t))  # slot t % 1 == 0
        assert np.array_equal(codes[:, slot], one_c[:, 0]) and np.array_equal(scales[:, slot], one_s[:, 0]), slot
