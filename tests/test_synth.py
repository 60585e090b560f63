"""Host checks of the seeded input generator's block quantisers (no method arithmetic:
they only have to write valid codes and scales, and the fp4 one is checked here against
brute-force nearest rounding so that the fp4 workloads have the intended spread)."""
import numpy as np
import torch

from lightning_indexer_top_amd import synth
from tests.test_oracle_formats import E2M1_TABLE


def _unpack(packed):
    p = packed.numpy()
    return np.stack([p & 15, p >> 4], axis=-1).reshape(*p.shape[:-1], 2 * p.shape[-1])


def test_fp4_quantiser_rounds_to_nearest_grid_value():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(64, 128, generator=g) * 3
    x[0, :32] = 0.0                      # an all-zero block
    packed, sc = synth.quantize_e2m1_ue8m0(x)
    assert packed.shape == (64, 64) and sc.shape == (64, 4)
    codes = _unpack(packed)
    lut = np.array(E2M1_TABLE + [-v for v in E2M1_TABLE])
    e = sc.numpy().astype(np.int32) - 127
    y = x.double().numpy().reshape(64, 4, 32) / (2.0 ** e)[..., None]
    assert np.abs(y).max() <= 6.0        # the scale keeps every block in range
    # amax of each nonzero block needs the chosen scale: half of it would overflow 6
    amax = np.abs(y).max(-1)
    assert np.all((amax > 3.0) | (amax == 0))
    got = lut[codes].reshape(64, 4, 32)
    grid = np.array(E2M1_TABLE)
    best = np.abs(np.abs(y)[..., None] - grid).min(-1)
    assert np.allclose(np.abs(np.abs(y) - np.abs(got)), best, atol=1e-12)
    assert np.all((np.sign(got) == np.sign(y)) | (got == 0))
    assert np.all(got.reshape(64, 128)[0, :32] == 0) and sc[0, 0] == 0


def test_fp4_quantiser_ties_go_to_even_codes():
    # midpoints between grid neighbours, scale 1 (the block's amax is 6)
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    even = [0, 2, 2, 4, 4, 6, 6]
    x = torch.zeros(32)
    x[0] = 6.0
    x[1:8] = torch.tensor(mids)
    x[8:15] = -torch.tensor(mids)
    packed, sc = synth.quantize_e2m1_ue8m0(x)
    assert int(sc[0]) == 127
    codes = _unpack(packed)
    assert list(codes[1:8]) == even
    assert list(codes[8:15]) == [c + 8 for c in even]


def test_fp4_workload_shapes():
    inp = synth.make_step(B=2, S=1, start_pos=99, ratio=2, Hi=16, Di=64, H=16, D=64, W=8,
                          index_topk=8, seed=4, index_fmt="e2m1", keys="boost")
    assert inp.index_fmt == "e2m1"
    assert inp.q8.shape == (2, 1, 16, 32) and inp.k8.shape == (2, 50, 32)
    assert inp.q_sc.shape == (2, 1, 16, 2) and inp.k_sc.shape == (2, 50, 2)
    assert inp.q8.dtype == np.uint8 and inp.k8.dtype == np.uint8


def test_fp4_kv_quantiser_minimal_e4m3_scales():
    g = torch.Generator().manual_seed(5)
    x = torch.randn(40, 192, generator=g) * 2
    x[3, :16] = 0.0
    packed, sc = synth.quantize_e2m1_e4m3(x)
    assert packed.shape == (40, 96) and sc.shape == (40, 12)
    s = sc.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    xb = x.double().numpy().reshape(40, 12, 16)
    amax = np.abs(xb).max(-1)
    assert np.all(amax / s <= 6.0)
    # the next smaller e4m3 value would not do (except for the all-zero block)
    prev = (sc.view(torch.uint8).int() - 1).clamp(min=0).to(torch.uint8)
    sp = prev.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.all((amax / np.where(sp > 0, sp, 1e-30) > 6.0) | (amax == 0))
    codes = _unpack(packed).reshape(40, 12, 16)
    lut = np.array(E2M1_TABLE + [-v for v in E2M1_TABLE])
    y = xb / s[..., None]
    best = np.abs(np.abs(y)[..., None] - np.array(E2M1_TABLE)).min(-1)
    assert np.allclose(np.abs(np.abs(y) - np.abs(lut[codes])), best, atol=1e-9)
