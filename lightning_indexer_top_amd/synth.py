"""Seeded synthetic inputs for the sparse-attention step.

This module is shared by the tests, the bench and the smoke check, and is the only
code both the HIP path's callers and the CPU oracle's callers use.  It holds no part
of the method's arithmetic: only random draws, the bf16 / e4m3 casts of a library
(torch), and the block quantisers that write e4m3 (or fp4 e2m1) codes with one ue8m0
scale per 32 values (the formats of the DeepSeek-V4.1-Flash-NVFP4 ``inference/model.py``
module globals and its indexer).  The quantisers' rounding rules are not on the pages;
any rule that yields valid bytes will do, because both sides consume the same bytes.

Recipe (per workload, ``numpy.random.Generator(PCG64(seed))``):

* attention q, window KV, compressed KV ~ N(0, 1), rounded to bf16 (RNE); with
  ``kv_fmt="quant"`` the window KV is e4m3 with a ue8m0 scale per 32 and the compressed
  KV fp4 e2m1 with an e4m3 scale per 16 (the smallest e4m3 value >= amax / 6);
* indexer q and keys ~ N(0, 1), quantised to e4m3 with a ue8m0 scale per 32
  values: scale exponent e = ceil(log2(amax / 448)), codes = RNE(x / 2^e);
  with ``index_fmt="e2m1"`` to fp4 instead: e = ceil(log2(amax / 6)), codes = RNE
  onto the e2m1 grid, two per byte (element 2j in the low nibble of byte j);
* head weights w ~ U(0, 1) in fp32;
* ``keys="boost"``: 5% of each sequence's key rows multiplied by 4, which leaves
  the codes unchanged and adds 2 to each of the row's scale bytes;
* ``keys="mixture"``: keys = mu_z + 0.1 * eps with 64 centroids mu ~ N(0, I),
  z uniform, eps ~ N(0, I).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float array -> uint16 bf16 bit patterns (round to nearest even, via torch)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def quantize_e4m3_ue8m0(x: torch.Tensor, block: int = 32):
    """Block quantiser: x [..., D] -> (codes uint8 [..., D], scales uint8 [..., D/block]).

    Works on CPU or GPU tensors.  The scale is the smallest power of two 2^e with
    amax / 2^e <= 448; an all-zero block gets the smallest scale byte (0).
    """
    assert x.shape[-1] % block == 0
    xf = x.float()
    xb = xf.unflatten(-1, (-1, block))
    amax = xb.abs().amax(dim=-1)
    safe = torch.where(amax > 0, amax, torch.ones_like(amax))
    e = torch.ceil(torch.log2(safe / E4M3_MAX))
    # guard the float log2 rounding: make sure amax / 2^e <= 448 really holds
    e = torch.where(safe / torch.exp2(e) > E4M3_MAX, e + 1, e)
    e = torch.where(amax > 0, e, torch.full_like(e, -127.0)).clamp(-127, 127)
    y = xb / torch.exp2(e).unsqueeze(-1)
    codes = y.clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
    scales = (e + 127).to(torch.uint8)
    return codes.flatten(-2), scales


def _pow2_scale(xb: torch.Tensor, vmax: float):
    """Per-block ue8m0 exponent: the smallest e with amax / 2^e <= vmax (all-zero block:
    -127).  Returns (e as float, scale bytes)."""
    amax = xb.abs().amax(dim=-1)
    safe = torch.where(amax > 0, amax, torch.ones_like(amax))
    e = torch.ceil(torch.log2(safe / vmax))
    e = torch.where(safe / torch.exp2(e) > vmax, e + 1, e)
    e = torch.where(amax > 0, e, torch.full_like(e, -127.0)).clamp(-127, 127)
    return e, (e + 127).to(torch.uint8)


def quantize_e2m1_ue8m0(x: torch.Tensor, block: int = 32):
    """fp4 block quantiser: x [..., D] -> (packed codes uint8 [..., D/2], scales uint8
    [..., D/block]).  Codes round to the nearest e2m1 value (0, 0.5, 1, 1.5, 2, 3, 4,
    6), ties to the even code; element 2j goes to the low nibble of byte j."""
    assert x.shape[-1] % block == 0 and block % 2 == 0
    xb = x.float().unflatten(-1, (-1, block))
    e, scales = _pow2_scale(xb, E2M1_MAX)
    y = (xb / torch.exp2(e).unsqueeze(-1)).clamp(-E2M1_MAX, E2M1_MAX)
    m = y.abs()
    # midpoints between neighbouring grid values; at a tie the even code wins, so the
    # comparison is strict above an even code and inclusive above an odd one
    code = ((m > 0.25).int() + (m >= 0.75).int() + (m > 1.25).int() + (m >= 1.75).int()
            + (m > 2.5).int() + (m >= 3.5).int() + (m > 5.0).int())
    code = code + 8 * (y < 0).int()
    code = code.flatten(-2)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).to(torch.uint8)
    return packed, scales


def quantize_e2m1_e4m3(x: torch.Tensor, block: int = 16):
    """fp4 quantiser with e4m3 scales (the compressed-KV format): x [..., D] -> (packed
    codes uint8 [..., D/2], scales uint8 [..., D/block] e4m3).  The scale is the smallest
    e4m3 value s with amax / s <= 6 (an all-zero block gets the smallest positive e4m3,
    code 1); codes round to the nearest e2m1 value, ties to the even code, element 2j in
    the low nibble of byte j."""
    assert x.shape[-1] % block == 0 and block % 2 == 0
    xb = x.float().unflatten(-1, (-1, block))
    amax = xb.abs().amax(dim=-1)
    want = torch.where(amax > 0, amax / E2M1_MAX, torch.full_like(amax, 2.0 ** -9))
    sc = want.clamp(max=E4M3_MAX).to(torch.float8_e4m3fn)
    # round the scale up where the cast rounded it down
    low = sc.to(torch.float32) < want
    codes = sc.view(torch.uint8).to(torch.int32) + low.to(torch.int32)
    scales = codes.clamp(max=0x7E).to(torch.uint8)
    s = scales.view(torch.float8_e4m3fn).to(torch.float32)
    y = (xb / s.unsqueeze(-1)).clamp(-E2M1_MAX, E2M1_MAX)
    m = y.abs()
    code = ((m > 0.25).int() + (m >= 0.75).int() + (m > 1.25).int() + (m >= 1.75).int()
            + (m > 2.5).int() + (m >= 3.5).int() + (m > 5.0).int())
    code = (code + 8 * (y < 0).int()).flatten(-2)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).to(torch.uint8)
    return packed, scales


def _quant_np(x: np.ndarray, fmt: str = "e4m3"):
    q = quantize_e2m1_ue8m0 if fmt == "e2m1" else quantize_e4m3_ue8m0
    c, s = q(torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)))
    return c.numpy().copy(), s.numpy().copy()


@dataclasses.dataclass
class StepInputs:
    """Host arrays for one step plus its sizes.  bf16 tensors are uint16 bit patterns."""
    name: str
    B: int
    S: int
    start_pos: int
    ratio: int
    Hi: int
    Di: int
    H: int
    D: int
    dv: int
    W: int
    R: int
    T_cap: int
    index_topk: int
    scale: float
    q8: np.ndarray       # [B,S,Hi,Di] u8 e4m3 (e2m1: [B,S,Hi,Di/2], two codes a byte)
    q_sc: np.ndarray     # [B,S,Hi,Di/32] u8 e8m0
    w: np.ndarray        # [B,S,Hi] f32
    k8: np.ndarray       # [B,T_cap,Di] u8 e4m3 (e2m1: [B,T_cap,Di/2])
    k_sc: np.ndarray     # [B,T_cap,Di/32] u8 e8m0
    q: np.ndarray        # [B,S,H,D] bf16 bits
    win_kv: np.ndarray   # [B,R,D] bf16 bits
    comp_kv: np.ndarray  # [B,T_cap,D] bf16 bits
    sink: Optional[np.ndarray] = None  # [H] f32 or None
    seed: int = 0
    index_fmt: str = "e4m3"  # code format of q8 / k8: "e4m3" or "e2m1"
    # quantised attention KV: win_kv "e4m3" -> uint8 [B,R,D] codes + win_sc [B,R,D/32]
    # ue8m0; comp_kv "e2m1" -> uint8 [B,T_cap,D/2] codes + comp_sc [B,T_cap,D/16] e4m3
    win_kv_fmt: str = "bf16"
    comp_kv_fmt: str = "bf16"
    win_sc: Optional[np.ndarray] = None
    comp_sc: Optional[np.ndarray] = None

    @property
    def end_pos(self) -> int:
        return self.start_pos + self.S

    @property
    def T(self) -> int:
        return self.end_pos // self.ratio if self.ratio > 0 else 0

    @property
    def k_eff(self) -> int:
        return min(self.index_topk, self.T)


def make_step(*, B: int, S: int, start_pos: int, ratio: int, Hi: int, Di: int, H: int,
              D: int, W: int, index_topk: int, seed: int, dv: Optional[int] = None,
              R: Optional[int] = None, T_cap: Optional[int] = None, keys: str = "normal",
              sink: Optional[np.ndarray] = None, scale: Optional[float] = None,
              index_fmt: str = "e4m3", name: str = "custom", cand_topk_blocks: int = 0,
              cand_block_size: int = 0, layers: int = 1, kv_fmt: str = "bf16",
              append_rd: int = 0) -> StepInputs:
    """Draw one step's inputs.  R defaults to the smallest window source that holds
    every needed position; T_cap defaults to the visible compressed row count.
    ``cand_topk_blocks`` / ``cand_block_size`` name a level-two workload's candidate
    source (the bench builds the candidates), ``layers`` the layers sharing one top-k
    (the bench draws the other layers' inputs), and ``append_rd`` a step preceded by its
    cache writes with that many rotated dims; they do not change the draw."""
    rng = np.random.Generator(np.random.PCG64(seed))
    end_pos = start_pos + S
    T = end_pos // ratio if ratio > 0 else 0
    if T_cap is None:
        T_cap = max(T, 1)
    if R is None:
        R = max(1, S if start_pos == 0 else W + S - 1)
    dv = D if dv is None else dv
    scale = D ** -0.5 if scale is None else scale
    f32 = np.float32

    assert index_fmt in ("e4m3", "e2m1")
    q8, q_sc = _quant_np(rng.standard_normal((B, S, Hi, Di), dtype=f32), index_fmt)
    w = rng.random((B, S, Hi), dtype=f32)
    if keys == "mixture":
        mu = rng.standard_normal((64, Di), dtype=f32)
        z = rng.integers(0, 64, size=(B, T_cap))
        kf = mu[z] + f32(0.1) * rng.standard_normal((B, T_cap, Di), dtype=f32)
    else:
        kf = rng.standard_normal((B, T_cap, Di), dtype=f32)
    k8, k_sc = _quant_np(kf, index_fmt)
    if keys == "boost":
        n_boost = max(1, int(round(0.05 * T_cap)))
        for b in range(B):
            rows = rng.choice(T_cap, size=n_boost, replace=False)
            # x4 = 2^2: codes stay, every block scale of the row rises by 2
            k_sc[b, rows] = np.minimum(k_sc[b, rows].astype(np.int32) + 2, 254).astype(np.uint8)
    q = to_bf16_bits(rng.standard_normal((B, S, H, D), dtype=f32))
    win_f = rng.standard_normal((B, R, D), dtype=f32)
    comp_f = rng.standard_normal((B, T_cap, D), dtype=f32)
    win_sc = comp_sc = None
    if kv_fmt == "quant":  # the pages' cache formats: e4m3/ue8m0-32 window, e2m1/e4m3-16 compressed
        win_kv, win_sc = _quant_np(win_f, "e4m3")
        c, sc_ = quantize_e2m1_e4m3(torch.from_numpy(comp_f))
        comp_kv, comp_sc = c.numpy().copy(), sc_.numpy().copy()
    else:
        assert kv_fmt == "bf16"
        win_kv, comp_kv = to_bf16_bits(win_f), to_bf16_bits(comp_f)
    return StepInputs(name=name, B=B, S=S, start_pos=start_pos, ratio=ratio, Hi=Hi, Di=Di,
                      H=H, D=D, dv=dv, W=W, R=R, T_cap=T_cap, index_topk=index_topk,
                      scale=scale, q8=q8, q_sc=q_sc, w=w, k8=k8, k_sc=k_sc, q=q,
                      win_kv=win_kv, comp_kv=comp_kv, sink=sink, seed=seed, index_fmt=index_fmt,
                      win_kv_fmt="e4m3" if kv_fmt == "quant" else "bf16",
                      comp_kv_fmt="e2m1" if kv_fmt == "quant" else "bf16",
                      win_sc=win_sc, comp_sc=comp_sc)


# The five workloads of the sparse-attention step.  Decode with "context L" is one query
# at start_pos = L-1 (so end_pos = L and L/r compressed rows are visible).
WORKLOADS = {
    "decode-1k": dict(B=1, S=1, start_pos=1023, ratio=2, Hi=16, Di=64, H=16, D=128, W=128,
                      index_topk=64, seed=20261212),
    "decode-4k-r2": dict(B=4, S=1, start_pos=4095, ratio=2, Hi=16, Di=64, H=16, D=128, W=128,
                         index_topk=64, seed=20261222, keys="boost"),
    "decode-4k-r1": dict(B=4, S=1, start_pos=4095, ratio=1, Hi=16, Di=64, H=16, D=128, W=128,
                         index_topk=64, seed=20261223, keys="boost"),
    "decode-16k": dict(B=8, S=1, start_pos=16383, ratio=2, Hi=64, Di=128, H=16, D=192, W=128,
                       index_topk=2048, seed=20261232),
    "prefill-16k": dict(B=1, S=4096, start_pos=12288, ratio=2, Hi=16, Di=64, H=16, D=128,
                        W=128, index_topk=512, seed=20261242),
    "decode-128k": dict(B=2, S=1, start_pos=131071, ratio=4, Hi=64, Di=128, H=16, D=128,
                        W=128, index_topk=2048, seed=20261252, keys="mixture"),
    # the 16K and 128K decode shapes with fp4 (e2m1) index queries and keys, the
    # indexer precision of DeepSeek-V4.1's own Indexer.forward
    "decode-16k-fp4": dict(B=8, S=1, start_pos=16383, ratio=2, Hi=64, Di=128, H=16, D=192,
                           W=128, index_topk=2048, seed=20261262, index_fmt="e2m1"),
    # decode-128k as a level-two layer of the two-level top-k (DeepSeek-V4.1's released
    # setting: 2048 candidate blocks of 8 rows from a candidate-source layer)
    "decode-128k-2level": dict(B=2, S=1, start_pos=131071, ratio=4, Hi=64, Di=128, H=16, D=128,
                               W=128, index_topk=2048, seed=20261282, keys="mixture",
                               cand_topk_blocks=2048, cand_block_size=8),
    # decode-16k as a level-two layer: 2048 blocks of 8 cover all 8192 rows, so the masked
    # kernel runs with nothing masked (the cost of the masking machinery alone)
    "decode-16k-2level": dict(B=8, S=1, start_pos=16383, ratio=2, Hi=64, Di=128, H=16, D=192,
                              W=128, index_topk=2048, seed=20261292, cand_topk_blocks=2048,
                              cand_block_size=8),
    # decode-16k for three layers sharing one indexer and top-k (DeepSeek-V4.1's
    # index_source_layers): the source layer's step, then the two other layers' attention
    # over its list in one call
    "decode-16k-3layer": dict(B=8, S=1, start_pos=16383, ratio=2, Hi=64, Di=128, H=16, D=192,
                              W=128, index_topk=2048, seed=20261302, layers=3),
    # decode-16k with the pages' quantised caches: window KV e4m3 (ue8m0 per 32),
    # compressed KV fp4 e2m1 (e4m3 scale per 16), dequantised on gather
    "decode-16k-qkv": dict(B=8, S=1, start_pos=16383, ratio=2, Hi=64, Di=128, H=16, D=192,
                           W=128, index_topk=2048, seed=20261312, kv_fmt="quant"),
    # the same step preceded by its cache writes: the new token into the compressor
    # (completing a group, so a compressed row is written) and into the window ring
    "decode-16k-qkv-append": dict(B=8, S=1, start_pos=16383, ratio=2, Hi=64, Di=128, H=16,
                                  D=192, W=128, index_topk=2048, seed=20261322, kv_fmt="quant",
                                  append_rd=64),
    "decode-128k-fp4": dict(B=2, S=1, start_pos=131071, ratio=4, Hi=64, Di=128, H=16, D=128,
                            W=128, index_topk=2048, seed=20261272, keys="mixture",
                            index_fmt="e2m1"),
}


def workload(name: str, **overrides) -> StepInputs:
    kw = dict(WORKLOADS[name])
    kw.update(overrides)
    return make_step(name=name, **kw)


def rope_table(rd: int, positions: int, base: float) -> np.ndarray:
    """Rotary table [positions, rd/2, 2] float32 (cos, sin): the frequencies
    1 / base^(2j/rd) times the position, in float32 as DeepSeek-V4.1-Flash-NVFP4
    model.py's precompute_freqs_cis tabulates them without YaRN (original_seq_len 0)."""
    freqs = 1.0 / (base ** (torch.arange(0, rd, 2, dtype=torch.float32) / rd))
    ang = torch.outer(torch.arange(positions, dtype=torch.float32), freqs)
    return torch.stack([torch.cos(ang), torch.sin(ang)], dim=-1).numpy().astype(np.float32)


@dataclasses.dataclass
class AppendInputs:
    """One decode step's producer inputs: the new token's compressor kv / gate score
    (fp32, after the projections) and window KV row (bf16 bits, after kv_norm), the
    RMSNorm weight, and the rotary table."""
    B: int
    D: int
    rd: int
    ratio: int
    kv: np.ndarray        # [steps, B, D] f32
    score: np.ndarray     # [steps, B, D] f32
    win: np.ndarray       # [steps, B, D] bf16 bits
    norm_w: np.ndarray    # [D] f32
    freqs: np.ndarray     # [positions, rd/2, 2] f32
    eps: float = 1e-20


def make_append(*, B: int, D: int, rd: int, ratio: int, steps: int, positions: int, seed: int,
                base: float = 40000.0) -> AppendInputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    f32 = np.float32
    return AppendInputs(B=B, D=D, rd=rd, ratio=ratio,
                        kv=rng.standard_normal((steps, B, D), dtype=f32),
                        score=rng.standard_normal((steps, B, D), dtype=f32),
                        win=to_bf16_bits(rng.standard_normal((steps, B, D), dtype=f32)),
                        norm_w=(0.5 + rng.random(D, dtype=f32)).astype(f32),
                        freqs=rope_table(rd, positions, base))


def random_scores(B: int, S: int, T: int, seed: int, ties: bool = False) -> np.ndarray:
    """fp32 score rows for testing a selector alone; with ``ties`` the values come from
    a small set so that many rows share a score."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if ties:
        return rng.integers(-4, 5, size=(B, S, T)).astype(np.float32)
    return rng.standard_normal((B, S, T), dtype=np.float32)


def draw_step_device(spec: dict, seed: int, device="cuda") -> dict:
    """The same recipe drawn directly on the GPU with torch's generator (for the bench's
    rotating input instances, which only need the shapes and distributions, not the
    host copies).  Returns device tensors keyed like StepInputs' arrays."""
    B, S, start_pos, ratio = spec["B"], spec["S"], spec["start_pos"], spec["ratio"]
    Hi, Di, H, D, W = spec["Hi"], spec["Di"], spec["H"], spec["D"], spec["W"]
    T = (start_pos + S) // ratio
    T_cap = max(T, 1)
    R = max(1, S if start_pos == 0 else W + S - 1)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    f32 = dict(dtype=torch.float32, device=device, generator=g)
    quant = quantize_e2m1_ue8m0 if spec.get("index_fmt", "e4m3") == "e2m1" else quantize_e4m3_ue8m0
    q8, q_sc = quant(torch.randn(B, S, Hi, Di, **f32))
    w = torch.rand(B, S, Hi, **f32)
    keys = spec.get("keys", "normal")
    if keys == "mixture":
        mu = torch.randn(64, Di, **f32)
        z = torch.randint(0, 64, (B, T_cap), device=device, generator=g)
        kf = mu[z] + 0.1 * torch.randn(B, T_cap, Di, **f32)
    else:
        kf = torch.randn(B, T_cap, Di, **f32)
    k8, k_sc = quant(kf)
    if keys == "boost":
        n_boost = max(1, int(round(0.05 * T_cap)))
        for b in range(B):
            rows = torch.randperm(T_cap, device=device, generator=g)[:n_boost]
            k_sc[b, rows] = (k_sc[b, rows].int() + 2).clamp(max=254).to(torch.uint8)
    bf = torch.bfloat16
    q = torch.randn(B, S, H, D, **f32).to(bf)
    win_f, comp_f = torch.randn(B, R, D, **f32), torch.randn(B, T_cap, D, **f32)
    win_sc = comp_sc = None
    if spec.get("kv_fmt", "bf16") == "quant":
        win_kv, win_sc = quantize_e4m3_ue8m0(win_f)
        comp_kv, comp_sc = quantize_e2m1_e4m3(comp_f)
        win_kv, win_sc = win_kv.contiguous(), win_sc.contiguous()
        comp_kv, comp_sc = comp_kv.contiguous(), comp_sc.contiguous()
    else:
        win_kv, comp_kv = win_f.to(bf), comp_f.to(bf)
    return dict(q8=q8.contiguous(), q_sc=q_sc.contiguous(), w=w, k8=k8.contiguous(),
                k_sc=k_sc.contiguous(), q=q, win_kv=win_kv, comp_kv=comp_kv, win_sc=win_sc,
                comp_sc=comp_sc, R=R, T_cap=T_cap)
