"""Helpers shared by the GPU tests: host arrays -> device tensors and back."""
import numpy as np
import torch


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return dev(np.ascontiguousarray(bits).view(np.int16), torch.bfloat16)


def bf16_host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def step_inputs_dev(inp):
    """Device copies of every array of a synth.StepInputs (quantised KV sources stay
    uint8 codes, with their scale bytes as win_sc / comp_sc)."""
    wq = getattr(inp, "win_kv_fmt", "bf16") != "bf16"
    cq = getattr(inp, "comp_kv_fmt", "bf16") != "bf16"
    return dict(q8=dev(inp.q8), q_sc=dev(inp.q_sc), w=dev(inp.w), k8=dev(inp.k8),
                k_sc=dev(inp.k_sc), q=bf16_dev(inp.q),
                win_kv=dev(inp.win_kv) if wq else bf16_dev(inp.win_kv),
                comp_kv=dev(inp.comp_kv) if cq else bf16_dev(inp.comp_kv),
                win_sc=dev(inp.win_sc) if wq else None, comp_sc=dev(inp.comp_sc) if cq else None,
                sink=None if inp.sink is None else dev(inp.sink))


def lib_dequant(codes, scales, fmt="e4m3"):
    """Codes x ue8m0 scales (for tolerance scales): e4m3 decoded with torch's casts,
    fp4 (e2m1, two codes a byte, element 2j low) with a table lookup."""
    s = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e8m0fnu).to(torch.float64)
    if fmt == "e2m1":
        from tests.test_oracle_formats import E2M1_TABLE
        p = np.ascontiguousarray(codes)
        lut = np.array(E2M1_TABLE + [-v for v in E2M1_TABLE])
        vals = np.stack([lut[p & 15], lut[p >> 4]], axis=-1).reshape(*p.shape[:-1], 2 * p.shape[-1])
        c = torch.from_numpy(vals)
    else:
        c = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64)
    return (c.unflatten(-1, (-1, 32)) * s.unsqueeze(-1)).flatten(-2).numpy()


def score_tolerance(inp):
    """Per-entry bound for fp32/MFMA scores: 1e-4 of sum_h w_h sum_d |q_hd k_td| (the
    magnitude the contraction accumulates) plus 1e-6 relative; see the design doc."""
    fmt = getattr(inp, "index_fmt", "e4m3")
    qd = np.abs(lib_dequant(inp.q8, inp.q_sc, fmt))     # [B,S,Hi,Di]
    kd = np.abs(lib_dequant(inp.k8, inp.k_sc, fmt))     # [B,T_cap,Di]
    T = inp.T
    out = np.empty((inp.B, inp.S, T))
    for b in range(inp.B):
        wq = np.einsum("sh,shd->sd", inp.w[b].astype(np.float64), qd[b])   # [S,Di]
        out[b] = wq @ kd[b, :T].T
    return out


def topk_sets_agree(orc_scores, orc_idx, gpu_idx, rel=1e-3):
    """The acceptance rule for top-k: identical sets, except that every row in the
    symmetric difference scores within rel * |s_k| of the oracle's k-th score s_k."""
    o = set(int(x) for x in orc_idx if x >= 0)
    g = set(int(x) for x in gpu_idx if x >= 0)
    if len(o) != len(g):
        return False, f"sizes differ {len(o)} vs {len(g)}"
    if o == g:
        return True, ""
    sk = min(orc_scores[t] for t in o)
    for t in o ^ g:
        if abs(orc_scores[t] - sk) > rel * abs(sk):
            return False, f"row {t} score {orc_scores[t]} vs k-th {sk}"
    return True, f"{len(o ^ g)} near-tie swaps"
