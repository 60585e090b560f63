"""lit_sparse_step_noalloc (the step on the library's own scratch, for callers that cannot
allocate) against lit_sparse_step on caller buffers, through the C ABI: identical top-k
lists and outputs on two calls in a row, the second with a smaller input, in both step
forms; no team timeout reported."""
import numpy as np
import pytest
import torch

import lightning_indexer_top_amd as L
from lightning_indexer_top_amd import synth
from tests.gpu_util import step_inputs_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.library()


def _args(inp, d, flags):
    return L.make_step_args(q8=d["q8"], q_sc=d["q_sc"], w=d["w"], k8=d["k8"], k_sc=d["k_sc"], q=d["q"],
                            win_kv=d["win_kv"], comp_kv=d["comp_kv"], start_pos=inp.start_pos,
                            ratio=inp.ratio, index_topk=inp.index_topk, W=inp.W, scale=inp.scale,
                            dv=inp.dv, sink=d["sink"], flags=flags, fmt=inp.index_fmt)


@pytest.mark.parametrize("flags", [0, L.LIT_STEP_UNFUSED], ids=["fused", "kernels"])
def test_noalloc_matches_step_twice(flags):
    for name in ["decode-16k", "decode-1k"]:   # the second input is smaller
        inp = synth.workload(name)
        d = step_inputs_dev(inp)
        args, idx, out = _args(inp, d, flags)
        state = L.attach_state(args) if flags == 0 else None
        ws = L.step_workspace(args)
        L.lit_sparse_step(args, ws)
        torch.cuda.synchronize()
        assert L.state_error(state) == 0
        ref_idx, ref_out = idx.clone(), out.clone()
        idx.fill_(-7)
        out.zero_()
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        L.lit_sparse_step_noalloc(args, err)
        torch.cuda.synchronize()
        assert err.item() == 0, name
        assert torch.equal(idx, ref_idx), name
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), name


def test_noalloc_refuses_a_workspace_beyond_its_scratch():
    inp = synth.workload("prefill-16k")   # 134 MB of scores: more than the 15 MiB workspace
    d = step_inputs_dev(inp)
    args, _, _ = _args(inp, d, 0)
    with pytest.raises(L.LitError) as e:
        L.lit_sparse_step_noalloc(args)
    assert e.value.status == 5   # LIT_E_WORKSPACE
