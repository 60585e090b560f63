"""Pins for the oracle's window row lists.

Definition: DeepSeek-V4.1-Flash-NVFP4 model.py, get_window_topk_idxs and
Attention._window_kv.  The expected lists below were derived by evaluating that
function's two branches by hand for the given (window, seqlen, start_pos):

* decode, window 4, start 2: oldest slot = 2 % 4 + 1 = 3; slots 3, 0, 1, 2; slot 3 is
  past start 2, so it is -1 (ring still filling);
* decode, window 4, start 3: slots 0..3, all filled;
* decode, window 4, start 5: oldest slot 2; slots 2, 3, 0, 1;
* prefill, window 3, 5 tokens: row i lists max(0, i-2) + (0, 1, 2), entries past i
  become -1;
* prefill, window 4, 2 tokens: width min(2, 4) = 2.

A brute-force set check covers the chunk generalisation (start > 0, several queries).
"""
import numpy as np
import pytest

DERIVED = [
    # (W, S, start_pos, expected rows)
    (4, 1, 2, [[-1, 0, 1, 2]]),
    (4, 1, 3, [[0, 1, 2, 3]]),
    (4, 1, 5, [[2, 3, 0, 1]]),
    (3, 5, 0, [[0, -1, -1], [0, 1, -1], [0, 1, 2], [1, 2, 3], [2, 3, 4]]),
    (4, 2, 0, [[0, -1], [0, 1]]),
]


@pytest.mark.parametrize("W,S,start_pos,rows", DERIVED)
def test_derived_cases(orc, W, S, start_pos, rows):
    R = W if start_pos > 0 else S
    got = orc.window_indices(2, S, start_pos, W, R)
    assert got.shape == (2, S, len(rows[0]))
    assert got[0].tolist() == rows and got[1].tolist() == rows


@pytest.mark.parametrize("W,S,start_pos,R", [(128, 1, 1023, 128), (128, 64, 12288, 191),
                                             (8, 20, 3, 40), (16, 5, 0, 5), (128, 300, 0, 300),
                                             (4, 7, 100, 10)])
def test_brute_force_sets(orc, W, S, start_pos, R):
    got = orc.window_indices(1, S, start_pos, W, R)
    for i in range(S):
        P = start_pos + i
        want = sorted(p % R for p in range(max(0, P - W + 1), P + 1))
        row = [x for x in got[0, i] if x >= 0]
        assert sorted(row) == want
        assert len(set(row)) == len(row)


def test_refuses_short_ring(orc):
    with pytest.raises(orc.OracleError):
        orc.window_indices(1, 8, 100, 16, 16)  # needs W + S - 1 = 23 slots
