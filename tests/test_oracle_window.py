"""Pins for the oracle's window row lists.

Definition: DeepSeek-V4.1-Flash-NVFP4 model.py, get_window_topk_idxs and
Attention._window_kv.  The expected lists in ``tests/golden/window_derived.txt`` were
derived by evaluating that function's two branches by hand for the given (window,
seqlen, start_pos): decode cases at starts 2, 3 and 5 with a window of 4 (the ring
filling, full, and wrapped) and prefill cases of 5 tokens with a window of 3 and 2 tokens
with a window of 4.

A brute-force set check covers the chunk generalisation (start > 0, several queries).
"""
import os

import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "window_derived.txt")


def _load_derived():
    cases = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        head, body = line.split("|")
        W, S, start_pos = (int(x) for x in head.split())
        rows = [[int(v) for v in row.split(",")] for row in body.split(";")]
        cases.append((W, S, start_pos, rows))
    return cases


DERIVED = _load_derived()


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
