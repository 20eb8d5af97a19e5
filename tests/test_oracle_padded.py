"""Pins of the oracle's right-padded form (``padded_positions``,
``padding_mask``, ``pad_rows``, ``unpad_rows``): hand-derived rows of the tiny
workload, agreement with the packed positions, round trips. CPU only."""
import numpy as np
import pytest

from oracle import pg_oracle as O
from workloads import make_workload


def test_tiny_workload_hand_derived():
    # groups P = 5, S = {3, 4} (12 tokens) and P = 9, S = {2, 6, 1} (18 tokens),
    # derived by hand from the verl page's loop: prompt 0..P-1, every response P..
    lay = O.layout([5, 9], [2, 3], [3, 4, 2, 6, 1])
    pos = O.padded_positions(lay, 20)
    assert pos[0].tolist() == [0, 1, 2, 3, 4, 5, 6, 7, 5, 6, 7, 8] + [0] * 8
    assert pos[1].tolist() == list(range(9)) + [9, 10] + list(range(9, 15)) + [9] + [0, 0]
    mask = O.padding_mask(lay, 20)
    assert mask[0].tolist() == [1] * 12 + [0] * 8 and mask[1].tolist() == [1] * 18 + [0] * 2
    assert mask.dtype == np.uint8


@pytest.mark.parametrize("shape", [
    ([5, 9], [[3, 4], [2, 6, 1]]), ([0, 7], [[4, 3], [5]]), ([6, 4, 3], [[], [0, 2], [0, 0]]),
    ([0], [[0, 3, 0]]), ([17], [[]]), ([0, 0], [[0], []])])
def test_real_tokens_carry_the_packed_positions(shape):
    P, S = shape
    lay = O.layout(P, [len(s) for s in S], [x for s in S for x in s])
    n = O.group_lens(lay)
    L = int(n.max()) + 3 if n.size else 3
    pos = O.padded_positions(lay, L)
    mask = O.padding_mask(lay, L)
    assert np.array_equal(O.unpad_rows(pos, lay), O.positions(lay))
    assert np.all(pos[mask == 0] == 0)
    x = np.arange(int(lay["total_tokens"]) * 3, dtype=np.int64).reshape(-1, 3) + 1
    padded = O.pad_rows(x, lay, L)
    assert np.array_equal(O.unpad_rows(padded, lay), x)
    assert np.all(padded[mask == 0] == 0) and np.all(padded[mask == 1] != 0)


def test_workload_round_trip_and_lengths():
    w = make_workload(1)
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    n = O.group_lens(lay)
    P = np.asarray(w.prefix_lens)
    sums = np.add.reduceat(np.asarray(w.suffix_lens), np.r_[0, np.cumsum(w.suffix_counts)[:-1]])
    assert np.array_equal(n, P + sums)
    pos = O.padded_positions(lay, int(n.max()))
    assert np.array_equal(O.unpad_rows(pos, lay), O.positions(lay))
