"""Pins of the oracle's pack/unpack gathers: a hand-written example and the
round trip. CPU only."""
import numpy as np

from oracle import pg_oracle as O


def _lay(P, S):
    return O.layout(P, [len(s) for s in S], [x for s in S for x in s])


def test_pack_hand_written_example():
    # group 0: prompt (10, 11), responses (20), (21, 22); group 1: no prompt,
    # one response (30, 31, 32); group 2: prompt (40), no response
    P, S = [2, 0, 1], [[1, 2], [3], []]
    lay = _lay(P, S)
    prefix = np.array([[10, 11], [0, 0], [40, 0]])
    suffix = np.array([[20, 0, 0], [21, 22, 0], [30, 31, 32]])
    packed = O.pack_rows(prefix, suffix, lay)
    assert packed.tolist() == [10, 11, 20, 21, 22, 30, 31, 32, 40]
    pre, suf = O.unpack_rows(packed, lay, 2, 3)
    assert pre.tolist() == [[10, 11], [0, 0], [40, 0]]
    # first column: the group's last prompt token (0 when there is no prompt)
    assert suf.tolist() == [[11, 20, 0, 0], [11, 21, 22, 0], [0, 30, 31, 32]]


def test_round_trip_on_random_rows():
    r = np.random.default_rng(0)
    P, S = [5, 0, 7, 1], [[3, 0, 4], [2], [], [1, 1]]
    lay = _lay(P, S)
    Pm, Sm = 8, 5
    prefix = r.standard_normal((len(P), Pm, 6))
    suffix = r.standard_normal((sum(len(s) for s in S), Sm, 6))
    packed = O.pack_rows(prefix, suffix, lay)
    assert packed.shape == (int(lay["total_tokens"]), 6)
    pre, suf = O.unpack_rows(packed, lay, Pm, Sm)
    k = 0
    for g, p in enumerate(P):
        assert np.array_equal(pre[g, :p], prefix[g, :p]) and not pre[g, p:].any()
        for _ in S[g]:
            s = lay["suffix_lens"][k]
            assert np.array_equal(suf[k, 1:1 + s], suffix[k, :s]) and not suf[k, 1 + s:].any()
            assert np.array_equal(suf[k, 0], prefix[g, p - 1] if p else np.zeros(6))
            k += 1
