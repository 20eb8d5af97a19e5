"""Pins of the oracle's decode step (``decode_attention``) against things other
than itself: the forward oracle's last row of every response on the compacted
layout, torch's float64 SDPA per response, closed forms and a planted mistake.
CPU only."""
import numpy as np
import pytest
import torch

from oracle import pg_oracle as O
from workloads import draw_decode, make_custom, make_workload

# (prompt lengths, response capacities per group, Hq, Hkv, d)
CASES = [
    ([5, 9], [[3, 4], [2, 6, 1]], 2, 1, 8),
    ([0, 7], [[4, 3], [5]], 4, 2, 8),        # prompt-less group
    ([6, 4, 3], [[], [1, 2], [3, 3, 3]], 6, 2, 4),   # response-less group
    ([12], [[7, 1, 9, 4]], 8, 8, 4),          # MHA
]


def _draw(P, S, hq, hkv, d, seed):
    r = np.random.default_rng(seed)
    lay = O.layout(P, [len(x) for x in S], [c for g in S for c in g])
    T, N = int(lay["total_tokens"]), len(lay["suffix_lens"])
    k = r.standard_normal((T, hkv, d))
    v = r.standard_normal((T, hkv, d))
    q = r.standard_normal((N, hq, d))
    caps = np.asarray(lay["suffix_lens"])
    cur = np.array([r.integers(1, c + 1) if c > 0 else 0 for c in caps], dtype=np.int64)
    return lay, q, k, v, cur


def _compact(lay, q_dec, k, v, cur, hq, rng):
    """The cache compacted to the valid rows, as a packed layout whose response
    lengths are the current ones, with each decode query placed at its
    response's last row (other query rows random)."""
    P = [int(x) for x in lay["prefix_lens"]]
    n = [int(x) for x in lay["suffix_counts"]]
    lay_c = O.layout(P, n, [int(x) for x in cur])
    keep, kk = [], 0
    for g in range(len(P)):
        a = int(lay["group_off"][g])
        keep.extend(range(a, a + P[g]))
        for _ in range(n[g]):
            s0 = int(lay["seg_off"][g + kk + 1])
            keep.extend(range(s0, s0 + int(cur[kk])))
            kk += 1
    keep = np.asarray(keep, dtype=np.int64)
    Tc = int(lay_c["total_tokens"])
    d = k.shape[2]
    qc = rng.standard_normal((Tc, hq, d))
    last = []
    for kk in range(len(cur)):
        g = int(O.response_group(lay_c)[kk])
        t = int(lay_c["seg_off"][g + kk + 1]) + int(cur[kk]) - 1
        qc[t] = q_dec[kk]
        last.append(t)
    return lay_c, qc, k[keep], v[keep], np.asarray(last)


@pytest.mark.parametrize("case", CASES)
def test_decode_equals_forward_last_rows(case):
    P, S, hq, hkv, d = case
    lay, q, k, v, cur = _draw(P, S, hq, hkv, d, seed=1)
    scale = 1.0 / np.sqrt(d)
    o, lse = O.decode_attention(q, k, v, lay, cur, scale, hq, hkv)
    lay_c, qc, kc, vc, last = _compact(lay, q, k, v, cur, hq, np.random.default_rng(2))
    of, lf = O.attention(qc, kc, vc, lay_c, scale, hq, hkv)
    assert np.abs(o - of[last]).max() < 1e-12
    assert np.abs(lse - lf[:, last]).max() < 1e-12


@pytest.mark.parametrize("case", CASES)
def test_decode_matches_torch_sdpa(case):
    P, S, hq, hkv, d = case
    lay, q, k, v, cur = _draw(P, S, hq, hkv, d, seed=3)
    scale = 0.3
    o, lse = O.decode_attention(q, k, v, lay, cur, scale, hq, hkv)
    r = hq // hkv
    for kk in range(len(cur)):
        rows = O.decode_key_rows(lay, cur, kk)
        ks = torch.tensor(k[rows]).transpose(0, 1).repeat_interleave(r, dim=0)   # [Hq, L, d]
        vs = torch.tensor(v[rows]).transpose(0, 1).repeat_interleave(r, dim=0)
        qs = torch.tensor(q[kk]).unsqueeze(1)                                    # [Hq, 1, d]
        ref = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, scale=scale)[:, 0]
        assert np.abs(o[kk] - ref.numpy()).max() < 1e-12
        s = scale * torch.einsum("hd,hld->hl", qs[:, 0], ks)
        assert np.abs(lse[:, kk] - torch.logsumexp(s, dim=1).numpy()).max() < 1e-12


def test_decode_closed_forms():
    r = np.random.default_rng(5)
    # one key: no prompt, one valid row -> o = v of that row, lse = its score
    lay = O.layout([0], [2], [3, 2])
    k = r.standard_normal((5, 1, 4)); v = r.standard_normal((5, 1, 4)); q = r.standard_normal((2, 2, 4))
    o, lse = O.decode_attention(q, k, v, lay, np.array([1, 1]), 0.5, 2, 1)
    for kk, row in ((0, 0), (1, 3)):
        assert np.allclose(o[kk], v[row, 0][None, :], atol=0)
        assert np.allclose(lse[:, kk], 0.5 * q[kk] @ k[row, 0], atol=1e-15)
    # empty key set: o = 0, lse = -inf
    o, lse = O.decode_attention(q, k, v, lay, np.array([0, 2]), 0.5, 2, 1)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[:, 0])) and np.all(np.isfinite(lse[:, 1]))
    # lengths clamp to [0, capacity]
    lay, q, k, v, cur = _draw([4], [[3, 5]], 2, 1, 4, seed=6)
    a = O.decode_attention(q, k, v, lay, np.array([3, 5]), 0.5, 2, 1)
    b = O.decode_attention(q, k, v, lay, np.array([99, 7]), 0.5, 2, 1)
    c = O.decode_attention(q, k, v, lay, np.array([-4, 0]), 0.5, 2, 1)
    e = O.decode_attention(q, k, v, lay, np.array([0, 0]), 0.5, 2, 1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(c[0], e[0])
    # constant V over the key set -> o = that V; identical keys -> lse = s + ln|K|
    kk = np.broadcast_to(k[:1], k.shape).copy()
    vv = np.broadcast_to(v[:1], v.shape).copy()
    o, lse = O.decode_attention(q, kk, vv, lay, np.array([2, 3]), 0.5, 2, 1)
    assert np.abs(o - v[0, 0]).max() < 1e-14
    nkeys = np.array([4 + 2, 4 + 3])
    s = 0.5 * np.einsum("khd,d->hk", q, k[0, 0])
    assert np.abs(lse - (s + np.log(nkeys)[None, :])).max() < 1e-13


def test_decode_gqa_equals_repeated_mha():
    lay, q, k, v, cur = _draw([5, 3], [[2, 4], [6]], 8, 2, 4, seed=7)
    o, lse = O.decode_attention(q, k, v, lay, cur, 0.4, 8, 2)
    o2, lse2 = O.decode_attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), lay, cur,
                                  0.4, 8, 8)
    assert np.abs(o - o2).max() < 1e-14 and np.abs(lse - lse2).max() < 1e-14


def test_sibling_leak_fails_the_pin():
    """A plausible mistake (reading the whole group up to the own end, sibling
    rows included) fails the forward pin."""
    P, S, hq, hkv, d = CASES[0]
    lay, q, k, v, cur = _draw(P, S, hq, hkv, d, seed=1)
    scale = 1.0 / np.sqrt(d)
    lay_c, qc, kc, vc, last = _compact(lay, q, k, v, cur, hq, np.random.default_rng(2))
    of, _ = O.attention(qc, kc, vc, lay_c, scale, hq, hkv)
    bad = np.zeros_like(q)
    for kk in range(len(cur)):
        g = int(O.response_group(lay)[kk])
        a = int(lay["group_off"][g])
        end = int(lay["seg_off"][g + kk + 1]) + int(cur[kk])
        rows = np.arange(a, end)
        for h in range(hq):
            s = scale * (k[rows, h // (hq // hkv)] @ q[kk, h])
            p = np.exp(s - s.max())
            bad[kk, h] = p @ v[rows, h // (hq // hkv)] / p.sum()
    # response 0 of each group has no sibling before it; later ones do
    assert np.abs(bad - of[last]).max() > 1e-3


def test_decode_bytes_hand_derived():
    lay = O.layout([5, 9, 4], [2, 3, 0], [3, 4, 2, 6, 1])
    # prompts of groups with responses: 5 + 9; valid rows 2 + 4 + 1 + 6 + 1
    b = O.decode_bytes(lay, np.array([2, 9, 1, 6, 1]), 8, 128, 2)
    assert b == (14 + 14) * 8 * 128 * 2 * 2


def test_decode_draws_in_range():
    for i in range(5):
        w = make_workload(i)
        x = draw_decode(w)
        caps = np.asarray(w.suffix_lens)
        assert x["cur_lens"].shape == caps.shape and x["q"].shape == (len(caps), w.num_q_heads, w.head_dim)
        assert np.all(x["cur_lens"] <= caps) and np.all(x["cur_lens"] >= np.minimum(caps, 1))
    w = make_custom([3], [[0, 2]], num_q_heads=2, num_kv_heads=1, head_dim=8, dtype="f32", seed=0)
    assert list(draw_decode(w)["cur_lens"][:1]) == [0]
