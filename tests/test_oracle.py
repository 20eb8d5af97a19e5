"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each check uses hand-derived
values (tests/golden), a closed form, a library routine (torch's float64
SDPA, numpy complex arithmetic), brute force, or an invariant.
"""
import math

import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import pg_oracle as O
from workloads import make_custom, make_workload, draw_qkv, bf16_bits_to_f32, f32_to_bf16_bits

# ------------------------------------------------------------ small cases --

EDGE_SHAPES = [
    # (prefix lens, suffix lens per group)
    ([5, 9], [[3, 4], [2, 6, 1]]),
    ([0, 7], [[4, 3], [5]]),              # P = 0: block-diagonal causal
    ([6, 4, 3], [[], [0, 2], [0, 0]]),    # n = 0 and zero-length suffixes
    ([1], [[1, 1, 1]]),
    ([31, 33], [[32, 1], [63, 65]]),      # lengths straddling tile sizes
    ([0], [[0, 3, 0]]),
    ([17], [[]]),
]


def _rand_qkv(T, hq, hkv, d, seed):
    r = np.random.default_rng(seed)
    return (r.standard_normal((T, hq, d)), r.standard_normal((T, hkv, d)),
            r.standard_normal((T, hkv, d)))


def _case(shape, hq=2, hkv=1, d=16, seed=0):
    P, S = shape
    lay = O.layout(P, [len(s) for s in S], [x for s in S for x in s])
    q, k, v = _rand_qkv(lay["total_tokens"], hq, hkv, d, seed)
    return lay, q, k, v


# ------------------------------------------------------------- layout pins --

def test_tiny_layout_matches_hand_derivation():
    gold = read_golden("tiny_layout.txt")
    w = make_workload(0)
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    assert lay["group_off"].tolist() == gold["group_off"]
    assert lay["seg_off"].tolist() == gold["seg_off"]
    assert O.positions(lay).tolist() == gold["pos"]
    assert [len(O.allowed_keys(lay, t)) for t in range(30)] == gold["num_keys"]
    assert O.useful_pairs(lay) == gold["useful_pairs"][0]
    assert O.unpacked_pairs(lay) == gold["unpacked_pairs"][0]
    assert O.useful_flop(lay, 1, 64) == gold["useful_flop_d64_h1"][0]


@pytest.mark.parametrize("shape", EDGE_SHAPES)
def test_positions_equal_unpacked_sequence_positions(shape):
    # Every unpacked sequence prefix || suffix_k must see positions 0..P+S-1.
    lay, *_ = _case(shape)
    pos = O.positions(lay)
    assert pos.dtype == np.int64
    for g, p0, P, (s0, s1) in O.sequences(lay):
        seq = np.concatenate([pos[p0:p0 + P], pos[s0:s1]])
        assert seq.tolist() == list(range(P + s1 - s0))


@pytest.mark.parametrize("shape", EDGE_SHAPES)
def test_pairs_closed_form_equals_mask_count(shape):
    lay, *_ = _case(shape)
    assert O.useful_pairs(lay) == int(O.dense_mask(lay).sum())
    assert O.useful_pairs(lay) == sum(len(O.allowed_keys(lay, t)) for t in range(lay["total_tokens"]))


# ---------------------------------------------------------- attention pins --

@pytest.mark.parametrize("shape", EDGE_SHAPES)
def test_packed_definition_equals_masked_and_dense(shape):
    lay, q, k, v = _case(shape, hq=4, hkv=2, d=8, seed=len(shape[0]))
    o1, l1 = O.attention(q, k, v, lay, 0.3, 4, 2)
    o2, l2 = O.attention_masked(q, k, v, lay, 0.3, 4, 2)
    o3, l3 = O.attention_dense(q, k, v, lay, 0.3, 4, 2)
    assert np.abs(o1 - o2).max() <= 1e-10 and np.abs(l1 - l2).max() <= 1e-10
    assert np.abs(o3 - o2).max() <= 1e-12 and np.abs(l3 - l2).max() <= 1e-12


@pytest.mark.parametrize("shape", EDGE_SHAPES)
def test_against_torch_sdpa_float64(shape):
    lay, q, k, v = _case(shape, hq=2, hkv=2, d=16, seed=7)
    o, lse = O.attention(q, k, v, lay, 0.25, 2, 2)
    M = torch.from_numpy(O.dense_mask(lay))
    qt = torch.from_numpy(q).permute(1, 0, 2)    # [H, T, d]
    kt = torch.from_numpy(k).permute(1, 0, 2)
    vt = torch.from_numpy(v).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=M, scale=0.25)
    assert np.abs(ref.permute(1, 0, 2).numpy() - o).max() <= 1e-12
    s = (qt @ kt.transpose(-1, -2)) * 0.25
    ref_lse = torch.logsumexp(s.masked_fill(~M, float("-inf")), dim=-1)
    assert np.abs(ref_lse.numpy() - lse).max() <= 1e-12


def test_single_suffix_is_textbook_causal():
    # n = 1: each group is one ordinary causal sequence (library routine).
    lay, q, k, v = _case(([12, 5], [[9], [20]]), hq=2, hkv=2, d=16, seed=3)
    o, _ = O.attention(q, k, v, lay, 0.2, 2, 2)
    for g in range(2):
        a, b = int(lay["group_off"][g]), int(lay["group_off"][g + 1])
        t = lambda x: torch.from_numpy(x[a:b]).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True, scale=0.2)
        assert np.abs(ref.permute(1, 0, 2).numpy() - o[a:b]).max() <= 1e-12


def test_zero_prefix_is_independent_causal_suffixes():
    lay, q, k, v = _case(([0], [[6, 11, 4]]), hq=1, hkv=1, d=16, seed=4)
    o, _ = O.attention(q, k, v, lay, 0.2, 1, 1)
    so = lay["seg_off"]
    for i in range(1, 4):
        a, b = int(so[i]), int(so[i + 1])
        t = lambda x: torch.from_numpy(x[a:b]).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True, scale=0.2)
        assert np.abs(ref.permute(1, 0, 2).numpy() - o[a:b]).max() <= 1e-12


def test_first_token_of_group_sees_only_itself():
    lay, q, k, v = _case(([5, 9], [[3, 4], [2, 6, 1]]), hq=2, hkv=1, d=16, seed=5)
    o, lse = O.attention(q, k, v, lay, 0.5, 2, 1)
    for a in lay["group_off"][:-1]:
        for h in range(2):
            assert np.array_equal(o[a, h], v[a, 0])
            assert lse[h, a] == pytest.approx(0.5 * float(q[a, h] @ k[a, 0]), abs=1e-14)


def test_constant_values_give_constant_output():
    lay, q, k, v = _case(([5, 9], [[3, 4], [2, 6, 1]]), hq=1, hkv=1, d=16, seed=6)
    v[:] = np.linspace(-2, 3, 16)
    o, _ = O.attention(q, k, v, lay, 0.5, 1, 1)
    assert np.abs(o - v).max() <= 1e-13


def test_identical_keys_give_log_count_and_mean():
    # All keys equal: every allowed score is the same s, so lse = s + ln|K(t)|
    # and o is the plain mean of V over K(t). |K(t)| is the hand-derived count.
    gold = read_golden("tiny_layout.txt")
    lay, q, k, v = _case(([5, 9], [[3, 4], [2, 6, 1]]), hq=1, hkv=1, d=16, seed=8)
    k[:] = k[0]
    o, lse = O.attention(q, k, v, lay, 0.25, 1, 1)
    M = O.dense_mask(lay)
    for t in range(30):
        s = 0.25 * float(q[t, 0] @ k[0, 0])
        assert lse[0, t] == pytest.approx(s + math.log(gold["num_keys"][t]), abs=1e-12)
        assert np.abs(o[t, 0] - v[M[t], 0].mean(axis=0)).max() <= 1e-13


def test_gqa_equals_mha_with_repeated_kv():
    lay, q, k, v = _case(([7, 3], [[4, 2], [5]]), hq=6, hkv=2, d=8, seed=9)
    o1, l1 = O.attention(q, k, v, lay, 0.3, 6, 2)
    kr = torch.from_numpy(k).repeat_interleave(3, dim=1).numpy()
    vr = torch.from_numpy(v).repeat_interleave(3, dim=1).numpy()
    o2, l2 = O.attention(q, kr, vr, lay, 0.3, 6, 6)
    assert np.abs(o1 - o2).max() == 0 and np.abs(l1 - l2).max() == 0


def test_attention_rows_match_full_oracle():
    w = make_workload(0)
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    qkv = draw_qkv(w)
    o, lse = O.attention(qkv["q"], qkv["k"], qkv["v"], lay, w.softmax_scale, 1, 1)
    toks = list(range(30))
    oo, ll = O.attention_rows(qkv["q"], qkv["k"], qkv["v"], lay, w.softmax_scale, 1, 1, toks, [0] * 30)
    assert np.abs(oo - o[:, 0]).max() <= 1e-12 and np.abs(ll - lse[0]).max() <= 1e-12


def test_attention_rows_match_full_oracle_gqa_any_order():
    """Rows requested in any order, with repeats and several heads per token
    and KV head, equal the definition's rows."""
    lay, q, k, v = _case(([7, 3], [[4, 2], [5]]), hq=6, hkv=2, d=8, seed=21)
    o, lse = O.attention(q, k, v, lay, 0.3, 6, 2)
    T = q.shape[0]
    r = np.random.default_rng(4)
    toks = np.concatenate([np.repeat(np.arange(T), 6), r.integers(0, T, size=50)])
    heads = np.concatenate([np.tile(np.arange(6), T), r.integers(0, 6, size=50)])
    perm = r.permutation(len(toks))
    toks, heads = toks[perm], heads[perm]
    oo, ll = O.attention_rows(q, k, v, lay, 0.3, 6, 2, toks, heads)
    assert np.abs(oo - o[toks, heads]).max() <= 1e-12
    assert np.abs(ll - lse[heads, toks]).max() <= 1e-12


# ---------------------------------------------------------------- RoPE pins --

def test_rope_position_zero_is_identity():
    x = np.random.default_rng(0).standard_normal((3, 2, 16))
    assert np.array_equal(O.rope(x, np.zeros(3, dtype=np.int64), 1e4), x)


def test_rope_equals_complex_rotation():
    r = np.random.default_rng(1)
    x = r.standard_normal((40, 3, 64))
    pos = r.integers(0, 20000, size=40)
    y = O.rope(x, pos, 5e5)
    half = 32
    z = x[..., :half] + 1j * x[..., half:]
    ang = np.outer(pos, np.power(5e5, -np.arange(half) / half))
    zr = z * np.exp(1j * ang)[:, None, :]
    assert np.abs(y[..., :half] - zr.real).max() <= 1e-12
    assert np.abs(y[..., half:] - zr.imag).max() <= 1e-12


def test_rope_d2_is_plain_rotation_matrix():
    x = np.array([[[0.6, -1.1]]])
    phi = 7.0   # omega_0 = 1, so phi = pos
    y = O.rope(x, np.array([7]), 1e4)[0, 0]
    R = np.array([[math.cos(phi), -math.sin(phi)], [math.sin(phi), math.cos(phi)]])
    assert np.abs(y - R @ x[0, 0]).max() <= 1e-15


def test_rope_frequency_schedule_hand_derived():
    """The frequency schedule omega_i = theta^(-2i/d), pinned by values worked
    out by hand (no program): with d = 8 and theta = 1e4 the four pairs turn at
    1, 1e4^(-1/4) = 0.1, 1e4^(-1/2) = 0.01 and 1e4^(-3/4) = 0.001 rad per
    position; with d = 4 at 1 and 0.01; with d = 128 and theta = 5e5 pair 32
    turns at 5e5^(-1/2) = sqrt(2)/1000. Pair i is (x_i, x_{i+d/2}). A schedule
    theta^(-i/d), an interleaved pairing (x_2i, x_2i+1) or a turn by -phi all
    move some output below by far more than the 1e-12 allowed."""
    def rotated(lo, hi, a):
        return lo * math.cos(a) - hi * math.sin(a), hi * math.cos(a) + lo * math.sin(a)

    # d = 8, theta = 1e4, position 3: angles 3, 0.3, 0.03, 0.003
    x = np.array([[[1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0, 8.0]]])
    y = O.rope(x, np.array([3]), 1e4)[0, 0]
    for i, a in enumerate([3.0, 0.3, 0.03, 0.003]):
        want = rotated(x[0, 0, i], x[0, 0, i + 4], a)
        assert abs(y[i] - want[0]) <= 1e-12 and abs(y[i + 4] - want[1]) <= 1e-12
    # d = 4, theta = 1e4, position 100: angles 100 and 1
    x = np.array([[[0.5, -1.5, 2.0, 0.25]]])
    y = O.rope(x, np.array([100]), 1e4)[0, 0]
    for i, a in enumerate([100.0, 1.0]):
        want = rotated(x[0, 0, i], x[0, 0, i + 2], a)
        assert abs(y[i] - want[0]) <= 1e-12 and abs(y[i + 2] - want[1]) <= 1e-12
    # d = 128, theta = 5e5, position 1000: pair 0 turns by 1000 rad, pair 32 by sqrt(2)
    x = np.zeros((1, 1, 128))
    x[0, 0, 0], x[0, 0, 64], x[0, 0, 32], x[0, 0, 96] = 1.0, 0.0, 1.0, 0.0
    y = O.rope(x, np.array([1000]), 5e5)[0, 0]
    assert abs(y[0] - math.cos(1000.0)) <= 1e-12 and abs(y[64] - math.sin(1000.0)) <= 1e-12
    assert abs(y[32] - math.cos(math.sqrt(2.0))) <= 1e-12
    assert abs(y[96] - math.sin(math.sqrt(2.0))) <= 1e-12


def test_rope_keeps_pair_norms_and_is_relative():
    r = np.random.default_rng(2)
    q = r.standard_normal((1, 1, 32))
    k = r.standard_normal((1, 1, 32))
    yq = O.rope(q, np.array([5]), 1e4)
    lo, hi = q[..., :16], q[..., 16:]
    ylo, yhi = yq[..., :16], yq[..., 16:]
    assert np.abs((lo**2 + hi**2) - (ylo**2 + yhi**2)).max() <= 1e-13
    base = float(O.rope(q, np.array([5]), 1e4).ravel() @ O.rope(k, np.array([12]), 1e4).ravel())
    for shift in (1, 100, 3000):
        sh = float(O.rope(q, np.array([5 + shift]), 1e4).ravel() @ O.rope(k, np.array([12 + shift]), 1e4).ravel())
        assert abs(sh - base) <= 1e-12


def test_round_to_bf16_ties_and_generator_agreement():
    assert O.round_to_bf16(np.array([1 + 2.0**-8]))[0] == 1.0
    assert O.round_to_bf16(np.array([1 + 3 * 2.0**-8]))[0] == 1 + 2.0**-6
    assert O.round_to_bf16(np.array([-(1 + 3 * 2.0**-8)]))[0] == -(1 + 2.0**-6)
    x = np.random.default_rng(3).standard_normal(100000).astype(np.float32)
    ref = bf16_bits_to_f32(f32_to_bf16_bits(x)).astype(np.float64)
    assert np.array_equal(O.round_to_bf16(x.astype(np.float64)), ref)


# ---------------------------------------------------- workloads (recipes) --

def test_workload_shapes_follow_recipes():
    w1 = make_workload(1)
    assert w1.num_groups == 8 and list(w1.suffix_counts) == [2] * 8
    assert w1.prefix_lens.min() >= 256 and w1.prefix_lens.max() <= 1024
    assert w1.suffix_lens.min() >= 64 and w1.suffix_lens.max() <= 512
    w2 = make_workload(2)
    assert w2.num_groups == 16 and list(w2.suffix_counts) == [8] * 16
    assert w2.suffix_lens.min() >= 32 and w2.suffix_lens.max() <= 2048
    w3 = make_workload(3)
    assert int(w3.suffix_counts.sum()) == 19 and (w3.suffix_counts > 0).sum() + (w3.suffix_counts == 0).sum() == w3.num_groups
    assert set(w3.suffix_counts[w3.suffix_counts > 0].tolist()) <= {2, 3, 4}
    assert (w3.prefix_lens[w3.suffix_counts > 0] == 1024).all()
    assert int((w3.suffix_counts == 0).sum()) == 64 - 19
    w4 = make_workload(4)
    assert (w4.prefix_lens == 16384).all() and w4.num_q_heads == 64 and w4.num_kv_heads == 8
    assert make_workload(2).total_tokens == w2.total_tokens   # deterministic


# ----------------------------------------------------- planted mistakes ----

def test_planted_sibling_leak_is_caught(monkeypatch):
    """Dropping the sibling-suffix exclusion from the key set must break the
    equality of the masked form with the definition."""
    lay, q, k, v = _case(([5, 9], [[3, 4], [2, 6, 1]]), seed=11)

    def leaky(lay_, t):
        j = np.arange(int(lay_["g0"][t]), t + 1)
        return j
    monkeypatch.setattr(O, "allowed_keys", leaky)
    o1, _ = O.attention(q, k, v, lay, 0.3, 2, 1)
    o2, _ = O.attention_masked(q, k, v, lay, 0.3, 2, 1)
    assert np.abs(o1 - o2).max() > 1e-3


def test_planted_gqa_mapping_is_caught(monkeypatch):
    lay, q, k, v = _case(([7, 3], [[4, 2], [5]]), hq=6, hkv=2, d=8, seed=9)
    monkeypatch.setattr(O, "_kv_head", lambda h, hq, hkv: h % hkv)
    o1, _ = O.attention(q, k, v, lay, 0.3, 6, 2)
    kr = torch.from_numpy(k).repeat_interleave(3, dim=1).numpy()
    vr = torch.from_numpy(v).repeat_interleave(3, dim=1).numpy()
    o2, _ = O.attention(q, kr, vr, lay, 0.3, 6, 6)
    assert np.abs(o1 - o2).max() > 1e-3


def test_planted_rope_sign_is_caught():
    r = np.random.default_rng(1)
    x = r.standard_normal((4, 1, 8))
    pos = np.array([1, 2, 3, 4])
    y = O.rope(x, pos, 1e4)
    half = 4
    ang = np.outer(pos, np.power(1e4, -np.arange(half) / half))
    wrong_lo = x[..., :half] * np.cos(ang)[:, None] + x[..., half:] * np.sin(ang)[:, None]
    assert np.abs(wrong_lo - y[..., :half]).max() > 1e-3
