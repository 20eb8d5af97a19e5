"""Pins of the oracle's backward (``attention_backward``) against things other
than itself: finite differences of the forward, torch's float64 SDPA autograd
on the unpacked sequences, and closed forms. CPU only."""
import numpy as np
import pytest
import torch

from oracle import pg_oracle as O
from workloads import draw_qkv, make_custom, make_workload

CASES = [
    ([3, 0], [[2, 1], [2]], 2, 1, 4),      # prompt-less group, two responses
    ([4], [[3, 0, 2]], 4, 2, 8),           # empty response in the middle, GQA 2
    ([1, 2], [[1, 1, 1], []], 3, 3, 4),    # one-token prompt, response-less group
]


def _inputs(P, S, hq, hkv, d, seed=0):
    w = make_custom(P, S, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype="f32", seed=seed)
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    x = draw_qkv(w)
    r = np.random.default_rng(100 + seed)
    do = r.standard_normal(x["q"].shape)
    return w, lay, x["q"].astype(np.float64), x["k"].astype(np.float64), x["v"].astype(np.float64), do


def _loss(q, k, v, do, lay, w):
    o, _ = O.attention(q, k, v, lay, w.softmax_scale, w.num_q_heads, w.num_kv_heads)
    return float((o * do).sum())


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_finite_differences(case):
    w, lay, q, k, v, do = _inputs(*case)
    dq, dk, dv = O.attention_backward(q, k, v, do, lay, w.softmax_scale, w.num_q_heads, w.num_kv_heads)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            xp = x.copy(); xp[i] += eps
            xm = x.copy(); xm[i] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, lay, w)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, lay, w)
            num[i] = (lp - lm) / (2 * eps)
        assert np.abs(num - g).max() <= 1e-6 * max(1.0, np.abs(g).max()), name


def _torch_unpacked_grads(w, lay, q, k, v, do):
    """Gradients by torch's float64 SDPA autograd over the unpacked sequences.
    Prompt tensors are shared leaves (so their K/V gradients sum over the
    responses); the prompt rows' output gradient is routed to the first
    sequence of the group only, because the packed batch holds those rows
    once."""
    Hq, Hkv = w.num_q_heads, w.num_kv_heads
    r = Hq // Hkv
    T, _, d = q.shape
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    tdo = torch.tensor(do)
    loss = 0.0
    seen = set()
    for g, p0, P, (s0, s1) in O.sequences(lay):
        idx = torch.tensor(list(range(p0, p0 + P)) + list(range(s0, s1)), dtype=torch.long)
        if len(idx) == 0:
            continue
        qs = tq[idx].transpose(0, 1)                              # [Hq, L, d]
        ks = tk[idx].transpose(0, 1).repeat_interleave(r, dim=0)  # [Hq, L, d]
        vs = tv[idx].transpose(0, 1).repeat_interleave(r, dim=0)
        o = torch.nn.functional.scaled_dot_product_attention(
            qs.unsqueeze(0), ks.unsqueeze(0), vs.unsqueeze(0), is_causal=True,
            scale=w.softmax_scale)[0].transpose(0, 1)             # [L, Hq, d]
        weight = torch.ones(len(idx), 1, 1, dtype=torch.float64)
        if g in seen:
            weight[:P] = 0.0
        seen.add(g)
        loss = loss + (o * tdo[idx] * weight).sum()
    loss.backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_torch_on_unpacked_sequences(case):
    w, lay, q, k, v, do = _inputs(*case, seed=3)
    dq, dk, dv = O.attention_backward(q, k, v, do, lay, w.softmax_scale, w.num_q_heads, w.num_kv_heads)
    rq, rk, rv = _torch_unpacked_grads(w, lay, q, k, v, do)
    assert np.abs(dq - rq).max() < 1e-10
    assert np.abs(dk - rk).max() < 1e-10
    assert np.abs(dv - rv).max() < 1e-10


def test_backward_matches_torch_on_tiny_workload():
    w = make_workload(0)
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    x = draw_qkv(w)
    q, k, v = (x[n].astype(np.float64) for n in ("q", "k", "v"))
    do = np.random.default_rng(7).standard_normal(q.shape)
    dq, dk, dv = O.attention_backward(q, k, v, do, lay, w.softmax_scale, w.num_q_heads, w.num_kv_heads)
    rq, rk, rv = _torch_unpacked_grads(w, lay, q, k, v, do)
    for a, b in ((dq, rq), (dk, rk), (dv, rv)):
        assert np.abs(a - b).max() < 1e-10


def test_backward_closed_forms():
    w, lay, q, k, v, do = _inputs([5, 2], [[3, 4], [1, 2]], 4, 2, 8, seed=5)
    dq, dk, dv = O.attention_backward(q, k, v, do, lay, w.softmax_scale, w.num_q_heads, w.num_kv_heads)
    r = w.num_q_heads // w.num_kv_heads
    # rows of P sum to one: summed over keys, dV equals dO summed over queries
    for hk in range(w.num_kv_heads):
        assert np.allclose(dv[:, hk].sum(axis=0), do[:, hk * r:(hk + 1) * r].sum(axis=(0, 1)), atol=1e-12)
    # a group's first token sees only itself: P = 1, dS = 0
    for g in range(2):
        assert np.abs(dq[int(lay["group_off"][g])]).max() < 1e-12
    # the same V for every key: O does not depend on the scores at all
    vc = np.broadcast_to(v[:1], v.shape).copy()
    dq2, dk2, _ = O.attention_backward(q, k, vc, do, lay, w.softmax_scale, w.num_q_heads, w.num_kv_heads)
    assert np.abs(dq2).max() < 1e-12 and np.abs(dk2).max() < 1e-12


@pytest.mark.parametrize("case", CASES + [([6, 3], [[4, 0, 5], [2, 3]], 8, 2, 16)])
def test_dq_rows_equal_the_dense_backward(case):
    """The per-row dQ (used at full size) equals the dense per-group backward,
    which finite differences and torch autograd pin, on every (token, head)."""
    P, S, hq, hkv, d = case
    w, lay, q, k, v, do = _inputs(P, S, hq, hkv, d, seed=11)
    dq, _, _ = O.attention_backward(q, k, v, do, lay, w.softmax_scale, hq, hkv)
    T = q.shape[0]
    tokens = np.repeat(np.arange(T), hq)
    heads = np.tile(np.arange(hq), T)
    rows = O.attention_backward_dq_rows(q, k, v, do, lay, w.softmax_scale, hq, hkv, tokens, heads)
    assert np.abs(rows - dq[tokens, heads]).max() <= 1e-12 * max(1.0, np.abs(dq).max())


def test_dq_rows_closed_forms():
    w, lay, q, k, v, do = _inputs([5, 2], [[3, 4], [1, 2]], 4, 2, 8, seed=6)
    T, hq = q.shape[0], w.num_q_heads
    tokens = np.repeat(np.arange(T), hq)
    heads = np.tile(np.arange(hq), T)
    # the same V for every key: the output does not depend on the scores
    vc = np.broadcast_to(v[:1], v.shape).copy()
    rows = O.attention_backward_dq_rows(q, k, vc, do, lay, w.softmax_scale, hq, w.num_kv_heads,
                                        tokens, heads)
    assert np.abs(rows).max() < 1e-12
    # a group's first token has one key: P = 1, so dS = dp - D = 0
    firsts = [int(lay["group_off"][g]) for g in range(2)]
    rows = O.attention_backward_dq_rows(q, k, v, do, lay, w.softmax_scale, hq, w.num_kv_heads,
                                        [t for t in firsts for _ in range(hq)], list(range(hq)) * 2)
    assert np.abs(rows).max() < 1e-12
    # a row with several keys does get a gradient
    last = O.attention_backward_dq_rows(q, k, v, do, lay, w.softmax_scale, hq, w.num_kv_heads, [T - 1], [0])
    assert np.abs(last).max() > 1e-3


@pytest.mark.parametrize("case", CASES + [([6, 3], [[4, 0, 5], [2, 3]], 8, 2, 16)])
def test_kv_rows_equal_the_dense_backward(case):
    """The per-key dK/dV (used at full size, where a prompt key is read by
    every response of its group) equals the dense per-group backward, which
    finite differences and torch autograd pin, on every (key, KV head)."""
    P, S, hq, hkv, d = case
    w, lay, q, k, v, do = _inputs(P, S, hq, hkv, d, seed=12)
    _, dk, dv = O.attention_backward(q, k, v, do, lay, w.softmax_scale, hq, hkv)
    T = q.shape[0]
    keys = np.repeat(np.arange(T), hkv)
    kvh = np.tile(np.arange(hkv), T)
    rk, rv = O.attention_backward_kv_rows(q, k, v, do, lay, w.softmax_scale, hq, hkv, keys, kvh)
    tol = 1e-12 * max(1.0, np.abs(dk).max(), np.abs(dv).max())
    assert np.abs(rk - dk[keys, kvh]).max() <= tol
    assert np.abs(rv - dv[keys, kvh]).max() <= tol
    # the forward's o and lse handed in give the same rows
    o, lse = O.attention(q, k, v, lay, w.softmax_scale, hq, hkv)
    rk2, rv2 = O.attention_backward_kv_rows(q, k, v, do, lay, w.softmax_scale, hq, hkv, keys, kvh,
                                            o=o, lse=lse)
    assert np.array_equal(rk, rk2) and np.array_equal(rv, rv2)


def test_kv_rows_closed_forms():
    w, lay, q, k, v, do = _inputs([5, 2], [[3, 4], [1, 2]], 4, 2, 8, seed=7)
    T, hq, hkv = q.shape[0], w.num_q_heads, w.num_kv_heads
    r = hq // hkv
    keys = np.repeat(np.arange(T), hkv)
    kvh = np.tile(np.arange(hkv), T)
    dk, dv = O.attention_backward_kv_rows(q, k, v, do, lay, w.softmax_scale, hq, hkv, keys, kvh)
    dk = dk.reshape(T, hkv, -1)
    dv = dv.reshape(T, hkv, -1)
    for g in range(2):
        a, b = int(lay["group_off"][g]), int(lay["group_off"][g + 1])
        for hk in range(hkv):
            # rows of P sum to one: over a group's keys dV sums to its dO
            assert np.allclose(dv[a:b, hk].sum(axis=0), do[a:b, hk * r:(hk + 1) * r].sum(axis=(0, 1)),
                               atol=1e-12)
            # rows of dS sum to zero: over a group's keys dK sums to zero
            assert np.abs(dk[a:b, hk].sum(axis=0)).max() < 1e-12
    # the same V for every key: no gradient reaches K
    vc = np.broadcast_to(v[:1], v.shape).copy()
    dk2, _ = O.attention_backward_kv_rows(q, k, vc, do, lay, w.softmax_scale, hq, hkv, keys, kvh)
    assert np.abs(dk2).max() < 1e-12


def test_backward_magnitudes_agree_across_forms():
    """The per-element term magnitudes (root sum of squares of the terms of
    each gradient sum, used to scale GPU tolerances) are the same in the dense
    form and in the per-row forms, and bound each sum by Cauchy-Schwarz:
    |sum of n terms| <= sqrt(n) * root sum of squares."""
    P, S, hq, hkv, d = [6, 3], [[4, 0, 5], [2, 3]], 8, 2, 16
    w, lay, q, k, v, do = _inputs(P, S, hq, hkv, d, seed=13)
    dq, dk, dv, mags = O.attention_backward(q, k, v, do, lay, w.softmax_scale, hq, hkv, magnitudes=True)
    T = q.shape[0]
    tokens = np.repeat(np.arange(T), hq)
    heads = np.tile(np.arange(hq), T)
    _, mq = O.attention_backward_dq_rows(q, k, v, do, lay, w.softmax_scale, hq, hkv, tokens, heads,
                                         magnitudes=True)
    assert np.abs(mq - mags["dq"][tokens, heads]).max() <= 1e-12 * np.abs(mq).max()
    keys = np.repeat(np.arange(T), hkv)
    kvh = np.tile(np.arange(hkv), T)
    _, _, mk, mv = O.attention_backward_kv_rows(q, k, v, do, lay, w.softmax_scale, hq, hkv, keys,
                                                kvh, magnitudes=True)
    assert np.abs(mk - mags["dk"][keys, kvh]).max() <= 1e-12 * np.abs(mk).max()
    assert np.abs(mv - mags["dv"][keys, kvh]).max() <= 1e-12 * np.abs(mv).max()
    n = T * hq   # more terms than any sum has
    for g, m in ((dq, mags["dq"]), (dk, mags["dk"]), (dv, mags["dv"])):
        assert (np.abs(g) <= np.sqrt(n) * m + 1e-12).all()
        assert (m >= 0).all() and m.max() > 0


def test_finite_differences_catch_a_dropped_term():
    """A plausible mistake (dS = P dP, the D term dropped) fails the pin."""
    w, lay, q, k, v, do = _inputs(*CASES[0])
    dq, _, _ = O.attention_backward(q, k, v, do, lay, w.softmax_scale, w.num_q_heads, w.num_kv_heads)
    # the mistaken gradient, rebuilt from the same pieces without the D term
    bad = np.zeros_like(dq)
    for g in range(len(lay["prefix_lens"])):
        a, b = int(lay["group_off"][g]), int(lay["group_off"][g + 1])
        if b == a:
            continue
        M = O.group_mask(lay, g)
        for h in range(w.num_q_heads):
            hk = h // (w.num_q_heads // w.num_kv_heads)
            s = np.where(M, w.softmax_scale * (q[a:b, h] @ k[a:b, hk].T), -np.inf)
            P = np.exp(s - s.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            bad[a:b, h] = w.softmax_scale * ((P * (do[a:b, h] @ v[a:b, hk].T)) @ k[a:b, hk])
    eps = 1e-6
    num = np.zeros_like(q)
    it = np.nditer(q, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp = q.copy(); xp[i] += eps
        xm = q.copy(); xm[i] -= eps
        num[i] = (_loss(xp, k, v, do, lay, w) - _loss(xm, k, v, do, lay, w)) / (2 * eps)
    assert np.abs(num - dq).max() < 1e-6
    assert np.abs(num - bad).max() > 1e-3


def test_backward_flop_count():
    w = make_workload(0)
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    # 217 allowed pairs (hand-derived), d = 64, one query head
    assert O.backward_flop(lay, 64, 1) == 10 * 64 * 217
