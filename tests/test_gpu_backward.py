"""GPU parity of pg_attn_bwd (dQ, dK, dV) against the fp64 oracle's
``attention_backward`` (dense per group) and its per-row forms
``attention_backward_dq_rows`` / ``attention_backward_kv_rows``.

Inputs: seeded bf16 Q, K, V and upstream gradient dO (generator stream 4); the
GPU backward takes the GPU forward's O and lse, as a training step would; the
oracle recomputes everything in fp64 from Q, K, V, dO.

Tolerance, derived per element. Each gradient element is a sum of terms
(dV_j: p_ij dO_i; dK_j: scale dS_ij q_i; dQ_i: scale dS_ij k_j). On the GPU
every term carries one bf16 rounding (P before the dV product, dS before the
dK and dQ products: relative error at most u = 2^-8), and D = rowsum(dO * O)
carries the bf16 rounding of O, which moves dS_ij by p_ij times a sum of
roundings of size delta_i = ||dO_i * O_i||_2; fp32 accumulation and the
forward's lse error (<= 1e-3, measured ~1e-6) are far smaller. Independent,
zero-mean rounding errors bounded by u t_i sum, by Hoeffding's inequality (the
lemma behind the probabilistic rounding error analysis of Higham and Mary,
SIAM J. Sci. Comput. 2019), to at most lambda u sqrt(sum t_i^2) except with
probability 2 exp(-lambda^2 / 2); the output's own rounding adds u |ref|:
  |gpu - ref| <= lambda u (|ref| + sqrt(sum_i t_i^2)) + 1e-6,   lambda = 8,
with t_i the magnitudes the oracle returns (|dS| widened by p delta). The worst
ratio error / bound is printed. A wrong index or a missing term is off by
order 100 % of the element, 16 times the bound. Per tensor the relative l2
error must also stay within 2 %.

Small workloads are compared on every row; GRPO and heterogeneous on whole
groups (the two smallest and a largest; groups are independent), the
long-prefix workload on sampled dQ rows and sampled dK/dV key rows (prompt
keys read by up to 21K queries of all four responses) plus properties that
hold at any size.
"""
import sys

import numpy as np
import pytest
import torch

import shared_prefix_packed_amd as pg
from oracle import pg_oracle as O
import oracle_units as U
from workloads import bf16_bits_to_f32, draw_tensor, make_custom, make_workload

pytestmark = pytest.mark.gpu

U_BF16 = 2.0 ** -8
LAMBDA = 8.0
ABS_FLOOR = 1e-6
REL_TOL = 2e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def host(t):
    return bf16_bits_to_f32(t.detach().cpu().view(torch.int16).numpy().view(np.uint16)).astype(np.float64)


def run_gpu(w):
    x = {n: draw_tensor(w, n) for n in ("q", "k", "v", "do")}
    L = pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, w.num_q_heads,
                           w.num_kv_heads, w.head_dim, w.rope_theta)
    q, k, v, do = (dev(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = pg.pg_attn_fwd(L, q, k, v, w.softmax_scale)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    pg.pg_attn_bwd(L, q, k, v, o, lse, do, w.softmax_scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return x, host(dq), host(dk), host(dv), L


def bound_of(ref, mag):
    return LAMBDA * U_BF16 * (np.abs(ref) + mag) + ABS_FLOOR


def compare(name, got, ref, mag):
    """Element-wise against the derived bound, plus relative l2. Returns the
    worst error / bound ratio."""
    assert np.isfinite(got).all(), name
    ratio = float((np.abs(got - ref) / bound_of(ref, mag)).max())
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    say(f"    {name}: max|err| {np.abs(got - ref).max():.3e}, worst err/bound {ratio:.3f}, "
        f"rel l2 {rel:.3e}")
    assert ratio <= 1.0, name
    assert rel <= REL_TOL, name
    return ratio


def check(w, groups=None):
    """Every row (groups None, dense oracle in one call) or every row of the
    given groups (oracle per (group, KV head) unit in parallel)."""
    x, dq, dk, dv, L = run_gpu(w)
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    f = {n: bf16_bits_to_f32(x[n]) for n in ("q", "k", "v", "do")}
    if groups is None:
        rq, rk, rv, mags = O.attention_backward(*(f[n].astype(np.float64) for n in ("q", "k", "v", "do")),
                                                lay, w.softmax_scale, w.num_q_heads,
                                                w.num_kv_heads, magnitudes=True)
        compare("dQ", dq, rq, mags["dq"])
        compare("dK", dk, rk, mags["dk"])
        compare("dV", dv, rv, mags["dv"])
        return
    r = w.num_q_heads // w.num_kv_heads
    got = {"dQ": [], "dK": [], "dV": []}
    want = {"dQ": [], "dK": [], "dV": []}
    mag = {"dQ": [], "dK": [], "dV": []}
    for g, hk, a, b, rq, rk, rv, m in U.backward_units(w, lay, f["q"], f["k"], f["v"], f["do"],
                                                       set(groups)):
        got["dQ"].append(dq[a:b, hk * r:(hk + 1) * r]); want["dQ"].append(rq); mag["dQ"].append(m["dq"])
        got["dK"].append(dk[a:b, hk]); want["dK"].append(rk); mag["dK"].append(m["dk"])
        got["dV"].append(dv[a:b, hk]); want["dV"].append(rv); mag["dV"].append(m["dv"])
    for name in ("dQ", "dK", "dV"):
        compare(name, *(np.concatenate([a.reshape(-1) for a in d[name]]) for d in (got, want, mag)))


EDGE = [
    ([5, 9], [[3, 4], [2, 6, 1]], 4, 1),
    ([0, 7], [[4, 3], [5]], 8, 2),
    ([6, 4, 3], [[], [0, 2], [0, 0]], 4, 4),
    ([1], [[1, 1, 1]], 2, 1),
    ([31, 33, 64], [[32, 1], [63, 65], [128, 129, 127]], 8, 1),
    ([300], [[1, 40, 0, 200, 33]], 6, 2),
    ([130, 257], [[130, 7], [300]], 16, 2),
    ([0], [[0, 3, 0]], 3, 1),
]


@pytest.mark.parametrize("case", range(len(EDGE)))
def test_backward_edge_shapes(case):
    P, S, hq, hkv = EDGE[case]
    w = make_custom(P, S, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, dtype="bf16", seed=case)
    say(f"backward edge case {case}: P={P} S={S} heads={hq}/{hkv}")
    check(w)


def test_backward_dpo_workload():
    w = make_workload(1)
    say(f"backward: workload {w.name} T={w.total_tokens}")
    check(w)


@pytest.mark.parametrize("i", [2, 3])
def test_backward_large_workloads_on_whole_groups(i):
    """Every row of every group: all 16 groups of GRPO (up to 7.5K tokens,
    eight responses on one prompt) and all 52 of the heterogeneous workload
    (up to one 10.7K-token shared group). The dense per-group oracle holds
    about 8 GB per (group, KV head) unit at 10.7K tokens, eight units at a
    time."""
    w = make_workload(i)
    sizes = np.diff(np.asarray(O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)["group_off"]))
    groups = [g for g in range(len(sizes)) if 0 < sizes[g] <= 12288]
    say(f"backward: workload {w.name} T={w.total_tokens}, {len(groups)} of {len(sizes)} groups, "
        f"largest {int(sizes[groups].max())} tokens")
    check(w, groups=groups)


def test_backward_long_prefix_properties():
    """At any size: rows of P sum to one, so over a group's keys dV sums to the
    group's dO (per KV head) and dK sums to zero (rows of dS sum to zero)."""
    run = long_prefix_run()
    w, x, dq, dk, dv = run["w"], run["x"], run["dq"], run["dk"], run["dv"]
    say(f"backward: workload {w.name} T={w.total_tokens} (properties)")
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    do = bf16_bits_to_f32(x["do"]).astype(np.float64)
    r = w.num_q_heads // w.num_kv_heads
    for g in range(len(w.prefix_lens)):
        a, b = int(lay["group_off"][g]), int(lay["group_off"][g + 1])
        for hk in range(w.num_kv_heads):
            want = do[a:b, hk * r:(hk + 1) * r].sum(axis=(0, 1))
            got = dv[a:b, hk].sum(axis=0)
            assert np.abs(got - want).max() <= 1e-2 * max(1.0, np.abs(want).max()) + 0.5
            ksum = dk[a:b, hk].sum(axis=0)
            assert np.abs(ksum).max() <= 1e-2 * np.abs(dk[a:b, hk]).sum(axis=0).max() + 1e-3
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()


def test_backward_returns_d_in_delta():
    """delta holds D = rowsum(dO * O) of every (head, token) row on return.
    The GPU forms D from its bf16 O, whose error against the fp64 O is at
    most 2^-9 |O_d| (rounding to bf16) plus 2^-9 sum_j p_j |v_jd| (P rounded
    to bf16 before the PV product; that sum is attention over |V|), so per row
      |D_gpu - D_ref| <= 2^-8 sum_d |dO_d| (|O_d| + sum_j p_j |v_jd|) + 1e-5,
    and over all rows the relative l2 error stays within the module's 2 %."""
    w = make_workload(1)
    x = {n: draw_tensor(w, n) for n in ("q", "k", "v", "do")}
    L = pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, w.num_q_heads,
                           w.num_kv_heads, w.head_dim, w.rope_theta)
    q, k, v, do = (dev(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = pg.pg_attn_fwd(L, q, k, v, w.softmax_scale)
    delta = torch.full((w.num_q_heads, w.total_tokens), float("nan"), dtype=torch.float32, device="cuda")
    pg.pg_attn_bwd(L, q, k, v, o, lse, do, w.softmax_scale, delta=delta)
    torch.cuda.synchronize()
    got = delta.cpu().numpy().astype(np.float64)
    f = {n: bf16_bits_to_f32(x[n]).astype(np.float64) for n in ("q", "k", "v", "do")}
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    o_ref, _ = O.attention(f["q"], f["k"], f["v"], lay, w.softmax_scale, w.num_q_heads, w.num_kv_heads)
    want = (f["do"] * o_ref).sum(axis=2).T                                  # [Hq, T]
    o_abs, _ = O.attention(f["q"], f["k"], np.abs(f["v"]), lay, w.softmax_scale, w.num_q_heads,
                           w.num_kv_heads)                                 # sum_j p_j |v_j|
    bound = 2.0 ** -8 * (np.abs(f["do"]) * (np.abs(o_ref) + o_abs)).sum(axis=2).T + 1e-5
    say(f"delta: {w.name}, worst |D_gpu - D_ref| / bound = {(np.abs(got - want) / bound).max():.3f}")
    assert np.isfinite(got).all()
    assert (np.abs(got - want) <= bound).all()
    assert np.linalg.norm(got - want) <= REL_TOL * np.linalg.norm(want)
    L.close()


class _Bf16Rows:
    """bf16 bit array read as float32 only where indexed (the oracle's per-row
    functions touch a few rows of tensors too large to widen whole)."""

    def __init__(self, bits):
        self.bits = bits
        self.shape = bits.shape

    def __getitem__(self, idx):
        return bf16_bits_to_f32(self.bits[idx])


_long = {}


def long_prefix_run():
    """The long-prefix backward on the GPU, once for the tests below."""
    if not _long:
        w = make_workload(4)
        x, dq, dk, dv, L = run_gpu(w)
        L.close()
        _long.update(w=w, x=x, dq=dq, dk=dk, dv=dv)
    return _long


def test_backward_long_prefix_sampled_dq_rows():
    """dQ rows at the long-prefix size against the oracle's per-row chain rule:
    prompt rows with up to 16K keys, response rows, every group's first and
    last prompt token and every response's last token, on random heads."""
    run = long_prefix_run()
    w, x, dq = run["w"], run["x"], run["dq"]
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    r = np.random.default_rng(404)
    go = np.asarray(lay["group_off"])
    picks = [w.total_tokens - 1]
    for g in range(len(w.prefix_lens)):
        picks += [int(go[g]), int(go[g]) + int(w.prefix_lens[g]) - 1]
    picks += [int(t) for t in r.integers(0, w.total_tokens, size=2048)]
    picks += [int(t) for t in np.nonzero(np.diff(np.asarray(lay["ss"])) != 0)[0]]   # last row of each segment
    tokens = sorted(set(picks))
    heads = [int(h) for h in r.integers(0, w.num_q_heads, size=len(tokens))]
    say(f"backward: workload {w.name} T={w.total_tokens}, {len(tokens)} sampled dQ rows")
    f = {n: _Bf16Rows(x[n]) for n in ("q", "k", "v", "do")}
    want, mag = O.attention_backward_dq_rows(f["q"], f["k"], f["v"], f["do"], lay, w.softmax_scale,
                                             w.num_q_heads, w.num_kv_heads, tokens, heads,
                                             magnitudes=True)
    compare("dQ rows", dq[tokens, heads], want, mag)


def test_backward_long_prefix_sampled_kv_rows():
    """dK and dV key rows at the long-prefix size against the oracle's per-key
    chain rule, on one (group, KV head): prompt keys, each read by every later
    prompt token and by all four responses (up to 21K query rows x 8 query
    heads), at the prompt's first and last rows, at 64-row block edges and at
    random; response keys at each response's first and last rows and at
    random. The forward's o and lse the chain rule needs come from the oracle
    (per query head, in parallel) on that group alone."""
    run = long_prefix_run()
    w, x, dk, dv = run["w"], run["x"], run["dk"], run["dv"]
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    r = w.num_q_heads // w.num_kv_heads
    g, hk = len(w.prefix_lens) - 1, 5
    (_, a, b, sub), = [u for u in U.group_layouts(w, lay) if u[0] == g]
    f = {n: _Bf16Rows(x[n]) for n in ("q", "k", "v", "do")}
    q, k = U.kv_head_slices(f["q"], f["k"], hk, r, a, b)
    do, v = U.kv_head_slices(f["do"], f["v"], hk, r, a, b)
    say(f"backward: workload {w.name}, oracle forward of group {g} ({b - a} tokens), KV head {hk}")
    o, lse = U.attention_heads(sub, q, k, v, w.softmax_scale)
    P = int(w.prefix_lens[g])
    rng = np.random.default_rng(405)
    keys = {0, 1, 63, 64, 127, 128, P // 2, P - 65, P - 64, P - 2, P - 1}
    keys |= {int(t) for t in rng.integers(0, P, size=512)}
    seg = np.asarray(sub["seg_off"])
    for j in range(1, len(seg) - 1):
        s0, s1 = int(seg[j]), int(seg[j + 1])
        if s1 > s0:
            keys |= {s0, s0 + 1, s1 - 1} | {int(t) for t in rng.integers(s0, s1, size=48)}
    keys = sorted(keys)
    say(f"  {len(keys)} sampled key rows")
    rk, rv, mk, mv = O.attention_backward_kv_rows(q, k, v, do, sub, w.softmax_scale, r, 1, keys,
                                                  [0] * len(keys), o=o, lse=lse, magnitudes=True)
    rows = [a + j for j in keys]
    compare("dK rows", dk[rows, hk], rk, mk)
    compare("dV rows", dv[rows, hk], rv, mv)


def test_backward_one_long_group():
    """One 65.5K-token group (a 60000-token prompt, responses of 3000, 1 and
    2500 tokens, 8 query heads on one KV head): every dQ, dK, dV element
    written and finite; sampled dQ rows (prompt and response edges, random)
    against the oracle's per-row chain rule; over the group's keys dV sums to
    its dO and dK to zero."""
    w = make_custom([60000], [[3000, 1, 2500]], num_q_heads=8, num_kv_heads=1, head_dim=128,
                    dtype="bf16", seed=7)
    x, dq, dk, dv, L = run_gpu(w)
    L.close()
    T = w.total_tokens
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    r = np.random.default_rng(707)
    tokens = {0, 1, 64, 59999, 60000, 62999, 63000, 63001, T - 1}
    tokens = sorted(tokens | {int(t) for t in r.integers(0, T, size=120)})
    heads = [int(h) for h in r.integers(0, w.num_q_heads, size=len(tokens))]
    say(f"backward: one long group, T={T}, {len(tokens)} sampled dQ rows")
    f = {n: _Bf16Rows(x[n]) for n in ("q", "k", "v", "do")}
    want, mag = O.attention_backward_dq_rows(f["q"], f["k"], f["v"], f["do"], lay, w.softmax_scale,
                                             w.num_q_heads, w.num_kv_heads, tokens, heads,
                                             magnitudes=True)
    compare("dQ rows", dq[tokens, heads], want, mag)
    assert np.isfinite(dk).all() and np.isfinite(dv).all()
    do = bf16_bits_to_f32(x["do"]).astype(np.float64)
    want_v = do.sum(axis=(0, 1))
    assert np.abs(dv[:, 0].sum(axis=0) - want_v).max() <= 1e-2 * max(1.0, np.abs(want_v).max()) + 0.5
    assert np.abs(dk[:, 0].sum(axis=0)).max() <= 1e-2 * np.abs(dk[:, 0]).sum(axis=0).max() + 1e-3


def test_backward_deterministic_and_fully_written():
    w = make_workload(1)
    x = {n: draw_tensor(w, n) for n in ("q", "k", "v", "do")}
    L = pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, w.num_q_heads,
                           w.num_kv_heads, w.head_dim, w.rope_theta)
    q, k, v, do = (dev(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = pg.pg_attn_fwd(L, q, k, v, w.softmax_scale)
    outs = []
    for fill in (float("nan"), float("inf")):
        dq = torch.full_like(q, fill)
        dk = torch.full_like(k, fill)
        dv = torch.full_like(v, fill)
        pg.pg_attn_bwd(L, q, k, v, o, lse, do, w.softmax_scale, dq=dq, dk=dk, dv=dv)
        outs.append((dq, dk, dv))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.isfinite(a.float()).all()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
