"""GPU parity of pg_attn_bwd (dQ, dK, dV) against the fp64 oracle's
``attention_backward``.

Inputs: seeded bf16 Q, K, V and upstream gradient dO (generator stream 4); the
GPU backward takes the GPU forward's O and lse, as a training step would; the
oracle recomputes everything in fp64 from Q, K, V, dO.

Tolerance (derived for bf16 operands and fp32 accumulation): per tensor,
max |gpu - ref| <= 3e-2 * max(1, max |ref|) and ||gpu - ref|| / ||ref|| <= 2e-2.
P and dS enter the matrix cores rounded to bf16 (relative 2^-9 each) and every
output is rounded to bf16 once, which alone gives about 0.3 % in relative l2.
D = rowsum(dO * O) uses the forward's bf16 O (about 0.3 % per element), and
dS = P (dP - D) cancels most on rows with few keys, where dQ itself is small:
the tiny cases reach about 1 %. A wrong index or a missing term is off by
order 100 %.

Small workloads are compared on every row; GRPO and heterogeneous on whole
groups (the oracle is dense per group, and groups are independent); the
long-prefix workload on properties that hold at any size.
"""
import sys

import numpy as np
import pytest
import torch

import shared_prefix_packed_amd as pg
from oracle import pg_oracle as O
from workloads import bf16_bits_to_f32, draw_tensor, make_custom, make_workload

pytestmark = pytest.mark.gpu

ABS_TOL = 3e-2
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
    dq, dk, dv = pg.pg_attn_bwd(L, q, k, v, o, lse, do, w.softmax_scale)
    torch.cuda.synchronize()
    return x, host(dq), host(dk), host(dv), L


def compare(name, got, ref):
    err = np.abs(got - ref)
    scale = max(1.0, float(np.abs(ref).max()))
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    say(f"    {name}: max|err| {err.max():.3e} (max|ref| {np.abs(ref).max():.3e}), rel l2 {rel:.3e}")
    assert np.isfinite(got).all()
    assert err.max() <= ABS_TOL * scale, name
    assert rel <= REL_TOL, name


def check(w, groups=None):
    x, dq, dk, dv, L = run_gpu(w)
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    q, k, v, do = (bf16_bits_to_f32(x[n]).astype(np.float64) for n in ("q", "k", "v", "do"))
    rq, rk, rv = O.attention_backward(q, k, v, do, lay, w.softmax_scale, w.num_q_heads,
                                      w.num_kv_heads, groups=groups)
    if groups is not None:
        rows = np.concatenate([np.arange(int(lay["group_off"][g]), int(lay["group_off"][g + 1]))
                               for g in groups])
        dq, dk, dv, rq, rk, rv = (a[rows] for a in (dq, dk, dv, rq, rk, rv))
    compare("dQ", dq, rq)
    compare("dK", dk, rk)
    compare("dV", dv, rv)


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
    w = make_workload(i)
    sizes = np.diff(np.asarray(O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)["group_off"]))
    groups = [int(g) for g in np.argsort(sizes)[:2]]
    say(f"backward: workload {w.name} T={w.total_tokens}, groups {groups} of sizes {sizes[groups].tolist()}")
    check(w, groups=groups)


def test_backward_long_prefix_properties():
    """At any size: rows of P sum to one, so over a group's keys dV sums to the
    group's dO (per KV head) and dK sums to zero (rows of dS sum to zero)."""
    w = make_workload(4)
    say(f"backward: workload {w.name} T={w.total_tokens} (properties)")
    x, dq, dk, dv, L = run_gpu(w)
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


def test_backward_long_prefix_sampled_dq_rows():
    """dQ rows at the long-prefix size against the oracle's per-row chain rule:
    prompt rows with up to 16K keys, response rows, every group's first and
    last prompt token and every response's last token, on random heads."""
    w = make_workload(4)
    x, dq, dk, dv, L = run_gpu(w)
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    r = np.random.default_rng(404)
    go = np.asarray(lay["group_off"])
    picks = [w.total_tokens - 1]
    for g in range(len(w.prefix_lens)):
        picks += [int(go[g]), int(go[g]) + int(w.prefix_lens[g]) - 1]
    picks += [int(t) for t in r.integers(0, w.total_tokens, size=16)]
    picks += [int(t) for t in np.nonzero(np.diff(np.asarray(lay["ss"])) != 0)[0]]   # last row of each segment
    tokens = sorted(set(picks))
    heads = [int(h) for h in r.integers(0, w.num_q_heads, size=len(tokens))]
    say(f"backward: workload {w.name} T={w.total_tokens}, {len(tokens)} sampled dQ rows")
    f = {n: _Bf16Rows(x[n]) for n in ("q", "k", "v", "do")}
    want = O.attention_backward_dq_rows(f["q"], f["k"], f["v"], f["do"], lay, w.softmax_scale,
                                        w.num_q_heads, w.num_kv_heads, tokens, heads)
    got = dq[tokens, heads]
    scale = max(1.0, np.abs(want).max())
    assert np.abs(got - want).max() <= ABS_TOL * scale, np.abs(got - want).max()
    assert np.linalg.norm(got - want) <= REL_TOL * np.linalg.norm(want)
    L.close()


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
