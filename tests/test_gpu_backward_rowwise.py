"""GPU parity of pg_attn_bwd's per-row path (fp32, and bf16 with d = 64)
against the fp64 oracle's ``attention_backward``, on every row.

fp32: the kernels compute in fp32 from fp32 inputs, so the error against the
fp64 oracle is fp32 rounding: each term of a gradient sum carries a few
roundings (the exponential, the dot products, the product), independent and
zero-mean, so by the same Hoeffding argument as the bf16 bound the error
stays below 64 u32 (|ref| + root sum of squares of the terms) (lambda = 8,
eight roundings' worth, u32 = 2^-24), on top of a 1e-5 absolute floor. The
tiny workload (two groups, head size 64, the hand-derived layout) has its
forward and backward both on this path.

bf16, d = 64: inputs and outputs in bf16, arithmetic in fp32; held to the
per-element bound of the MFMA backward's tests (lambda u (|ref| + root sum of
squares of the terms) + 1e-6, u = 2^-8, lambda = 8), which this path meets
with room to spare (it rounds only its outputs).
"""
import sys

import numpy as np
import pytest
import torch

import shared_prefix_packed_amd as pg
from oracle import pg_oracle as O
from workloads import bf16_bits_to_f32, draw_tensor, make_custom, make_workload

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(w, a):
    if w.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def host(w, t):
    t = t.detach().cpu()
    if w.dtype == "f32":
        return t.numpy().astype(np.float64)
    return bf16_bits_to_f32(t.view(torch.int16).numpy().view(np.uint16)).astype(np.float64)


def vals(w, a):
    return (a if w.dtype == "f32" else bf16_bits_to_f32(a)).astype(np.float64)


def run(w):
    x = {n: draw_tensor(w, n) for n in ("q", "k", "v", "do")}
    L = pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, w.num_q_heads,
                           w.num_kv_heads, w.head_dim, w.rope_theta)
    q, k, v, do = (dev(w, x[n]) for n in ("q", "k", "v", "do"))
    o, lse = pg.pg_attn_fwd(L, q, k, v, w.softmax_scale)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    delta = torch.full((w.num_q_heads, w.total_tokens), float("nan"), device="cuda")
    pg.pg_attn_bwd(L, q, k, v, o, lse, do, w.softmax_scale, dq=dq, dk=dk, dv=dv, delta=delta)
    torch.cuda.synchronize()
    got = (host(w, dq), host(w, dk), host(w, dv), delta.cpu().numpy().astype(np.float64),
           host(w, o))
    L.close()
    return x, got


def check(w):
    x, (dq, dk, dv, delta, o) = run(w)
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    f = {n: vals(w, x[n]) for n in ("q", "k", "v", "do")}
    rq, rk, rv, mags = O.attention_backward(f["q"], f["k"], f["v"], f["do"], lay, w.softmax_scale,
                                            w.num_q_heads, w.num_kv_heads, magnitudes=True)
    for name, got, ref, mag in (("dQ", dq, rq, mags["dq"]), ("dK", dk, rk, mags["dk"]),
                                ("dV", dv, rv, mags["dv"])):
        assert np.isfinite(got).all(), name
        err = np.abs(got - ref)
        if w.dtype == "f32":
            bound = F32_TOL + 64 * 2.0 ** -24 * (np.abs(ref) + mag)
            say(f"    {name}: max|err| {err.max():.3e} (max|ref| {np.abs(ref).max():.2e}), "
                f"worst err/bound {(err / bound).max():.3f}")
            assert (err <= bound).all(), name
        else:
            bound = 8.0 * 2.0 ** -8 * (np.abs(ref) + mag) + 1e-6
            say(f"    {name}: max|err| {err.max():.3e}, worst err/bound {(err / bound).max():.3f}")
            assert (err <= bound).all(), name
    # delta holds D = rowsum(dO * O) of the forward's O as handed over
    want_d = (f["do"] * o).sum(axis=2).T
    assert np.abs(delta - want_d).max() <= 1e-5 * max(1.0, np.abs(want_d).max())


def test_tiny_fp32_workload_forward_and_backward():
    w = make_workload(0)
    say(f"per-row backward: workload {w.name} (fp32, d = 64)")
    check(w)


EDGE = [
    ([5, 9], [[3, 4], [2, 6, 1]], 4, 1),
    ([0, 7], [[4, 3], [5]], 8, 2),
    ([6, 4, 3], [[], [0, 2], [0, 0]], 4, 4),
    ([1], [[1, 1, 1]], 2, 1),
    ([31, 33, 64], [[32, 1], [63, 65], [128, 129, 127]], 8, 1),
    ([300], [[1, 40, 0, 200, 33]], 6, 2),
    ([0], [[0, 3, 0]], 3, 1),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", range(len(EDGE)))
def test_fp32_edge_shapes(case, d):
    P, S, hq, hkv = EDGE[case]
    w = make_custom(P, S, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype="f32", seed=case)
    say(f"per-row backward fp32 d={d} case {case}: P={P} S={S} heads={hq}/{hkv}")
    check(w)


@pytest.mark.parametrize("case", range(len(EDGE)))
def test_bf16_d64_edge_shapes(case):
    P, S, hq, hkv = EDGE[case]
    w = make_custom(P, S, num_q_heads=hq, num_kv_heads=hkv, head_dim=64, dtype="bf16", seed=case)
    say(f"per-row backward bf16 d=64 case {case}: P={P} S={S} heads={hq}/{hkv}")
    check(w)


def test_rowwise_backward_is_deterministic():
    w = make_custom([37, 80], [[20, 9], [64]], num_q_heads=4, num_kv_heads=2, head_dim=64,
                    dtype="f32", seed=5)
    _, a = run(w)
    _, b = run(w)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
