"""Two layouts used at once from two streams and two host threads.

Layout A (DPO-shaped) and layout B (a small custom batch) are built and
uploaded from two Python threads at the same time, each on its own stream.
Then the forward of A runs on one stream while the forward and backward of B
run on the other, three times over. Every output must equal, bit for bit,
what the same calls give one after another on a single stream. The kernels
use no atomics, so the results do not depend on how the two streams
interleave.
"""
import threading

import numpy as np
import pytest
import torch

import shared_prefix_packed_amd as pg
from workloads import draw_tensor, make_custom, make_workload

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def test_two_streams_two_threads_match_sequential():
    wa = make_workload(1)
    wb = make_custom([300, 90], [[120, 64, 7], [200]], num_q_heads=16, num_kv_heads=4,
                     head_dim=128, dtype="bf16", seed=21)
    print(f"streams: A {wa.name} T={wa.total_tokens}, B T={wb.total_tokens}", flush=True)
    ta = {n: dev(draw_tensor(wa, n)) for n in ("q", "k", "v")}
    tb = {n: dev(draw_tensor(wb, n)) for n in ("q", "k", "v", "do")}

    def args(w):
        return (w.prefix_lens, w.suffix_counts, w.suffix_lens, w.num_q_heads, w.num_kv_heads,
                w.head_dim, w.rope_theta)

    # sequential reference on the current stream
    La = pg.pg_build_layout(*args(wa))
    Lb = pg.pg_build_layout(*args(wb))
    oa, la = pg.pg_attn_fwd(La, ta["q"], ta["k"], ta["v"], wa.softmax_scale)
    ob, lb = pg.pg_attn_fwd(Lb, tb["q"], tb["k"], tb["v"], wb.softmax_scale)
    gb = pg.pg_attn_bwd(Lb, tb["q"], tb["k"], tb["v"], ob, lb, tb["do"], wb.softmax_scale)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (oa, la, ob, lb) + tuple(gb)]
    La.close()
    Lb.close()

    # layouts built concurrently, each uploaded on its own stream
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    built, errors = {}, []

    def build(name, w, s):
        try:
            built[name] = pg.pg_build_layout(*args(w), stream=s)
        except Exception as e:   # reported below
            errors.append(repr(e))

    th = [threading.Thread(target=build, args=("a", wa, sa)),
          threading.Thread(target=build, args=("b", wb, sb))]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errors, errors
    La, Lb = built["a"], built["b"]

    oa2, la2 = torch.empty_like(oa), torch.empty_like(la)
    ob2, lb2 = torch.empty_like(ob), torch.empty_like(lb)
    dq2, dk2, dv2 = (torch.empty_like(t) for t in gb)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (oa2, la2, ob2, lb2, dq2, dk2, dv2):
            t.view(torch.uint8).fill_(0xFF)
        torch.cuda.synchronize()
        with torch.cuda.stream(sa):
            pg.pg_attn_fwd(La, ta["q"], ta["k"], ta["v"], wa.softmax_scale, o=oa2, lse=la2, stream=sa)
        with torch.cuda.stream(sb):
            pg.pg_attn_fwd(Lb, tb["q"], tb["k"], tb["v"], wb.softmax_scale, o=ob2, lse=lb2, stream=sb)
            pg.pg_attn_bwd(Lb, tb["q"], tb["k"], tb["v"], ob2, lb2, tb["do"], wb.softmax_scale,
                           dq=dq2, dk=dk2, dv=dv2, stream=sb)
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip((oa2, la2, ob2, lb2, dq2, dk2, dv2), ref)):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), (rep, i)
        print(f"  round {rep}: 7 outputs bit-identical to the sequential run", flush=True)
    La.close()
    Lb.close()
