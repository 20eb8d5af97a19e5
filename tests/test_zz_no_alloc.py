"""GPU check of pg_attn_decode_noalloc: the decode step with its partial
results in the library's static per-GPU scratch array instead of a caller
workspace. Through the C ABI it must give exactly the outputs of
pg_attn_decode (same kernels), on two calls in a row, the second on a smaller
layout, so that the array's contents left by the first call cannot leak into
the second; and it must refuse, before any launch, a step whose partial
results would not fit. The outputs of the reference calls are also checked
against the fp64 oracle's decode_attention to the decode tolerances."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import shared_prefix_packed_amd as pg
from shared_prefix_packed_amd import _lib
from oracle import pg_oracle as O
from workloads import bf16_bits_to_f32, draw_decode, draw_tensor, make_custom, make_workload

pytestmark = pytest.mark.gpu

O_TOL = 2e-2
LSE_TOL = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, dtype):
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def host(t, dtype):
    if dtype == "f32":
        return t.detach().cpu().numpy().astype(np.float64)
    return bf16_bits_to_f32(t.detach().cpu().view(torch.int16).numpy().view(np.uint16)).astype(np.float64)


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def step_inputs(w):
    dx = draw_decode(w)
    L = pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, w.num_q_heads,
                           w.num_kv_heads, w.head_dim, w.rope_theta)
    q = dev(dx["q"], w.dtype)
    kc, vc = dev(draw_tensor(w, "k"), w.dtype), dev(draw_tensor(w, "v"), w.dtype)
    cur = torch.from_numpy(dx["cur_lens"]).cuda()
    return L, dx, q, kc, vc, cur


def noalloc_via_abi(L, q, kc, vc, cur, w, o, lse):
    """Direct C ABI call (no binding logic in between)."""
    lib = _lib.load()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    dtype = _lib.PG_BF16 if w.dtype == "bf16" else _lib.PG_F32
    return lib.pg_attn_decode_noalloc(L.handle, P(q), P(kc), P(vc), P(cur), P(o), P(lse), dtype,
                                      ctypes.c_float(w.softmax_scale), stream)


@pytest.mark.parametrize("names", [("grpo-bf16", "dpo-bf16"), ("heterogeneous-bf16", "tiny-fp32")])
def test_noalloc_equals_workspace_call_twice(names):
    """Two calls in a row on one GPU, the second on a smaller layout; each
    bit-identical to pg_attn_decode with a caller workspace."""
    index = {"tiny-fp32": 0, "dpo-bf16": 1, "grpo-bf16": 2, "heterogeneous-bf16": 3}
    for name in names:
        w = make_workload(index[name])
        L, dx, q, kc, vc, cur = step_inputs(w)
        need = L.decode_workspace_size()
        say(f"no-alloc decode: {w.name}, {L.summary().num_dec_items} items, scratch {need} of "
            f"{_lib.PG_DECODE_SCRATCH_BYTES} bytes")
        assert need <= _lib.PG_DECODE_SCRATCH_BYTES
        o_ref, l_ref = pg.pg_attn_decode(L, q, kc, vc, cur, w.softmax_scale)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((w.num_q_heads, q.shape[0]), float("nan"), device="cuda")
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        assert noalloc_via_abi(L, q, kc, vc, cur, w, o, lse) == 0
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert torch.equal(bits(o), bits(o_ref)), w.name
        assert torch.equal(lse.view(torch.int32), l_ref.view(torch.int32)), w.name
        # the reference call itself against the oracle
        lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
        N = q.shape[0]
        resp = sorted(set(np.linspace(0, N - 1, num=min(N, 12)).astype(int).tolist()))
        f = lambda a: (a if w.dtype == "f32" else bf16_bits_to_f32(a)).astype(np.float64)
        ko = O.decode_attention(f(dx["q"]), f(draw_tensor(w, "k")), f(draw_tensor(w, "v")), lay,
                                dx["cur_lens"], w.softmax_scale, w.num_q_heads, w.num_kv_heads,
                                responses=resp)
        eo = np.abs(host(o, w.dtype)[resp] - ko[0][resp]).max()
        el = np.abs(lse.cpu().numpy()[:, resp] - ko[1][:, resp]).max()
        say(f"  {w.name}: bit-identical to the workspace call; {len(resp)} responses vs oracle: "
            f"max|dO|={eo:.2e} max|dlse|={el:.2e}")
        assert eo <= O_TOL and el <= LSE_TOL
        L.close()


def test_noalloc_refuses_a_step_larger_than_the_scratch():
    """300 responses x 8 KV heads make 2400 work items, 40 MB of partial
    results: refused with PG_ERR_INVALID_ARG before any launch; the outputs
    stay untouched. A step that fits (240 responses) runs."""
    for n, fits in ((300, False), (240, True)):
        w = make_custom([0], [[64] * n], num_q_heads=32, num_kv_heads=8, head_dim=128,
                        dtype="bf16", seed=3)
        L, dx, q, kc, vc, cur = step_inputs(w)
        need = L.decode_workspace_size()
        assert (need <= _lib.PG_DECODE_SCRATCH_BYTES) == fits
        o = torch.full_like(q, float("nan"))
        lse = torch.full((w.num_q_heads, q.shape[0]), float("nan"), device="cuda")
        st = noalloc_via_abi(L, q, kc, vc, cur, w, o, lse)
        torch.cuda.synchronize()
        if fits:
            assert st == 0
            o_ref, l_ref = pg.pg_attn_decode(L, q, kc, vc, cur, w.softmax_scale)
            torch.cuda.synchronize()
            assert torch.equal(bits(o), bits(o_ref)) and torch.equal(lse, l_ref)
        else:
            assert st == -1
            assert "scratch" in _lib.load().pg_last_error().decode()
            assert torch.isnan(o.float()).all() and torch.isnan(lse).all()
        say(f"  {n} responses: {need} bytes of partial results -> "
            f"{'ran' if fits else 'refused'}")
        L.close()
