"""GPU checks of pg_rope's single-pair mode: rotating K alone (or Q alone)
gives the same bits as the call that rotates both, and leaves nothing else
written. A decode loop uses it to rotate the new token's K before appending
it to the cache."""
import numpy as np
import pytest
import torch

import shared_prefix_packed_amd as pg
from workloads import draw_qkv, make_custom, make_workload

pytestmark = pytest.mark.gpu


def dev(w, a):
    if w.dtype == "f32":
        return torch.from_numpy(a).cuda()
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("w", [make_workload(0), make_workload(1), make_workload(3),
                               make_custom([0, 7], [[4, 3], [5]], num_q_heads=6,
                                           num_kv_heads=2, head_dim=64, dtype="bf16", seed=2)],
                         ids=lambda w: w.name)
def test_single_pair_equals_pair_call(w):
    x = draw_qkv(w)
    L = pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, w.num_q_heads,
                           w.num_kv_heads, w.head_dim, w.rope_theta)
    pos = pg.pg_position_ids(L)
    q, k = dev(w, x["q"]), dev(w, x["k"])
    qr, kr = pg.pg_rope(L, pos, q, k)
    k_out = torch.full_like(k, float("nan"))
    nq, k_only = pg.pg_rope(L, pos, None, k, k_out=k_out)
    q_out = torch.full_like(q, float("nan"))
    q_only, nk = pg.pg_rope(L, pos, q, None, q_out=q_out)
    torch.cuda.synchronize()
    assert nq is None and nk is None
    assert torch.equal(bits(k_only), bits(kr)) and torch.equal(bits(q_only), bits(qr))


def test_single_pair_argument_errors_on_device():
    """Malformed pair arguments are refused before any launch; every pointer
    passed is a real device tensor of the right size, so nothing here depends
    on the order of the checks."""
    w = make_workload(0)
    L = pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, w.num_q_heads,
                           w.num_kv_heads, w.head_dim, w.rope_theta)
    from shared_prefix_packed_amd import _lib
    import ctypes
    lib = _lib.load()
    x = draw_qkv(w)
    q, k = dev(w, x["q"]), dev(w, x["k"])
    pos = pg.pg_position_ids(L)
    q_out, k_out = torch.empty_like(q), torch.empty_like(k)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    torch.cuda.synchronize()
    # nothing to rotate
    assert lib.pg_rope(L.handle, P(pos), None, None, None, None, 0, None) == -1
    # half a pair: an input without its output, an output without its input
    assert lib.pg_rope(L.handle, P(pos), P(q), None, None, None, 0, None) == -1
    assert lib.pg_rope(L.handle, P(pos), None, None, None, P(k_out), 0, None) == -1
    # no positions
    assert lib.pg_rope(L.handle, None, P(q), P(k), P(q_out), P(k_out), 0, None) == -1
    torch.cuda.synchronize()
