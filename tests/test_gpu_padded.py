"""GPU parity of the right-padded compatibility form against the oracle:
pg_position_ids_padded (positions with zero padding, padding mask),
pg_pad_rows and pg_unpad_rows, bit-exact; and the padded route through the
packed path (unpad -> positions/RoPE/attention -> pad) against the packed path
itself."""
import numpy as np
import pytest
import torch

import shared_prefix_packed_amd as pg
from oracle import pg_oracle as O
from workloads import draw_qkv, make_custom, make_workload

pytestmark = pytest.mark.gpu

SHAPES = [
    ([5, 9], [[3, 4], [2, 6, 1]]),
    ([0, 7], [[4, 3], [5]]),
    ([6, 4, 3], [[], [0, 2], [0, 0]]),
    ([0], [[0, 3, 0]]),
    ([17], [[]]),
    ([0, 0], [[0], []]),
    ([300], [[1, 40, 0, 200, 33]]),
]


def workloads():
    out = [make_workload(i) for i in range(5)]
    for P, S in SHAPES:
        out.append(make_custom(P, S, num_q_heads=4, num_kv_heads=1, head_dim=64, dtype="bf16"))
    return out


def build(w):
    return pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, w.num_q_heads,
                              w.num_kv_heads, w.head_dim, w.rope_theta)


@pytest.mark.parametrize("w", workloads(), ids=lambda w: f"{w.name}-{len(w.prefix_lens)}")
def test_padded_positions_and_mask(w):
    L = build(w)
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    width = L.summary().max_group_len + 5
    pos, mask = pg.pg_position_ids_padded(L, width)
    torch.cuda.synchronize()
    assert np.array_equal(pos.cpu().numpy(), O.padded_positions(lay, width))
    assert np.array_equal(mask.cpu().numpy(), O.padding_mask(lay, width))


ROWS = [(np.int64, (1,)), (np.float32, (3,)), (np.float16, (128,))]


@pytest.mark.parametrize("w", workloads(), ids=lambda w: f"{w.name}-{len(w.prefix_lens)}")
@pytest.mark.parametrize("row", ROWS, ids=lambda r: f"{np.dtype(r[0]).name}x{r[1][0]}")
def test_pad_and_unpad_bit_exact(w, row):
    dtype, tail = row
    if w.total_tokens > 20000 and tail[0] == 128:
        tail = (8,)
    L = build(w)
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    width = L.summary().max_group_len + 3
    r = np.random.default_rng(5)
    nbytes = w.total_tokens * int(np.prod(tail)) * np.dtype(dtype).itemsize
    x = r.integers(0, 256, size=nbytes, dtype=np.uint8).view(dtype).reshape((w.total_tokens,) + tail)
    xd = torch.from_numpy(x).cuda()
    padded = torch.full((len(w.prefix_lens), width) + tail, 7, dtype=xd.dtype, device="cuda")
    pg.pg_pad_rows(L, xd, padded=padded)
    back = torch.full_like(xd, 9)
    pg.pg_unpad_rows(L, padded, packed=back)
    torch.cuda.synchronize()
    ref = O.pad_rows(x, lay, width)
    assert np.array_equal(padded.cpu().numpy().view(np.uint8), ref.view(np.uint8))
    assert np.array_equal(back.cpu().numpy().view(np.uint8), x.view(np.uint8))
    assert np.array_equal(O.unpad_rows(ref, lay).view(np.uint8), x.view(np.uint8))


@pytest.mark.parametrize("index", [1, 3])
def test_padded_route_equals_packed_path(index):
    """A caller holding padded Q, K, V unpads them, runs the packed path and
    pads the output back: the real rows equal the packed path's, the padding
    is zero."""
    w = make_workload(index)
    x = draw_qkv(w)
    L = build(w)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    qp, kp, vp = (pg.pg_pad_rows(L, t) for t in (q, k, v))
    qu, ku, vu = (pg.pg_unpad_rows(L, t) for t in (qp, kp, vp))
    pos = pg.pg_position_ids(L)
    qr, kr = pg.pg_rope(L, pos, qu, ku)
    o, _ = pg.pg_attn_fwd(L, qr, kr, vu, w.softmax_scale)
    op = pg.pg_pad_rows(L, o)
    qr2, kr2 = pg.pg_rope(L, pos, q, k)
    o2, _ = pg.pg_attn_fwd(L, qr2, kr2, v, w.softmax_scale)
    _, mask = pg.pg_position_ids_padded(L)
    torch.cuda.synchronize()
    m = mask.bool()
    assert torch.equal(op[m].view(torch.int16), o2.view(torch.int16))
    assert torch.all(op[~m].view(torch.int16) == 0)
