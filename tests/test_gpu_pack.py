"""GPU parity of pg_pack_rows / pg_unpack_rows against the oracle's
pack_rows / unpack_rows: byte-for-byte equality (a gather computes nothing).
Row types: 8-byte ids, 12-byte rows (4-byte units), 256-byte bf16 rows."""
import numpy as np
import pytest
import torch

import shared_prefix_packed_amd as pg
from oracle import pg_oracle as O
from workloads import make_custom, make_workload

pytestmark = pytest.mark.gpu

ROW_TYPES = [((), np.int64), ((3,), np.float32), ((128,), np.float16)]


def _check(w, tail, dtype, seed):
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    G, N = len(w.prefix_lens), len(w.suffix_lens)
    ppad = int(max(w.prefix_lens.max(initial=0), 0)) + 3
    spad = int(max(w.suffix_lens.max(initial=0), 0)) + 2
    r = np.random.default_rng(seed)
    # uniformly random bytes viewed as the row type, so every bit of every
    # element varies (a gather moves bit patterns, NaN and inf included)
    isz = np.dtype(dtype).itemsize
    prefix = r.integers(0, 256, size=(G, ppad) + tail + (isz,), dtype=np.uint8).view(dtype)[..., 0]
    suffix = r.integers(0, 256, size=(N, spad) + tail + (isz,), dtype=np.uint8).view(dtype)[..., 0]
    L = pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, w.num_q_heads,
                           w.num_kv_heads, w.head_dim, w.rope_theta)
    tp, ts = torch.from_numpy(prefix).cuda(), torch.from_numpy(suffix).cuda()
    T = int(lay["total_tokens"])
    poisoned = torch.full((T,) + tail, 7, dtype=tp.dtype, device="cuda")
    packed = pg.pg_pack_rows(L, tp, ts, packed=poisoned)
    pre, suf = pg.pg_unpack_rows(L, packed, ppad, spad)
    torch.cuda.synchronize()
    want = O.pack_rows(prefix, suffix, lay)
    assert np.array_equal(packed.cpu().numpy().view(np.uint8), want.view(np.uint8))
    wp, ws = O.unpack_rows(want, lay, ppad, spad)
    assert np.array_equal(pre.cpu().numpy().view(np.uint8), wp.view(np.uint8))
    assert np.array_equal(suf.cpu().numpy().view(np.uint8), ws.view(np.uint8))


@pytest.mark.parametrize("i", range(5))
@pytest.mark.parametrize("rt", range(len(ROW_TYPES)))
def test_pack_unpack_workloads(i, rt):
    w = make_workload(i)
    tail, dtype = ROW_TYPES[rt]
    if i >= 2 and rt == 2:
        tail = (8,)   # keep the padded inputs of the large workloads small
    print(f"pack/unpack: workload {w.name}, rows {tail} {np.dtype(dtype).name}", flush=True)
    _check(w, tail, dtype, seed=10 * i + rt)


EDGE = [([5, 9], [[3, 4], [2, 6, 1]]), ([0, 7], [[4, 3], [5]]), ([6, 4, 3], [[], [0, 2], [0, 0]]),
        ([1], [[1, 1, 1]]), ([0], [[0, 3, 0]]), ([17], [[]]), ([0, 0], [[0], []])]


@pytest.mark.parametrize("case", range(len(EDGE)))
def test_pack_unpack_edge_shapes(case):
    P, S = EDGE[case]
    w = make_custom(P, S)
    for rt, (tail, dtype) in enumerate(ROW_TYPES):
        _check(w, tail, dtype, seed=100 + case)


@pytest.mark.parametrize("row", [4096, 4100])
def test_gathers_larger_than_the_last_level_cache(row):
    """Hidden-state-sized rows on the GRPO-shaped workload: every gather
    writes more than 256 MB, so the kernels take their streaming-store branch
    (the cases above, all smaller, take the ordinary one). 4096-byte rows move
    in 16-byte units, 4100-byte rows in 4-byte units."""
    w = make_workload(2)
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    G, N, T = len(w.prefix_lens), len(w.suffix_lens), int(w.total_tokens)
    ppad, spad = int(w.prefix_lens.max()), int(w.suffix_lens.max())
    assert T * row > 256 << 20
    print(f"large gathers: {w.name} T={T}, {row}-byte rows", flush=True)
    r = np.random.default_rng(77 + row)
    prefix = r.integers(0, 256, size=(G, ppad, row), dtype=np.uint8)
    suffix = r.integers(0, 256, size=(N, spad, row), dtype=np.uint8)
    L = pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, w.num_q_heads,
                           w.num_kv_heads, w.head_dim, w.rope_theta)
    packed = pg.pg_pack_rows(L, torch.from_numpy(prefix).cuda(), torch.from_numpy(suffix).cuda())
    pre, suf = pg.pg_unpack_rows(L, packed, ppad, spad)
    width = L.summary().max_group_len
    padded = torch.full((G, width, row), 7, dtype=torch.uint8, device="cuda")
    pg.pg_pad_rows(L, packed, padded=padded)
    back = torch.full_like(packed, 9)
    pg.pg_unpad_rows(L, padded, packed=back)
    torch.cuda.synchronize()
    want = O.pack_rows(prefix, suffix, lay)
    assert np.array_equal(packed.cpu().numpy(), want)
    wp, ws = O.unpack_rows(want, lay, ppad, spad)
    assert np.array_equal(pre.cpu().numpy(), wp)
    assert np.array_equal(suf.cpu().numpy(), ws)
    assert np.array_equal(padded.cpu().numpy(), O.pad_rows(want, lay, width))
    assert np.array_equal(back.cpu().numpy(), want)
    L.close()
