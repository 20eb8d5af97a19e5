"""The hot path under HIP graph capture.

Positions, RoPE, the forward, the backward, one decode step and the
pack / unpack / pad / unpad gathers are captured once into a single graph,
on a layout built and uploaded before the capture. The graph is then
replayed several times, with eager work between the replays
(every output is overwritten with 0xff bytes first). Each replay must
reproduce the eager outputs bit for bit. So none of these calls may allocate,
synchronise, or leave a memset node that only the first replay honours.
"""
import numpy as np
import pytest
import torch

import shared_prefix_packed_amd as pg
from workloads import draw_decode, draw_tensor, make_workload

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def test_hot_path_replays_bit_exactly_under_graph_capture():
    w = make_workload(1)   # DPO-shaped: small enough to replay quickly
    print(f"graph capture on {w.name}: T={w.total_tokens}", flush=True)
    L = pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, w.num_q_heads,
                           w.num_kv_heads, w.head_dim, w.rope_theta)
    q, k, v, do = (dev(draw_tensor(w, n)) for n in ("q", "k", "v", "do"))
    T, Hq, d = q.shape
    dx = draw_decode(w)
    qd = dev(dx["q"])
    cur = torch.from_numpy(dx["cur_lens"]).cuda()
    N = qd.shape[0]

    pos = torch.empty(T, dtype=torch.int64, device="cuda")
    qr, kr = torch.empty_like(q), torch.empty_like(k)
    o = torch.empty_like(q)
    lse = torch.empty((Hq, T), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((Hq, T), dtype=torch.float32, device="cuda")
    od = torch.empty_like(qd)
    ld = torch.empty((Hq, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, L.decode_workspace_size()), dtype=torch.uint8, device="cuda")
    # gathers over 256-byte rows
    G, Nr = len(w.prefix_lens), len(w.suffix_lens)
    ppad, spad = int(max(w.prefix_lens)) + 3, int(max(w.suffix_lens)) + 2
    r = np.random.default_rng(7)
    pre_in = torch.from_numpy(r.integers(-2**31, 2**31, size=(G, ppad, 64)).astype(np.int32)).cuda()
    suf_in = torch.from_numpy(r.integers(-2**31, 2**31, size=(Nr, spad, 64)).astype(np.int32)).cuda()
    packed = torch.empty((T, 64), dtype=torch.int32, device="cuda")
    pre_out = torch.empty((G, ppad, 64), dtype=torch.int32, device="cuda")
    suf_out = torch.empty((Nr, spad + 1, 64), dtype=torch.int32, device="cuda")
    width = L.summary().max_group_len + 1
    padded = torch.empty((G, width, 64), dtype=torch.int32, device="cuda")
    back = torch.empty_like(packed)
    outs = [pos, qr, kr, o, lse, dq, dk, dv, delta, od, ld, packed, pre_out, suf_out, padded, back]

    def path():
        s = torch.cuda.current_stream()
        pg.pg_position_ids(L, pos=pos, stream=s)
        pg.pg_rope(L, pos, q, k, q_out=qr, k_out=kr, stream=s)
        pg.pg_attn_fwd(L, qr, kr, v, w.softmax_scale, o=o, lse=lse, stream=s)
        pg.pg_attn_bwd(L, qr, kr, v, o, lse, do, w.softmax_scale, dq=dq, dk=dk, dv=dv, delta=delta,
                       stream=s)
        pg.pg_attn_decode(L, qd, kr, v, cur, w.softmax_scale, o=od, lse=ld, workspace=ws, stream=s)
        pg.pg_pack_rows(L, pre_in, suf_in, packed=packed, stream=s)
        pg.pg_unpack_rows(L, packed, ppad, spad, prefix_out=pre_out, suffix_out=suf_out, stream=s)
        pg.pg_pad_rows(L, packed, padded=padded, stream=s)
        pg.pg_unpad_rows(L, padded, packed=back, stream=s)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        path()   # eager run (also the warm-up the capture wants)
    torch.cuda.synchronize()
    assert torch.equal(back, packed)   # unpad undoes pad
    ref = [t.clone() for t in outs]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path()
    torch.cuda.synchronize()

    for rep in range(3):
        for t in outs:
            t.view(torch.uint8).fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(outs, ref)):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), (rep, i)
        print(f"  replay {rep}: all {len(outs)} outputs bit-identical to the eager run", flush=True)
    del g
    L.close()


def test_graph_replays_after_its_layout_is_destroyed():
    """A layout used under capture keeps its upload buffer: after the layout
    is destroyed and new layouts of the same size are built, uploaded and used
    (which recycles every idle buffer), the graph still replays the captured
    forward bit for bit."""
    w = make_workload(1)
    L = pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, w.num_q_heads,
                           w.num_kv_heads, w.head_dim, w.rope_theta)
    q, k, v = (dev(draw_tensor(w, n)) for n in ("q", "k", "v"))
    T, Hq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((Hq, T), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pg.pg_attn_fwd(L, q, k, v, w.softmax_scale, o=o, lse=lse, stream=side)
    torch.cuda.synchronize()
    ref = (o.clone(), lse.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pg.pg_attn_fwd(L, q, k, v, w.softmax_scale, o=o, lse=lse)
    torch.cuda.synchronize()
    L.close()
    # other layouts of the same size (other lengths, so other tables) take
    # every idle upload buffer and overwrite it
    others = []
    for seed in range(4):
        pl = np.roll(w.prefix_lens, seed + 1)
        sl = np.roll(w.suffix_lens, 2 * seed + 1)
        L2 = pg.pg_build_layout(pl, w.suffix_counts, sl, w.num_q_heads, w.num_kv_heads,
                                w.head_dim, w.rope_theta)
        pg.pg_position_ids(L2)
        others.append(L2)
    torch.cuda.synchronize()
    for L2 in others:
        L2.close()
    for rep in range(2):
        o.view(torch.uint8).fill_(0xFF)
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref[0].view(torch.int16)), rep
        assert torch.equal(lse, ref[1]), rep
    print("  graph replayed bit-identically after its layout was destroyed", flush=True)
    del g
