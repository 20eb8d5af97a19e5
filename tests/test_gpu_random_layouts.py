"""GPU parity on seeded random layouts: random group counts, prompt and
response lengths (zeros included), head shapes and tile-boundary lengths,
each checked end to end against the fp64 oracle -- forward (O, lse), backward
(dQ, dK, dV), one decode step, and the pack / unpack / pad / unpad gathers
(bit-exact) for bf16 with d = 128; forward and decode for fp32 (d = 64, 128)
and bf16 d = 64. Sizes stay small enough for the dense oracle."""
import numpy as np
import pytest
import torch

import shared_prefix_packed_amd as pg
from oracle import pg_oracle as O
from workloads import bf16_bits_to_f32, draw_decode, draw_tensor, make_custom

pytestmark = pytest.mark.gpu

HEADS = [(4, 1), (8, 2), (32, 8), (6, 3), (16, 16)]


def random_case(seed):
    r = np.random.default_rng(10_000 + seed)
    G = int(r.integers(1, 6))
    P, S = [], []
    for _ in range(G):
        # lengths near tile edges (31/32/33, 63/64/65, 127/128/129) as often as random ones
        edge = [0, 1, 31, 32, 33, 63, 64, 65, 127, 128, 129]
        pick = lambda hi: int(r.choice(edge)) if r.random() < 0.4 else int(r.integers(0, hi))
        P.append(pick(300))
        S.append([pick(160) for _ in range(int(r.integers(0, 5)))])
    hq, hkv = HEADS[seed % len(HEADS)]
    return P, S, hq, hkv


def dev(a):
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def host(t):
    return bf16_bits_to_f32(t.detach().cpu().view(torch.int16).numpy().view(np.uint16)).astype(np.float64)


@pytest.mark.parametrize("seed", range(40))
def test_random_layout_end_to_end(seed):
    P, S, hq, hkv = random_case(seed)
    w = make_custom(P, S, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, dtype="bf16",
                    seed=seed, name=f"random-{seed}")
    print(f"random layout {seed}: P={P} S={S} heads {hq}/{hkv} T={w.total_tokens}", flush=True)
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    L = pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, hq, hkv, 128, w.rope_theta)
    x = {n: draw_tensor(w, n) for n in ("q", "k", "v", "do")}
    q, k, v, do = (dev(x[n]) for n in ("q", "k", "v", "do"))
    qh, kh, vh, doh = (bf16_bits_to_f32(x[n]).astype(np.float64) for n in ("q", "k", "v", "do"))

    # forward
    o, lse = pg.pg_attn_fwd(L, q, k, v, w.softmax_scale)
    ro, rl = O.attention(qh, kh, vh, lay, w.softmax_scale, hq, hkv)
    torch.cuda.synchronize()
    if w.total_tokens:
        assert np.abs(host(o) - ro).max() <= 2e-2
        assert np.abs(lse.cpu().numpy() - rl).max() <= 1e-3

    # backward (tolerance as in test_gpu_backward.py)
    if w.total_tokens:
        dq, dk, dv = pg.pg_attn_bwd(L, q, k, v, o, lse, do, w.softmax_scale)
        rq, rk, rv = O.attention_backward(qh, kh, vh, doh, lay, w.softmax_scale, hq, hkv)
        torch.cuda.synchronize()
        for got, ref in ((host(dq), rq), (host(dk), rk), (host(dv), rv)):
            scale = max(1.0, float(np.abs(ref).max()))
            assert np.abs(got - ref).max() <= 3e-2 * scale
            nr = np.linalg.norm(ref)
            if nr > 0:
                assert np.linalg.norm(got - ref) / nr <= 2e-2

    # one decode step over the layout taken as the cache at capacity
    N = len(w.suffix_lens)
    if N:
        dx = draw_decode(w)
        od, ld = pg.pg_attn_decode(L, dev(dx["q"]), k, v, torch.from_numpy(dx["cur_lens"]).cuda(),
                                   w.softmax_scale)
        rod, rld = O.decode_attention(bf16_bits_to_f32(dx["q"]).astype(np.float64), kh, vh, lay,
                                      dx["cur_lens"], w.softmax_scale, hq, hkv)
        torch.cuda.synchronize()
        empty = np.isneginf(rld)
        assert np.array_equal(np.isneginf(ld.cpu().numpy()), empty)
        assert np.abs(host(od) - rod).max() <= 2e-2
        if (~empty).any():
            assert np.abs(ld.cpu().numpy()[~empty] - rld[~empty]).max() <= 1e-3

    # gathers, bit-exact
    rows = np.random.default_rng(seed).integers(0, 256, size=(w.total_tokens, 48), dtype=np.uint8)
    packed = torch.from_numpy(rows.view(np.int32)).cuda()
    ppad, spad = max(P) + 1, max([s for g in S for s in g] + [0]) + 2
    pre = O.unpack_rows(rows.view(np.int32), lay, ppad, spad)
    pu, su = pg.pg_unpack_rows(L, packed, ppad, spad)
    width = L.summary().max_group_len + 1
    padded = pg.pg_pad_rows(L, packed, max_len=width)
    back = pg.pg_unpad_rows(L, padded)
    torch.cuda.synchronize()
    assert np.array_equal(pu.cpu().numpy(), pre[0]) and np.array_equal(su.cpu().numpy(), pre[1])
    repacked = pg.pg_pack_rows(L, pu, su[:, 1:].contiguous())   # row 0 of a response part is the prompt's last
    torch.cuda.synchronize()
    assert np.array_equal(repacked.cpu().numpy(), rows.view(np.int32))
    assert np.array_equal(padded.cpu().numpy(), O.pad_rows(rows.view(np.int32), lay, width))
    assert np.array_equal(back.cpu().numpy(), rows.view(np.int32))


def _to_dev(a, dtype):
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return dev(a)


def _host(t, dtype):
    return t.detach().cpu().numpy().astype(np.float64) if dtype == "f32" else host(t)


def _f64(a, dtype):
    return (a if dtype == "f32" else bf16_bits_to_f32(a)).astype(np.float64)


@pytest.mark.parametrize("seed", range(24))
def test_random_layout_other_dtypes(seed):
    """The same random layouts through the fp32 (d = 64, 128) and bf16 d = 64
    kernels: forward and one decode step against the oracle (fp32: 1e-5)."""
    P, S, hq, hkv = random_case(seed)
    dtype, d = [("f32", 64), ("f32", 128), ("bf16", 64)][seed % 3]
    w = make_custom(P, S, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype,
                    seed=seed, name=f"random-{dtype}-{d}-{seed}")
    print(f"random layout {seed} ({dtype}, d={d}): P={P} S={S} heads {hq}/{hkv}", flush=True)
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    L = pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, hq, hkv, d, w.rope_theta)
    x = {n: draw_tensor(w, n) for n in ("q", "k", "v")}
    q, k, v = (_to_dev(x[n], dtype) for n in ("q", "k", "v"))
    tol_o, tol_l = (1e-5, 1e-5) if dtype == "f32" else (2e-2, 1e-3)
    if w.total_tokens:
        o, lse = pg.pg_attn_fwd(L, q, k, v, w.softmax_scale)
        ro, rl = O.attention(_f64(x["q"], dtype), _f64(x["k"], dtype), _f64(x["v"], dtype), lay,
                             w.softmax_scale, hq, hkv)
        torch.cuda.synchronize()
        assert np.abs(_host(o, dtype) - ro).max() <= tol_o
        assert np.abs(lse.cpu().numpy() - rl).max() <= tol_l
    if len(w.suffix_lens):
        dx = draw_decode(w)
        od, ld = pg.pg_attn_decode(L, _to_dev(dx["q"], dtype), k, v,
                                   torch.from_numpy(dx["cur_lens"]).cuda(), w.softmax_scale)
        rod, rld = O.decode_attention(_f64(dx["q"], dtype), _f64(x["k"], dtype), _f64(x["v"], dtype),
                                      lay, dx["cur_lens"], w.softmax_scale, hq, hkv)
        torch.cuda.synchronize()
        empty = np.isneginf(rld)
        assert np.array_equal(np.isneginf(ld.cpu().numpy()), empty)
        assert np.abs(_host(od, dtype) - rod).max() <= tol_o
        if (~empty).any():
            assert np.abs(ld.cpu().numpy()[~empty] - rld[~empty]).max() <= tol_l
    L.close()
