"""GPU parity of pg_attn_decode (one decode step over a group-contiguous KV
cache) against the fp64 oracle's ``decode_attention``.

Inputs: the workload's layout taken as the cache with every response segment
at capacity; seeded K and V cache rows (generator streams 2, 3), and the
step's current lengths and queries (stream 5, uniform lengths in
[1, capacity]). Tolerance as for the forward: O max-abs <= 2e-2 and lse
max-abs <= 1e-3 (P enters the matrix cores rounded to bf16; O is rounded to
bf16 once). bf16 d = 128 runs the MFMA kernel, every other case the
one-workgroup-per-row kernel.
"""
import sys

import numpy as np
import pytest
import torch

import shared_prefix_packed_amd as pg
from oracle import pg_oracle as O
from workloads import bf16_bits_to_f32, draw_decode, draw_tensor, make_custom, make_workload

pytestmark = pytest.mark.gpu

O_TOL = 2e-2
LSE_TOL = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a, dtype):
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def to_host(t, dtype):
    if dtype == "f32":
        return t.detach().cpu().numpy().astype(np.float64)
    return bf16_bits_to_f32(t.detach().cpu().view(torch.int16).numpy().view(np.uint16)).astype(np.float64)


def as_f64(a, dtype):
    return (a if dtype == "f32" else bf16_bits_to_f32(a)).astype(np.float64)


def run(w, cur_lens=None, responses=None, poison=True, workspace=None, layout=None):
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    dx = draw_decode(w)
    cur = dx["cur_lens"] if cur_lens is None else np.asarray(cur_lens, dtype=np.int32)
    kc, vc = draw_tensor(w, "k"), draw_tensor(w, "v")
    L = layout or pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, w.num_q_heads,
                                     w.num_kv_heads, w.head_dim, w.rope_theta)
    q = to_dev(dx["q"], w.dtype)
    o = torch.full_like(q, float("nan")) if poison else None
    lse = torch.full((w.num_q_heads, q.shape[0]), float("nan"), device="cuda") if poison else None
    say(f"  decode {w.name}: N={q.shape[0]} T={lay['total_tokens']} heads {w.num_q_heads}/"
        f"{w.num_kv_heads} d={w.head_dim} {w.dtype} items={L.summary().num_dec_items}")
    o, lse = pg.pg_attn_decode(L, q, to_dev(kc, w.dtype), to_dev(vc, w.dtype),
                               torch.from_numpy(cur).cuda(), w.softmax_scale, o=o, lse=lse,
                               workspace=workspace)
    torch.cuda.synchronize()
    ro, rl = O.decode_attention(as_f64(dx["q"], w.dtype), as_f64(kc, w.dtype), as_f64(vc, w.dtype),
                                lay, cur, w.softmax_scale, w.num_q_heads, w.num_kv_heads,
                                responses=responses)
    return to_host(o, w.dtype), lse.cpu().numpy().astype(np.float64), ro, rl, cur, L


def compare(go, gl, ro, rl, responses=None):
    if responses is not None:
        idx = np.asarray(list(responses))
        go, ro, gl, rl = go[idx], ro[idx], gl[:, idx], rl[:, idx]
    assert np.isfinite(go).all(), "O not written or not finite"
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(gl), empty), "empty key sets disagree"
    assert not np.isnan(gl).any()
    eo = float(np.abs(go - ro).max()) if go.size else 0.0
    el = float(np.abs(gl[~empty] - rl[~empty]).max()) if (~empty).any() else 0.0
    say(f"    O max|err| {eo:.3e}, lse max|err| {el:.3e}, empty rows {int(empty.sum())}")
    assert eo <= O_TOL and el <= LSE_TOL
    if empty.any():
        assert np.all(go[np.nonzero(empty.T)] == 0)


@pytest.mark.parametrize("index", [0, 1, 2, 3])
def test_decode_matches_oracle_on_workloads(index):
    w = make_workload(index)
    go, gl, ro, rl, _, _ = run(w)
    compare(go, gl, ro, rl)


def test_decode_long_prefix_all_responses():
    """Every response of the long-prefix workload: 16K-token prompts, each
    read once per step for its four responses."""
    w = make_workload(4)
    go, gl, ro, rl, _, _ = run(w)
    compare(go, gl, ro, rl)


EDGE = [
    # (P, capacities, Hq, Hkv, cur_lens or None)
    ([5, 9], [[3, 4], [2, 6, 1]], 4, 1, None),
    ([0, 7], [[40, 33], [5]], 8, 2, [0, 33, 5]),                 # empty key set, prompt only
    ([31, 33, 64], [[32, 1], [63, 65], [128, 129, 127]], 32, 8, None),
    ([600], [[700, 3, 0, 64, 65, 1, 2, 3, 4, 513]], 16, 2, None),  # 80 rows: three row blocks
    ([1500], [[50, 1100]], 32, 1, [-3, 4000]),                    # clamping, r = 32: 64 rows
    ([0, 0], [[0], []], 4, 4, [5]),                               # no tokens at all
    ([100, 0, 37], [[], [17, 0], [1, 1, 1]], 2, 2, [17, 0, 1, 0, 1]),
    ([4097, 40], [[100, 2000], [7]], 8, 2, None),                 # prompt past 4096 rows: longer pieces
]


@pytest.mark.parametrize("case", EDGE)
@pytest.mark.parametrize("kind", [("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_decode_edge_shapes(case, kind):
    P, S, hq, hkv, cur = case
    dtype, d = kind
    w = make_custom(P, S, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype, seed=11)
    go, gl, ro, rl, _, _ = run(w, cur_lens=cur)
    compare(go, gl, ro, rl)


def test_decode_full_capacity_and_workspace_reuse():
    """Two steps on one layout and one workspace: full capacity, then the
    drawn lengths; both match the oracle (nothing of the first call leaks)."""
    w = make_workload(2)
    L = pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, w.num_q_heads,
                           w.num_kv_heads, w.head_dim, w.rope_theta)
    ws = torch.empty(L.decode_workspace_size(), dtype=torch.uint8, device="cuda")
    caps = np.asarray(w.suffix_lens, dtype=np.int32)
    resp = list(range(0, len(caps), 7))
    go, gl, ro, rl, _, _ = run(w, cur_lens=caps, responses=resp, workspace=ws, layout=L)
    compare(go, gl, ro, rl, responses=resp)
    go, gl, ro, rl, _, _ = run(w, responses=resp, workspace=ws, layout=L)
    compare(go, gl, ro, rl, responses=resp)


def test_decode_equals_forward_last_rows_on_gpu():
    """At full capacity, response k's decode row is the forward's output at the
    response's last token when that token's query is the decode query."""
    w = make_custom([40, 0], [[9, 70, 33], [64]], num_q_heads=8, num_kv_heads=2, head_dim=128,
                    dtype="bf16", seed=5)
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    L = pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, 8, 2, 128, w.rope_theta)
    dx = draw_decode(w)
    qf = draw_tensor(w, "q")
    last = [int(lay["seg_off"][g + k + 1]) + int(c) - 1
            for k, (g, c) in enumerate(zip(O.response_group(lay), w.suffix_lens))]
    qf[last] = dx["q"]
    k, v = to_dev(draw_tensor(w, "k"), "bf16"), to_dev(draw_tensor(w, "v"), "bf16")
    of, lf = pg.pg_attn_fwd(L, to_dev(qf, "bf16"), k, v, w.softmax_scale)
    caps = torch.from_numpy(np.asarray(w.suffix_lens, dtype=np.int32)).cuda()
    od, ld = pg.pg_attn_decode(L, to_dev(dx["q"], "bf16"), k, v, caps, w.softmax_scale)
    torch.cuda.synchronize()
    a, b = to_host(od, "bf16"), to_host(of, "bf16")[last]
    say(f"    decode vs forward: O max|diff| {np.abs(a - b).max():.3e}")
    assert np.abs(a - b).max() <= O_TOL
    assert np.abs(ld.cpu().numpy() - lf.cpu().numpy()[:, last]).max() <= LSE_TOL


def test_decode_is_deterministic():
    w = make_workload(1)
    L = pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, w.num_q_heads,
                           w.num_kv_heads, w.head_dim, w.rope_theta)
    dx = draw_decode(w)
    q = to_dev(dx["q"], "bf16")
    k, v = to_dev(draw_tensor(w, "k"), "bf16"), to_dev(draw_tensor(w, "v"), "bf16")
    cur = torch.from_numpy(dx["cur_lens"]).cuda()
    o1, l1 = pg.pg_attn_decode(L, q, k, v, cur, w.softmax_scale)
    o2, l2 = pg.pg_attn_decode(L, q, k, v, cur, w.softmax_scale)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
