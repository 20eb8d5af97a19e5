"""GPU parity of libpg.so against the fp64 oracle.

Tolerances (stated for this path): position ids and layout bit-exact; RoPE
within 1 ulp of the storage dtype (bf16: count of 1-ulp differences reported
and bounded; fp32: 1e-6 abs); attention output O max-abs error <= 2e-2 and
lse error <= 1e-3, for fp32 and bf16.

Attention is checked on every (token, head) row of all five workloads (GRPO,
heterogeneous and long-prefix with the oracle run per (group, query head)
unit in parallel, tests/oracle_units.py), in the same launch configuration
the benchmark times, with O and lse filled with NaN before the launch, so an
element the kernel leaves unwritten fails. The whole pipeline (positions ->
RoPE -> attention) is checked the same way on every row of every workload.
"""
import sys

import numpy as np
import pytest
import torch

import shared_prefix_packed_amd as pg
from oracle import pg_oracle as O
import oracle_units as U
from workloads import bf16_bits_to_f32, draw_qkv, f32_to_bf16_bits, make_custom, make_workload

pytestmark = pytest.mark.gpu

O_TOL = 2e-2
LSE_TOL = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(w, a):
    if w.dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def to_host_f32(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(t.view(torch.int16).numpy().view(np.uint16))
    return t.numpy().astype(np.float32)


def host_vals(w, a):
    return bf16_bits_to_f32(a) if w.dtype == "bf16" else a


def layout_of(w):
    return pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, w.num_q_heads,
                              w.num_kv_heads, w.head_dim, w.rope_theta)


def oracle_layout(w):
    return O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)


_cache = {}


def workload_inputs(i):
    if i not in _cache:
        w = make_workload(i)
        _cache.clear()
        _cache[i] = (w, draw_qkv(w))
    return _cache[i]


def poisoned_outputs(q, num_q_heads):
    """O and lse filled with NaN, so any element the kernel does not write shows."""
    T = q.shape[0]
    return (torch.full_like(q, float("nan")),
            torch.full((num_q_heads, T), float("nan"), dtype=torch.float32, device=q.device))


def check_attn(w, o_gpu, lse_gpu, q, k, v, lay, full):
    """Compare GPU (o, lse) with the oracle on every row.

    full=True: the whole oracle in one call (small workloads); "units": every
    row, the oracle run per (group, query head) unit in parallel."""
    Hq = w.num_q_heads
    o_g = to_host_f32(o_gpu)
    l_g = lse_gpu.detach().cpu().numpy()
    # every element written (the outputs were NaN-filled before the launch)
    assert np.isfinite(o_g).all() and np.isfinite(l_g).all()
    if full == "units":
        eo, el, rows = U.max_errors(w, lay, q, k, v, o_g, l_g)
        assert rows == w.total_tokens * Hq
        what = f"all {rows} rows"
    elif full:
        o_ref, l_ref = O.attention(q, k, v, lay, w.softmax_scale, Hq, w.num_kv_heads)
        eo = np.abs(o_g.astype(np.float64) - o_ref).max()
        el = np.abs(l_g.astype(np.float64) - l_ref).max()
        what = f"all {w.total_tokens * Hq} rows"
    else:
        raise ValueError(f"full={full!r}")
    say(f"  {w.name}: {what}: max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= O_TOL, eo
    assert el <= LSE_TOL, el


def parity_mode(i):
    """How much of workload i the oracle checks: everything in one call for
    the small ones, every row in parallel (group, query head) units for GRPO,
    heterogeneous and long-prefix (about a minute for long-prefix on 16 cores)."""
    return True if i <= 1 else "units"


# --------------------------------------------------------------- positions --

@pytest.mark.parametrize("i", range(5))
def test_position_ids_bit_exact(i):
    w = make_workload(i)
    say(f"positions: workload {w.name} T={w.total_tokens}")
    L = layout_of(w)
    pos = pg.pg_position_ids(L)
    torch.cuda.synchronize()
    ref = O.positions(oracle_layout(w))
    assert np.array_equal(pos.cpu().numpy(), ref)


def test_position_ids_edge_shapes():
    for P, S in [([0, 7], [[4, 3], [5]]), ([6, 4, 3], [[], [0, 2], [0, 0]]), ([1], [[1, 1, 1]])]:
        w = make_custom(P, S)
        L = layout_of(w)
        pos = pg.pg_position_ids(L)
        assert np.array_equal(pos.cpu().numpy(), O.positions(oracle_layout(w)))


# -------------------------------------------------------------------- RoPE --

def _rope_compare(w, got, ref_f64):
    if w.dtype == "bf16":
        ref = O.round_to_bf16(ref_f64)
        diff = np.abs(got.astype(np.float64) - ref)
        ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(ref), 1e-30))[1] - 8)
        n_off = int((diff > 0).sum())
        say(f"  rope {w.name}: {n_off} of {diff.size} elements differ by <= 1 ulp")
        assert (diff <= ulp * 1.0000001).all()
        assert n_off <= max(10, diff.size // 1000)
    else:
        assert np.abs(got.astype(np.float64) - ref_f64).max() <= 1e-6


@pytest.mark.parametrize("i", range(5))
def test_rope_against_oracle(i):
    w, qkv = workload_inputs(i)
    say(f"rope: workload {w.name}")
    L = layout_of(w)
    pos = pg.pg_position_ids(L)
    q, k = to_dev(w, qkv["q"]), to_dev(w, qkv["k"])
    qr, kr = pg.pg_rope(L, pos, q, k)
    torch.cuda.synchronize()
    lay = oracle_layout(w)
    opos = O.positions(lay)
    r = np.random.default_rng(5)
    toks = np.unique(np.concatenate([r.integers(0, w.total_tokens, size=512),
                                     [0, w.total_tokens - 1, int(np.argmax(opos))]]))
    q_h = host_vals(w, qkv["q"][toks])
    k_h = host_vals(w, qkv["k"][toks])
    _rope_compare(w, to_host_f32(qr[torch.from_numpy(toks).cuda()]), O.rope(q_h, opos[toks], w.rope_theta))
    _rope_compare(w, to_host_f32(kr[torch.from_numpy(toks).cuda()]), O.rope(k_h, opos[toks], w.rope_theta))


def test_rope_in_place_equals_out_of_place():
    w, qkv = workload_inputs(1)
    L = layout_of(w)
    pos = pg.pg_position_ids(L)
    q, k = to_dev(w, qkv["q"]), to_dev(w, qkv["k"])
    qr, kr = pg.pg_rope(L, pos, q, k)
    q2, k2 = q.clone(), k.clone()
    pg.pg_rope(L, pos, q2, k2, q_out=q2, k_out=k2)
    torch.cuda.synchronize()
    assert torch.equal(q2.view(torch.int16), qr.view(torch.int16))
    assert torch.equal(k2.view(torch.int16), kr.view(torch.int16))


def test_rope_near_cancellation():
    """Rotations whose exact result nearly cancels: x = y tan(phi) rounded to
    bf16 makes x cos - y sin a rounding residual of x, hundreds of times
    smaller than the inputs (and -x / tan(phi) does the same to y cos + x sin
    in the other heads). These are the cases where a rotation in plain fp32
    misses the nearest bf16 by many ulps; the kernel must stay within one."""
    w = make_custom([700, 0], [[300, 0, 450], [260]], num_q_heads=4, num_kv_heads=2)
    L = layout_of(w)
    pos = pg.pg_position_ids(L)
    opos = O.positions(oracle_layout(w))
    T, d = w.total_tokens, w.head_dim
    half = d // 2
    r = np.random.default_rng(11)
    omega = w.rope_theta ** (-2.0 * np.arange(half) / d)
    tan = np.tan(opos[:, None].astype(np.float64) * omega[None, :])[:, None, :]
    ok = (np.abs(tan) <= 8.0) & (np.abs(tan) >= 1.0 / 8.0)

    def make(H):
        a = O.round_to_bf16(r.standard_normal((T, H, half)))
        b = O.round_to_bf16(r.standard_normal((T, H, half)))
        lo = np.where(ok, O.round_to_bf16(a * tan), b)     # lo x cos - hi sin ~ 0 (hi = a)
        x = np.concatenate([lo, a], axis=-1)
        hi = np.where(ok, O.round_to_bf16(-a * tan), b)    # hi x cos + lo sin ~ 0 (lo = a)
        x2 = np.concatenate([a, hi], axis=-1)
        return np.concatenate([x[:, :(H + 1) // 2], x2[:, (H + 1) // 2:]], axis=1)

    qv, kv = make(w.num_q_heads), make(w.num_kv_heads)
    ref_q, ref_k = O.rope(qv, opos, w.rope_theta), O.rope(kv, opos, w.rope_theta)
    # the cancelling outputs really are small next to their inputs
    m = np.broadcast_to(ok, ref_q[:, :1, :half].shape)
    assert np.median(np.abs(ref_q[:, :1, :half])[m] / np.abs(qv[:, :1, half:])[m]) < 2.0 ** -6
    bits = lambda v: f32_to_bf16_bits(v.astype(np.float32))
    q, k = to_dev(w, bits(qv)), to_dev(w, bits(kv))
    qr, kr = pg.pg_rope(L, pos, q, k)
    torch.cuda.synchronize()
    _rope_compare(w, to_host_f32(qr), ref_q)
    _rope_compare(w, to_host_f32(kr), ref_k)


# --------------------------------------------------------------- attention --

@pytest.mark.parametrize("i", range(5))
def test_attention_against_oracle(i):
    """pg_attn_fwd alone, fed exactly the oracle's Q/K/V."""
    w, qkv = workload_inputs(i)
    say(f"attn: workload {w.name} T={w.total_tokens} heads={w.num_q_heads}/{w.num_kv_heads}")
    L = layout_of(w)
    q, k, v = (to_dev(w, qkv[n]) for n in ("q", "k", "v"))
    o, lse = poisoned_outputs(q, w.num_q_heads)
    pg.pg_attn_fwd(L, q, k, v, w.softmax_scale, o=o, lse=lse)
    torch.cuda.synchronize()
    lay = oracle_layout(w)
    check_attn(w, o, lse, host_vals(w, qkv["q"]), host_vals(w, qkv["k"]),
               host_vals(w, qkv["v"]), lay, full=parity_mode(i))


@pytest.mark.parametrize("i", range(5))
def test_pipeline_against_oracle(i):
    """positions -> RoPE -> attention, against the oracle pipeline (RoPE output
    rounded to the storage dtype where the GPU hands it over), on every row
    of every workload (the heterogeneous one mixes unshared and shared groups
    on a 1024-token prompt)."""
    w, qkv = workload_inputs(i)
    say(f"pipeline: workload {w.name}")
    L = layout_of(w)
    pos = pg.pg_position_ids(L)
    q, k, v = (to_dev(w, qkv[n]) for n in ("q", "k", "v"))
    qr, kr = pg.pg_rope(L, pos, q, k)
    o, lse = poisoned_outputs(q, w.num_q_heads)
    pg.pg_attn_fwd(L, qr, kr, v, w.softmax_scale, o=o, lse=lse)
    torch.cuda.synchronize()
    del qr, kr
    lay = oracle_layout(w)
    opos = O.positions(lay)
    qh, kh, vh = (host_vals(w, qkv[n]) for n in ("q", "k", "v"))
    k_ref = O.storage_round(O.rope(kh, opos, w.rope_theta), w.dtype).astype(np.float32)
    # bf16-rounded values are exact in float32
    q_ref = O.storage_round(O.rope(qh, opos, w.rope_theta), w.dtype).astype(np.float32)
    del qh
    check_attn(w, o, lse, q_ref, k_ref, vh, lay, full=parity_mode(i))


def test_attention_one_long_group():
    """One group far longer than any workload's: a 60000-token prompt and three
    responses (3000, 1 and 2500 tokens), 8 query heads on one KV head, so one
    (group, KV head) cluster spans about a thousand work items and a response
    row's prompt span about 940 key tiles. Every output is written (NaN
    poison); sampled rows (both ends of the prompt and of every response,
    64-token block edges, random) against the oracle's per-row definition."""
    w = make_custom([60000], [[3000, 1, 2500]], num_q_heads=8, num_kv_heads=1, seed=7)
    x = draw_qkv(w)
    L = layout_of(w)
    q, k, v = (to_dev(w, x[n]) for n in ("q", "k", "v"))
    o, lse = poisoned_outputs(q, w.num_q_heads)
    pg.pg_attn_fwd(L, q, k, v, w.softmax_scale, o=o, lse=lse)
    torch.cuda.synchronize()
    o_g, l_g = to_host_f32(o), lse.cpu().numpy()
    assert np.isfinite(o_g).all() and np.isfinite(l_g).all()
    T = w.total_tokens
    r = np.random.default_rng(17)
    tokens = {0, 1, 63, 64, 30000, 59999, 60000, 60001, 62999, 63000, 63001, 63002, T - 1}
    tokens = sorted(tokens | {int(t) for t in r.integers(0, T, size=240)})
    heads = [int(h) for h in r.integers(0, w.num_q_heads, size=len(tokens))]
    qh, kh, vh = (host_vals(w, x[n]) for n in ("q", "k", "v"))
    ro, rl = O.attention_rows(qh, kh, vh, oracle_layout(w), w.softmax_scale, w.num_q_heads,
                              w.num_kv_heads, tokens, heads)
    eo = np.abs(o_g[tokens, heads].astype(np.float64) - ro).max()
    el = np.abs(l_g[heads, tokens].astype(np.float64) - rl).max()
    say(f"  one long group (T={T}): {len(tokens)} sampled rows: max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= O_TOL and el <= LSE_TOL


EDGE = [
    # prefix lens, suffix lens, (Hq, Hkv), d
    ([0, 7], [[4, 3], [5]], (4, 1), 128),
    ([6, 4, 3], [[], [0, 2], [0, 0]], (4, 1), 128),
    ([1], [[1, 1, 1]], (8, 2), 128),
    ([31, 33, 64], [[32, 1], [63, 65], [128, 129, 127]], (32, 8), 128),
    ([65, 127, 129], [[64, 63], [1], [200, 0, 31]], (64, 8), 128),
    ([300], [[1, 40, 0, 200, 33]], (2, 2), 128),
    ([100, 0], [[70, 90], [33, 97]], (6, 2), 128),
    ([45], [[19, 77, 3]], (3, 1), 128),
    ([0], [[0, 130, 0]], (1, 1), 128),
    ([200], [[]], (4, 4), 128),
    ([37, 80], [[20, 9], [64]], (4, 2), 64),     # bf16, d = 64: per-row kernel
]


@pytest.mark.parametrize("case", range(len(EDGE)))
def test_attention_edge_shapes(case):
    P, S, (hq, hkv), d = EDGE[case]
    w = make_custom(P, S, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, seed=case)
    say(f"attn edge case {case}: P={P} S={S} heads={hq}/{hkv} d={d}")
    qkv = draw_qkv(w)
    L = layout_of(w)
    q, k, v = (to_dev(w, qkv[n]) for n in ("q", "k", "v"))
    o, lse = pg.pg_attn_fwd(L, q, k, v, w.softmax_scale)
    torch.cuda.synchronize()
    if w.total_tokens == 0:
        return
    check_attn(w, o, lse, host_vals(w, qkv["q"]), host_vals(w, qkv["k"]),
               host_vals(w, qkv["v"]), oracle_layout(w), full=True)


def test_attention_fp32_edge_shapes():
    for case, (P, S, (hq, hkv), d) in enumerate(EDGE[:4]):
        w = make_custom(P, S, num_q_heads=hq, num_kv_heads=hkv, head_dim=64, dtype="f32",
                        seed=case)
        say(f"attn fp32 edge case {case}")
        qkv = draw_qkv(w)
        L = layout_of(w)
        q, k, v = (to_dev(w, qkv[n]) for n in ("q", "k", "v"))
        o, lse = pg.pg_attn_fwd(L, q, k, v, w.softmax_scale)
        torch.cuda.synchronize()
        o_ref, l_ref = O.attention(qkv["q"], qkv["k"], qkv["v"], oracle_layout(w),
                                   w.softmax_scale, hq, hkv)
        assert np.abs(o.cpu().numpy() - o_ref).max() <= 1e-5
        assert np.abs(lse.cpu().numpy() - l_ref).max() <= 1e-5


def test_empty_layout_launches_nothing():
    w = make_custom([0, 0], [[0], []])
    L = layout_of(w)
    z = torch.empty((0, 4, 128), dtype=torch.bfloat16, device="cuda")
    zk = torch.empty((0, 1, 128), dtype=torch.bfloat16, device="cuda")
    o, lse = pg.pg_attn_fwd(L, z, zk, zk, 0.1)
    pos = pg.pg_position_ids(L)
    assert o.shape[0] == 0 and pos.shape[0] == 0


# -------------------------------------------------------------- robustness --

def test_deterministic_and_fully_written():
    w, qkv = workload_inputs(1)
    say("determinism / poison: workload dpo-bf16")
    L = layout_of(w)
    q, k, v = (to_dev(w, qkv[n]) for n in ("q", "k", "v"))
    T, Hq, d = q.shape
    o1 = torch.full_like(q, float("nan"))
    l1 = torch.full((Hq, T), float("nan"), device="cuda")
    pg.pg_attn_fwd(L, q, k, v, w.softmax_scale, o=o1, lse=l1)
    o2 = torch.full_like(q, float("inf"))
    l2 = torch.full((Hq, T), float("inf"), device="cuda")
    pg.pg_attn_fwd(L, q, k, v, w.softmax_scale, o=o2, lse=l2)
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_no_writes_past_outputs():
    w, qkv = workload_inputs(1)
    L = layout_of(w)
    q, k, v = (to_dev(w, qkv[n]) for n in ("q", "k", "v"))
    T, Hq, d = q.shape
    pad = 4096
    obuf = torch.full((T * Hq * d + pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((Hq * T + pad,), 7.0, dtype=torch.float32, device="cuda")
    o = obuf[:T * Hq * d].view(T, Hq, d)
    lse = lbuf[:Hq * T].view(Hq, T)
    pg.pg_attn_fwd(L, q, k, v, w.softmax_scale, o=o, lse=lse)
    pos = torch.full((T + pad,), -3, dtype=torch.int64, device="cuda")
    pg.pg_position_ids(L, pos=pos[:T])
    torch.cuda.synchronize()
    assert (obuf[T * Hq * d:] == 7.0).all() and (lbuf[Hq * T:] == 7.0).all()
    assert (pos[T:] == -3).all()


def test_packed_equals_unpacked_on_gpu():
    """The same kernel on the unpacked layout (prefix duplicated per suffix)
    gives the packed rows back: preference packing changes no result."""
    from shared_prefix_packed_amd.baseline import unpacked_workload
    w, qkv = workload_inputs(1)
    say("packed vs unpacked on the GPU: workload dpo-bf16")
    L = layout_of(w)
    q, k, v = (to_dev(w, qkv[n]) for n in ("q", "k", "v"))
    o, lse = pg.pg_attn_fwd(L, q, k, v, w.softmax_scale)
    un = unpacked_workload(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    idx = torch.from_numpy(un.gather).cuda()
    Lu = pg.pg_build_layout(un.prefix_lens, un.suffix_counts, un.suffix_lens, w.num_q_heads,
                            w.num_kv_heads, w.head_dim, w.rope_theta)
    ou, lu = pg.pg_attn_fwd(Lu, q[idx].contiguous(), k[idx].contiguous(), v[idx].contiguous(),
                            w.softmax_scale)
    torch.cuda.synchronize()
    # every unpacked row maps to one packed row; compare all of them
    d_o = (ou.float() - o[idx].float()).abs().max().item()
    d_l = (lu - lse[:, idx]).abs().max().item()
    say(f"  unpacked vs packed: max|dO|={d_o:.3e} max|dlse|={d_l:.3e}")
    assert d_o <= 2 * O_TOL and d_l <= 2 * LSE_TOL


def test_layouts_destroyed_while_work_is_in_flight():
    """pg_layout_destroy returns at once and recycles the upload buffer only
    after the enqueued work that reads it has finished: layouts of different
    sizes built and destroyed behind a long-running kernel all give the
    oracle's results."""
    shapes = [([5, 9], [[3, 4], [2, 6, 1]]), ([300], [[1, 40, 0, 200, 33]]),
              ([31, 33, 64], [[32, 1], [63, 65], [128, 129, 127]]), ([0, 7], [[4, 3], [5]])]
    a = torch.randn(4096, 4096, device="cuda")
    say("layout recycling: 12 layouts destroyed behind a busy stream")
    outs = []
    for rep in range(3):
        b = a @ a          # keeps the stream busy while the layouts below are recycled
        for P, S in shapes:
            w = make_custom(P, S, num_q_heads=4, num_kv_heads=1)
            L = layout_of(w)
            pos = pg.pg_position_ids(L)
            qkv = draw_qkv(w)
            q, k, v = (to_dev(w, qkv[n]) for n in ("q", "k", "v"))
            o, lse = pg.pg_attn_fwd(L, q, k, v, w.softmax_scale)
            L.close()
            outs.append((w, qkv, pos, o, lse))
    torch.cuda.synchronize()
    del b
    for w, qkv, pos, o, lse in outs:
        lay = oracle_layout(w)
        assert np.array_equal(pos.cpu().numpy(), O.positions(lay))
        check_attn(w, o, lse, host_vals(w, qkv["q"]), host_vals(w, qkv["k"]),
                   host_vals(w, qkv["v"]), lay, full=True)
