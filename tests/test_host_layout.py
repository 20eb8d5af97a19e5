"""CPU tests of libpg.so's host side: exported symbols, the layout builder
against the oracle (bit-exact), work-list invariants and error paths.

No compute entry point is called here (there is no GPU in this run)."""
import ctypes
import os
import re

import numpy as np
import pytest

import shared_prefix_packed_amd as pg
from shared_prefix_packed_amd import _lib
from conftest import ROOT, read_golden
from oracle import pg_oracle as O
from workloads import make_workload

SHAPES = [
    ([5, 9], [[3, 4], [2, 6, 1]]),
    ([0, 7], [[4, 3], [5]]),
    ([6, 4, 3], [[], [0, 2], [0, 0]]),
    ([1], [[1, 1, 1]]),
    ([31, 33, 64], [[32, 1], [63, 65], [128, 129, 127]]),
    ([0], [[0, 3, 0]]),
    ([17], [[]]),
    ([300], [[1, 40, 0, 200, 33]]),
    ([], []),
    ([0, 0], [[0], []]),
]


def _flat(S):
    return [len(s) for s in S], [x for s in S for x in s]


def _build(P, S, hq=4, hkv=1, d=128, theta=1e4):
    n, flat = _flat(S)
    return pg.pg_build_layout_host(P, n, flat, hq, hkv, d, theta)


def test_library_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "pg.h")).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[\w]+\**\s+\**(pg_\w+)\s*\(", header, re.M))
    assert {"pg_build_layout", "pg_position_ids", "pg_rope", "pg_attn_fwd"} <= declared
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(_lib.SIGNATURES), "binding and header disagree"


@pytest.mark.parametrize("shape", SHAPES)
def test_layout_bit_exact_against_oracle(shape):
    P, S = shape
    n, flat = _flat(S)
    L = _build(P, S)
    lay = O.layout(P, n, flat)
    g, seg = L.offsets()
    assert g.tolist() == lay["group_off"].tolist()
    assert seg.tolist() == lay["seg_off"].tolist()
    g0, pe, ss = L.tokens()
    assert g0.tolist() == lay["g0"].tolist()
    assert pe.tolist() == lay["pe"].tolist()
    assert ss.tolist() == lay["ss"].tolist()
    s = L.summary()
    assert s.total_tokens == lay["total_tokens"]
    assert s.useful_pairs == O.useful_pairs(lay)
    assert s.unpacked_pairs == O.unpacked_pairs(lay)
    pos = O.positions(lay)
    assert s.max_position == (int(pos.max()) if pos.size else -1)
    assert s.device_ready == 0


def test_tiny_workload_against_hand_derivation():
    gold = read_golden("tiny_layout.txt")
    w = make_workload(0)
    L = pg.pg_build_layout_host(w.prefix_lens, w.suffix_counts, w.suffix_lens, 1, 1, 64, 1e4)
    g, seg = L.offsets()
    assert g.tolist() == gold["group_off"] and seg.tolist() == gold["seg_off"]
    assert L.summary().useful_pairs == gold["useful_pairs"][0]
    assert L.summary().unpacked_pairs == gold["unpacked_pairs"][0]


XCDS = 8


def _check_work_invariants(L, P, S, hq, hkv):
    n, flat = _flat(S)
    lay = O.layout(P, n, flat)
    T = lay["total_tokens"]
    r = hq // hkv
    items, spans = L.work()
    s = L.summary()
    hpw = s.heads_per_item
    assert hpw == np.gcd(r, 8)
    assert s.block_tokens == 256 // hpw
    cover = np.zeros((T, hq), dtype=np.int64)
    total_cost = 0
    xcd_of_cluster = {}
    xcd_cost = np.zeros(XCDS, dtype=np.int64)
    last = {}   # per XCD: (cluster, cost) of the previous real item
    seen_done = set()
    for p, it in enumerate(items):
        if it["nspan"] == 0:
            assert it["cost"] == 0 and it["t1"] == it["t0"] and it["ntiles"] == 0
            continue
        t0, t1, hq0 = int(it["t0"]), int(it["t1"]), int(it["hq0"])
        assert 0 < t1 - t0 <= s.block_tokens
        assert int(lay["g0"][t0]) == int(lay["g0"][t1 - 1]), "item crosses a group"
        assert it["pe"] == lay["pe"][t0]
        assert hq0 // r == (hq0 + hpw - 1) // r, "item mixes KV heads"
        cover[t0:t1, hq0:hq0 + hpw] += 1
        # spans: disjoint, ascending, inside the group; their union equals the
        # union of the allowed keys of the item's tokens
        sp = spans[it["span0"]:it["span0"] + it["nspan"]]
        # the tile count and the copy of the first span the kernel starts from
        assert it["ntiles"] == sum((k1 - k0 + 63) // 64 for k0, k1 in sp)
        assert (it["k0"], it["k1"]) == tuple(sp[0])
        keys = set()
        prev = -1
        for k0, k1 in sp:
            assert k0 < k1 and k0 >= prev
            prev = k1
            keys.update(range(k0, k1))
        need = set()
        pairs = 0
        for t in range(t0, t1):
            kt = O.allowed_keys(lay, t)
            need.update(kt.tolist())
            pairs += len(kt)
        assert keys == need
        assert it["cost"] == pairs * hpw and it["cost"] >= 1
        total_cost += int(it["cost"])
        # launch order: a (group, KV head) cluster lives on one XCD, runs as one
        # contiguous stretch of that XCD's queue, cost-descending inside it
        x = p % XCDS
        cl = (int(lay["g0"][t0]), hq0 // r)
        assert xcd_of_cluster.setdefault(cl, x) == x
        xcd_cost[x] += int(it["cost"])
        if x in last:
            pcl, pcost = last[x]
            if pcl == cl:
                assert it["cost"] <= pcost
            else:
                assert cl not in seen_done, "cluster split in its XCD queue"
                seen_done.add(pcl)
        last[x] = (cl, int(it["cost"]))
    assert (cover == 1).all(), "every (token, head) in exactly one item"
    assert total_cost == O.useful_pairs(lay) * hq
    real = items[items["nspan"] > 0]
    assert s.max_item_cost == (int(real["cost"].max()) if real.size else 0)
    assert s.max_xcd_cost == int(xcd_cost.max())
    assert items.size == 0 or items[-1]["nspan"] > 0, "no trailing padding"
    return xcd_cost


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("heads", [(4, 1), (32, 8), (64, 8), (2, 2), (6, 2), (3, 1)])
def test_work_list_invariants(shape, heads):
    P, S = shape
    L = _build(P, S, hq=heads[0], hkv=heads[1])
    _check_work_invariants(L, P, S, *heads)


def test_work_list_on_dpo_workload():
    w = make_workload(1)
    L = pg.pg_build_layout_host(w.prefix_lens, w.suffix_counts, w.suffix_lens, 32, 8, 128, 5e5)
    P = w.prefix_lens.tolist()
    S = [s for _, s in w.groups()]
    cost = _check_work_invariants(L, P, S, 32, 8)
    # LPT over 64 clusters: the heaviest XCD within 10 % of the mean
    assert cost.max() <= 1.10 * cost.mean()


@pytest.mark.parametrize("i", [2, 3, 4])
def test_xcd_balance_of_large_workloads(i):
    w = make_workload(i)
    L = pg.pg_build_layout_host(w.prefix_lens, w.suffix_counts, w.suffix_lens,
                                w.num_q_heads, w.num_kv_heads, w.head_dim, w.rope_theta)
    items, _ = L.work()
    real = items[items["nspan"] > 0]
    mean = real["cost"].sum() / 8
    assert L.summary().max_xcd_cost <= 1.10 * mean
    # padding stays small next to the real items
    assert (items["nspan"] == 0).sum() <= 0.25 * real.size


def test_layouts_of_all_workloads_match_oracle_counts():
    for i in range(5):
        w = make_workload(i)
        L = pg.pg_build_layout_host(w.prefix_lens, w.suffix_counts, w.suffix_lens,
                                    w.num_q_heads, w.num_kv_heads, w.head_dim, w.rope_theta)
        lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
        s = L.summary()
        assert s.total_tokens == w.total_tokens
        assert s.useful_pairs == O.useful_pairs(lay)
        g, seg = L.offsets()
        assert g.tolist() == lay["group_off"].tolist()
        assert seg.tolist() == lay["seg_off"].tolist()
        items, _ = L.work()
        assert int(items["cost"].sum()) == O.useful_pairs(lay) * w.num_q_heads


# ----------------------------------------------------------- error paths --

def _status(fn, *args):
    try:
        fn(*args)
    except pg.PgError as e:
        return e.status
    return 0


@pytest.mark.parametrize("args,status", [
    (([5], [1], [-1], 4, 1, 128, 1e4), -1),       # negative suffix
    (([-5], [1], [1], 4, 1, 128, 1e4), -1),       # negative prefix
    (([5], [-1], [], 4, 1, 128, 1e4), -1),        # negative count
    (([5], [1], [3], 6, 4, 128, 1e4), -1),        # Hq % Hkv != 0
    (([5], [1], [3], 0, 1, 128, 1e4), -1),        # no heads
    (([5], [1], [3], 4, 1, 96, 1e4), -2),         # unsupported head_dim
    (([5], [1], [3], 4, 1, 128, 0.0), -1),        # theta
    (([2**30, 2**30], [0, 0], [], 4, 1, 128, 1e4), -1),   # T >= 2^31
    (([2**30 - 1], [1], [2], 4, 1, 128, 1e4), -1),        # T = 2^30 + 1: one past the limit
])
def test_invalid_arguments_are_reported(args, status):
    assert _status(pg.pg_build_layout_host, *args) == status


def test_null_pointers_are_reported():
    lib = _lib.load()
    out = ctypes.c_void_p()
    P = (ctypes.c_int32 * 1)(3)
    assert lib.pg_build_layout_host(1, None, P, None, 1, 1, 64, 1e4, ctypes.byref(out)) == -1
    assert b"NULL" in lib.pg_last_error()
    n = (ctypes.c_int32 * 1)(1)
    assert lib.pg_build_layout_host(1, P, n, None, 1, 1, 64, 1e4, ctypes.byref(out)) == -1
    assert lib.pg_build_layout_host(1, P, n, P, 1, 1, 64, 1e4, None) == -1
    assert lib.pg_layout_info(None, None) == -1
    assert lib.pg_position_ids(None, None, None) == -1
    assert lib.pg_attn_fwd(None, None, None, None, None, None, 1, ctypes.c_float(1.0), None) == -1


def test_compute_calls_need_an_uploaded_layout():
    lib = _lib.load()
    L = _build([5], [[3]])
    dummy = ctypes.c_void_p(16)
    assert lib.pg_position_ids(L.handle, dummy, None) == -5
    assert lib.pg_rope(L.handle, dummy, dummy, dummy, dummy, dummy, 1, None) == -5
    assert lib.pg_attn_fwd(L.handle, dummy, dummy, dummy, dummy, None, 1, ctypes.c_float(0.1), None) == -5
    assert lib.pg_status_string(-5) == b"bad state"


def test_empty_layout_is_a_no_op():
    lib = _lib.load()
    L = _build([], [])
    s = L.summary()
    assert s.total_tokens == 0 and s.num_items == 0 and s.max_position == -1
    L2 = _build([0, 0], [[0], []])
    assert L2.summary().total_tokens == 0


# ------------------------------------------------------ backward work list --

def _check_kv_invariants(L, P, S, hq, hkv):
    n, flat = _flat(S)
    lay = O.layout(P, n, flat)
    T = lay["total_tokens"]
    r = hq // hkv
    grp, seg, _ = O.segment_ids(lay)
    # readers of each key, counted from the oracle's key sets
    readers = np.zeros(T, dtype=np.int64)
    last_reader = np.full(T, -1, dtype=np.int64)
    for t in range(T):
        for j in O.allowed_keys(lay, t):
            readers[j] += 1
            last_reader[j] = max(last_reader[j], t)
    kv = L.kv_work()
    assert L.summary().num_kv_items == kv.size
    cover = np.zeros((T, hkv), dtype=np.int64)
    xcd_of_cluster = {}
    for p, it in enumerate(kv):
        k0, k1, hk, qend = int(it["k0"]), int(it["k1"]), int(it["hk"]), int(it["qend"])
        if k1 <= k0:
            assert it["cost"] == 0
            continue
        assert k1 - k0 <= 128 and 0 <= hk < hkv
        assert grp[k0] == grp[k1 - 1] and seg[k0] == seg[k1 - 1], "block crosses a segment"
        cover[k0:k1, hk] += 1
        # every reader of these keys lies in [k0, qend), and qend is reached
        assert last_reader[k0:k1].max() == qend - 1
        assert it["cost"] == readers[k0:k1].sum() * r
        cl = (int(grp[k0]), hk)
        assert xcd_of_cluster.setdefault(cl, p % 8) == p % 8
    assert (cover == 1).all(), "every (key, KV head) in exactly one block"
    assert kv.size == 0 or kv[-1]["k1"] > kv[-1]["k0"], "no trailing padding"


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("heads", [(4, 1), (32, 8), (6, 2)])
def test_backward_work_list_invariants(shape, heads):
    P, S = shape
    L = _build(P, S, hq=heads[0], hkv=heads[1])
    _check_kv_invariants(L, P, S, *heads)


def test_backward_work_list_on_dpo_workload():
    w = make_workload(1)
    L = pg.pg_build_layout_host(w.prefix_lens, w.suffix_counts, w.suffix_lens, 32, 8, 128, 5e5)
    _check_kv_invariants(L, w.prefix_lens.tolist(), [s for _, s in w.groups()], 32, 8)


def test_backward_needs_an_uploaded_layout():
    """Every dtype and head size has a backward (bf16 d = 128 on the MFMA
    kernels, the rest per row); without a device copy the call is refused."""
    lib = _lib.load()
    L = _build([5], [[3]], hq=4, hkv=1, d=64)
    dummy = ctypes.c_void_p(16)
    args = [dummy] * 10
    assert lib.pg_attn_bwd(L.handle, *args, 1, ctypes.c_float(0.1), None) == -5   # not uploaded
    assert lib.pg_attn_bwd(None, *args, 1, ctypes.c_float(0.1), None) == -1


def test_pack_and_unpack_argument_errors():
    lib = _lib.load()
    L = _build([5], [[3]])
    dummy = ctypes.c_void_p(16)
    # not uploaded yet
    assert lib.pg_pack_rows(L.handle, dummy, 8, dummy, 8, dummy, 16, None) == -5
    assert lib.pg_unpack_rows(L.handle, dummy, 16, dummy, 8, dummy, 8, None) == -5
    E = _build([], [])   # no tokens: argument checks still apply
    assert lib.pg_pack_rows(E.handle, None, 0, None, 0, None, 6, None) == -1   # not a multiple of 4
    assert lib.pg_unpack_rows(E.handle, None, 0, None, 0, None, 0, None) == -1


# -------------------------------------------------------- decode work list --

def _check_decode_invariants(L, P, S, hq, hkv, d=128):
    n, flat = _flat(S)
    lay = O.layout(P, n, flat)
    T, N, r = int(lay["total_tokens"]), len(flat), hq // hkv
    group_off = np.asarray(lay["group_off"])
    items, off, refs = L.decode_work()
    s = L.summary()
    assert s.num_dec_items == items.size and s.num_dec_refs == refs.size
    assert off.size == N * hkv + 1 and off[0] == 0 and off[-1] == refs.size
    assert L.decode_workspace_size() == items.size * 32 * (d + 2) * 4
    resp_group = O.response_group(lay)
    cov = np.zeros((N * r, hkv, T), dtype=np.int64)
    xcd_of_chunk = {}
    for p, it in enumerate(items):
        k0, k1, hk, resp = int(it["k0"]), int(it["k1"]), int(it["hk"]), int(it["resp"])
        seg0, seg1, row0, nrow = int(it["seg0"]), int(it["seg1"]), int(it["row0"]), int(it["nrow"])
        if nrow == 0:
            assert (k0, k1, hk, resp, seg0, seg1, row0) == (0, 0, 0, -1, 0, 0, 0)
            continue
        assert 1 <= nrow <= 32 and 0 <= hk < hkv
        # pieces of at most 512 rows; of a prompt longer than 4096 rows, 1024
        most = 1024 if (resp < 0 and seg1 - seg0 > 4096) else 512
        assert seg0 <= k0 < k1 <= seg1 and k1 - k0 <= most and (k0 - seg0) % 32 == 0
        if resp < 0:
            g = int(np.searchsorted(group_off, seg0, side="right") - 1)
            assert seg0 == group_off[g] and seg1 == group_off[g] + P[g]
            members = np.nonzero(resp_group == g)[0]
            assert members.size > 0
            assert members[0] * r <= row0 and row0 + nrow <= (members[-1] + 1) * r
        else:
            g = int(resp_group[resp])
            assert seg0 == int(lay["seg_off"][g + resp + 1]) and seg1 - seg0 == flat[resp]
            assert resp * r <= row0 and row0 + nrow <= (resp + 1) * r
        cov[row0:row0 + nrow, hk, k0:k1] += 1
        assert xcd_of_chunk.setdefault((k0, k1, hk), p % 8) == p % 8, "row blocks split over XCDs"
    caps = np.asarray(flat, dtype=np.int64)
    for k in range(N):
        want = np.zeros(T, dtype=np.int64)
        want[O.decode_key_rows(lay, caps, k)] = 1
        for i in range(r):
            for hk in range(hkv):
                assert np.array_equal(cov[k * r + i, hk], want), (k, i, hk)
        for hk in range(hkv):
            got = set(refs[off[k * hkv + hk]:off[k * hkv + hk + 1]].tolist())
            exp = {p for p, it in enumerate(items) if it["nrow"] > 0 and it["hk"] == hk
                   and it["row0"] < (k + 1) * r and it["row0"] + it["nrow"] > k * r}
            assert got == exp, (k, hk)
    assert items.size == 0 or items[-1]["nrow"] > 0, "no trailing padding"


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("heads", [(4, 1), (32, 8), (6, 2), (64, 1), (3, 3)])
def test_decode_work_list_invariants(shape, heads):
    P, S = shape
    L = _build(P, S, hq=heads[0], hkv=heads[1])
    _check_decode_invariants(L, P, S, *heads)


def test_decode_work_list_on_long_segments():
    # a 1500-row prompt (balanced chunks of at most 512 rows) with 10 responses
    # of 4 query heads each (40 rows: two row blocks per prompt chunk)
    P, S = [1500], [[700, 3, 0, 64, 65, 1, 2, 3, 4, 513]]
    L = _build(P, S, hq=8, hkv=2)
    _check_decode_invariants(L, P, S, 8, 2)
    items, _, _ = L.decode_work()
    real = items[items["nrow"] > 0]
    # chunks of one segment and KV head: all but the last of one length, a
    # multiple of 32, the last no longer
    for s0 in set(real["seg0"].tolist()):
        seg = real[(real["seg0"] == s0) & (real["hk"] == 0)]
        starts = sorted(set(seg["k0"].tolist()))
        ends = sorted(set(seg["k1"].tolist()))
        sizes = [e - b for b, e in zip(starts, ends)]
        assert all(x == sizes[0] and x % 32 == 0 for x in sizes[:-1]) and sizes[-1] <= sizes[0]
    # the chunk length aims at about 1024 items: 2855 rows x 2 KV heads -> 64
    assert int((real["k1"] - real["k0"]).max()) == 64


def test_decode_work_list_long_prompt_pieces():
    # a prompt longer than 4096 rows is cut into pieces of up to 1024 rows
    # (10000 rows: ten balanced pieces of 1024, the last 784); its responses
    # keep the ordinary chunk length
    P, S = [10000], [[300, 700]]
    L = _build(P, S, hq=8, hkv=2)
    _check_decode_invariants(L, P, S, 8, 2)
    items, _, _ = L.decode_work()
    real = items[(items["nrow"] > 0) & (items["hk"] == 0)]
    prompt = real[real["resp"] < 0]
    sizes = sorted(set((prompt["k1"] - prompt["k0"]).tolist()))
    assert sizes == [784, 1024]
    resp = real[real["resp"] >= 0]
    assert int((resp["k1"] - resp["k0"]).max()) <= 512


def test_decode_work_list_on_dpo_workload():
    w = make_workload(1)
    L = pg.pg_build_layout_host(w.prefix_lens, w.suffix_counts, w.suffix_lens, 32, 8, 128, 5e5)
    _check_decode_invariants(L, w.prefix_lens.tolist(), [s for _, s in w.groups()], 32, 8)


def test_decode_argument_errors():
    lib = _lib.load()
    L = _build([5], [[3]])
    dummy = ctypes.c_void_p(16)
    f = ctypes.c_float
    args = lambda scale: [dummy] * 7 + [ctypes.c_size_t(1 << 20), 1, f(scale), None]
    assert lib.pg_attn_decode(L.handle, *args(0.1)) == -5          # not uploaded
    assert lib.pg_attn_decode(None, *args(0.1)) == -1
    E = _build([0, 0], [[0], []])        # no tokens, one response: argument checks still apply
    assert lib.pg_attn_decode(E.handle, *args(0.0)) == -1           # scale
    assert lib.pg_attn_decode(E.handle, None, None, None, None, None, None, None,
                              ctypes.c_size_t(0), 1, f(0.1), None) == -1   # NULL tensors
    assert lib.pg_attn_decode(E.handle, *([dummy] * 7), ctypes.c_size_t(0), 7, f(0.1), None) == -1
    n = ctypes.c_size_t(123)
    assert lib.pg_decode_workspace_size(E.handle, ctypes.byref(n)) == 0 and n.value == 0
    assert lib.pg_decode_workspace_size(None, ctypes.byref(n)) == -1


def test_single_pair_rope_argument_errors():
    lib = _lib.load()
    dummy = ctypes.c_void_p(16)
    L = _build([5], [[3]])
    assert lib.pg_rope(L.handle, dummy, None, dummy, None, dummy, 1, None) == -5   # not uploaded
    E = _build([0, 0], [[0], []])   # no tokens: a no-op whatever is passed
    assert lib.pg_rope(E.handle, dummy, None, dummy, None, dummy, 1, None) == 0
    lay = pg.pg_build_layout_host([5], [1], [3], 4, 1, 128, 1e4)
    # argument checks need a device copy; they are exercised on the GPU
    assert lib.pg_rope(lay.handle, dummy, None, None, None, None, 1, None) == -5


@pytest.mark.parametrize("shape", SHAPES)
def test_max_group_len_matches_oracle(shape):
    P, S = shape
    L = _build(P, S)
    n, flat = _flat(S)
    gl = O.group_lens(O.layout(P, n, flat))
    assert L.summary().max_group_len == (int(gl.max()) if gl.size else 0)
    assert L.summary().reserved == 0


def test_padded_form_argument_errors():
    lib = _lib.load()
    dummy = ctypes.c_void_p(16)
    L = _build([5], [[3]])
    assert lib.pg_position_ids_padded(L.handle, 8, dummy, None, None) == -5   # not uploaded
    assert lib.pg_pad_rows(L.handle, dummy, 16, dummy, 8, None) == -5
    assert lib.pg_unpad_rows(L.handle, dummy, 8, 16, dummy, None) == -5
    E = _build([0, 0], [[0], []])   # no tokens: argument checks still apply
    assert lib.pg_pad_rows(E.handle, None, 6, dummy, 4, None) == -1          # row bytes
    assert lib.pg_unpad_rows(E.handle, None, 4, 0, None, None) == -1         # row bytes
    assert lib.pg_position_ids_padded(E.handle, -1, dummy, None, None) == -1  # width
    assert lib.pg_position_ids_padded(None, 4, dummy, None, None) == -1
