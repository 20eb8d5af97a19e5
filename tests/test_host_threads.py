"""The host library from several threads at once (ctypes releases the GIL
around each call, so the calls really overlap).

* Every thread sees its own error text: the last-error slot is per thread, so
  a thread whose call failed reads its own message even while other threads'
  calls fail or succeed.
* Layouts built concurrently equal the same layouts built one after another
  (offsets, per-token descriptors and the forward work list).
"""
import threading

import numpy as np
import pytest

import shared_prefix_packed_amd as pg
from workloads import make_workload

# (arguments of pg_build_layout_host, a piece of the error text it must give)
BAD = [
    (([5, -1], [1, 0], [3], 8, 2, 128, 1e4), "prefix_lens[1] < 0"),
    (([5], [1], [3], 6, 4, 128, 1e4), "not a multiple of Hkv"),
    (([5], [1], [3], 8, 2, 96, 1e4), "head_dim 96 not supported"),
    (([5], [2], [3, -4], 8, 2, 128, 1e4), "suffix_lens[1] < 0"),
    (([5], [1], [3], 8, 2, 128, -1.0), "rope_theta"),
]


def test_each_thread_reads_its_own_error():
    failures = []
    barrier = threading.Barrier(len(BAD) * 2)

    def worker(args, text, also_valid):
        barrier.wait()
        for _ in range(200):
            try:
                pg.pg_build_layout_host(*args).close()
                failures.append(f"{text}: no error")
                return
            except pg.PgError as e:
                if text not in str(e):
                    failures.append(f"expected '{text}', got '{e}'")
                    return
            if also_valid:   # a successful call between failures must not disturb others
                pg.pg_build_layout_host([7, 3], [2, 1], [4, 5, 6], 8, 2, 128, 1e4).close()

    threads = [threading.Thread(target=worker, args=(a, t, v)) for a, t in BAD for v in (False, True)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not failures, failures[:5]


def snapshot(L):
    go, so = L.offsets()
    g0, pe, ss = L.tokens()
    it, sp = L.work()
    return [np.asarray(x).copy() for x in (go, so, g0, pe, ss, sp)] + [it.copy()]


@pytest.mark.parametrize("index", [1, 3])
def test_concurrent_builds_equal_sequential(index):
    w = make_workload(index)
    args = (w.prefix_lens, w.suffix_counts, w.suffix_lens, w.num_q_heads, w.num_kv_heads,
            w.head_dim, w.rope_theta)
    L = pg.pg_build_layout_host(*args)
    want = snapshot(L)
    L.close()
    got, errors = [None] * 6, []

    def worker(i):
        try:
            for _ in range(3):
                Li = pg.pg_build_layout_host(*args)
                got[i] = snapshot(Li)
                Li.close()
        except Exception as e:   # reported below, not lost in the thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(6)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for g in got:
        assert len(g) == len(want)
        for a, b in zip(g, want):
            assert np.array_equal(a, b)
