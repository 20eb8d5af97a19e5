"""Runs the fp64 oracle over a whole full-size workload in parallel units.

Groups never attend across each other, and query heads are independent, so
the oracle's ``attention`` (the definition: causal attention of every
unpacked prompt || response sequence) can be evaluated one (group, query
head) at a time on that group alone, with its own one-group layout. The
units run on a thread pool (numpy releases the GIL inside its loops and
matrix products), each with one BLAS thread, and the caller consumes each
unit's result as it arrives, so a whole workload is compared without ever
holding its fp64 output at once.

Test infrastructure: only the tests import this module. It computes nothing
itself; every number comes from ``oracle.pg_oracle``.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Callable, Iterator, Tuple

import numpy as np

from oracle import pg_oracle as O

try:
    from threadpoolctl import threadpool_limits
except ImportError:   # pragma: no cover - threadpoolctl is part of the image
    threadpool_limits = None


def workers() -> int:
    """Pool size: the CPUs this process may use, at most 16 (one GPU's share
    of a host's cores)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:   # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def group_layouts(w, lay):
    """(group, first token, end token, one-group oracle layout) per non-empty group."""
    out = []
    soff = 0
    for g in range(len(w.prefix_lens)):
        n = int(w.suffix_counts[g])
        sub = O.layout(w.prefix_lens[g:g + 1], w.suffix_counts[g:g + 1], w.suffix_lens[soff:soff + n])
        soff += n
        a, b = int(lay["group_off"][g]), int(lay["group_off"][g + 1])
        if b > a:
            out.append((g, a, b, sub))
    return out


def attention_units(w, lay, q, k, v, heads=None, groups=None,
                    ) -> Iterator[Tuple[int, int, int, int, np.ndarray, np.ndarray]]:
    """Yields (group, head, a, b, o [b - a, d], lse [b - a]) of the oracle's
    ``attention`` for every (group, query head) unit, in completion order.

    q: [T, Hq, d], k, v: [T, Hkv, d], float arrays (or any object whose
    [a:b, h] slices are float arrays). heads / groups restrict the units.
    """
    r = w.num_q_heads // w.num_kv_heads
    units = [(g, a, b, sub, h) for (g, a, b, sub) in group_layouts(w, lay)
             if groups is None or g in groups
             for h in (range(w.num_q_heads) if heads is None else heads)]

    def run(unit):
        g, a, b, sub, h = unit
        hk = h // r
        qq = np.asarray(q[a:b, h:h + 1], dtype=np.float64)
        kk = np.asarray(k[a:b, hk:hk + 1], dtype=np.float64)
        vv = np.asarray(v[a:b, hk:hk + 1], dtype=np.float64)
        if threadpool_limits is not None:
            with threadpool_limits(1):
                o, lse = O.attention(qq, kk, vv, sub, w.softmax_scale, 1, 1)
        else:
            o, lse = O.attention(qq, kk, vv, sub, w.softmax_scale, 1, 1)
        return g, h, a, b, o[:, 0], lse[0]

    # largest units first, so the pool's tail is short
    units.sort(key=lambda u: -(u[2] - u[1]))
    with ThreadPoolExecutor(max_workers=workers()) as ex:
        for res in ex.map(run, units):
            yield res


def max_errors(w, lay, q, k, v, o_gpu, lse_gpu, heads=None, groups=None,
               on_unit: Callable = None) -> Tuple[float, float, int]:
    """Largest |O_gpu - O_ref| and |lse_gpu - lse_ref| over every row of the
    selected units, and the number of rows compared. o_gpu: [T, Hq, d] and
    lse_gpu: [Hq, T] host arrays."""
    eo = 0.0
    el = 0.0
    rows = 0
    for g, h, a, b, o, lse in attention_units(w, lay, q, k, v, heads=heads, groups=groups):
        eo = max(eo, float(np.abs(o_gpu[a:b, h].astype(np.float64) - o).max()))
        el = max(el, float(np.abs(lse_gpu[h, a:b].astype(np.float64) - lse).max()))
        rows += b - a
        if on_unit is not None:
            on_unit(g, h, a, b, o, lse)
    return eo, el, rows


def _limited(fn, *args, **kw):
    if threadpool_limits is None:   # pragma: no cover
        return fn(*args, **kw)
    with threadpool_limits(1):
        return fn(*args, **kw)


def kv_head_slices(x_q, x_kv, hk, r, a, b):
    """Rows [a, b) of the r query heads of KV head hk and of that KV head, as
    float64 arrays shaped for a one-KV-head problem ([n, r, d] and [n, 1, d])."""
    q = np.asarray(x_q[a:b, hk * r:(hk + 1) * r], dtype=np.float64)
    kv = np.asarray(x_kv[a:b, hk:hk + 1], dtype=np.float64)
    return q, kv


def attention_heads(sub, q, k, v, scale):
    """The oracle's ``attention`` on a one-group, one-KV-head problem (q [n, r,
    d], k, v [n, 1, d], ``sub`` its layout), one query head per pool unit.
    Returns o [n, r, d] and lse [r, n] in fp64."""
    n, r, d = q.shape
    o = np.zeros((n, r, d))
    lse = np.zeros((r, n))

    def run(h):
        return h, _limited(O.attention, q[:, h:h + 1], k, v, sub, scale, 1, 1)

    with ThreadPoolExecutor(max_workers=workers()) as ex:
        for h, (oh, lh) in ex.map(run, range(r)):
            o[:, h] = oh[:, 0]
            lse[h] = lh[0]
    return o, lse


def backward_units(w, lay, q, k, v, do, groups):
    """Yields (group, KV head, a, b, dq [n, r, d], dk [n, d], dv [n, d], mags)
    of the oracle's dense ``attention_backward`` (with term magnitudes) for
    every (group, KV head) of ``groups``, each unit on its group alone with
    its KV head's r query heads, in parallel."""
    r = w.num_q_heads // w.num_kv_heads
    subs = {g: (a, b, sub) for (g, a, b, sub) in group_layouts(w, lay) if g in groups}
    units = [(g, hk) for g in subs for hk in range(w.num_kv_heads)]

    def run(unit):
        g, hk = unit
        a, b, sub = subs[g]
        qq, kk = kv_head_slices(q, k, hk, r, a, b)
        dd, vv = kv_head_slices(do, v, hk, r, a, b)
        dq, dk, dv, mags = _limited(O.attention_backward, qq, kk, vv, dd, sub, w.softmax_scale,
                                    r, 1, magnitudes=True)
        return g, hk, a, b, dq, dk[:, 0], dv[:, 0], {"dq": mags["dq"], "dk": mags["dk"][:, 0],
                                                     "dv": mags["dv"][:, 0]}

    # dense per group: memory grows with the square of the group, so at most 8 at once
    with ThreadPoolExecutor(max_workers=min(8, workers())) as ex:
        for res in ex.map(run, units):
            yield res
