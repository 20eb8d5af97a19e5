"""Unpacked comparison layout: every prompt+response sequence on its own.

This is what preference packing removes ("Preference Packing", core idea: the
shared prompt is otherwise attended once per response). The benchmark runs
the same attention kernel on this layout, one launch, with the prefix Q/K/V
duplicated for each response, and reports t(unpacked) / t(packed).
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass
class Unpacked:
    prefix_lens: np.ndarray    # int32 [num sequences]: whole sequence as one causal prefix
    suffix_counts: np.ndarray  # int32 zeros
    suffix_lens: np.ndarray    # int32 empty
    gather: np.ndarray         # int64 [T_unpacked]: packed token of each unpacked token


def unpacked_workload(prefix_lens, suffix_counts, suffix_lens) -> Unpacked:
    P = np.asarray(prefix_lens, dtype=np.int64)
    n = np.asarray(suffix_counts, dtype=np.int64)
    S = np.asarray(suffix_lens, dtype=np.int64)
    seq_lens = []
    parts = []
    start = 0
    k = 0
    for g in range(P.shape[0]):
        pre = np.arange(start, start + P[g])
        cur = start + P[g]
        if n[g] == 0:
            seq_lens.append(int(P[g]))
            parts.append(pre)
        for _ in range(int(n[g])):
            s = int(S[k])
            k += 1
            seq_lens.append(int(P[g]) + s)
            parts.append(np.concatenate([pre, np.arange(cur, cur + s)]))
            cur += s
        start = cur
    gather = np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)
    m = len(seq_lens)
    return Unpacked(np.asarray(seq_lens, dtype=np.int32), np.zeros(m, dtype=np.int32),
                    np.zeros(0, dtype=np.int32), gather.astype(np.int64))


def unpacked_decode_workload(prefix_lens, suffix_counts, suffix_lens) -> Unpacked:
    """Decode comparison layout: every response with its own copy of its
    group's prompt (one group per response, the response slot at capacity), so
    a decode step reads each prompt once per response instead of once per
    group. Groups without responses decode nothing and are left out."""
    P = np.asarray(prefix_lens, dtype=np.int64)
    n = np.asarray(suffix_counts, dtype=np.int64)
    S = np.asarray(suffix_lens, dtype=np.int64)
    pre_lens, caps, parts = [], [], []
    start = 0
    k = 0
    for g in range(P.shape[0]):
        pre = np.arange(start, start + P[g])
        cur = start + P[g]
        for _ in range(int(n[g])):
            s = int(S[k])
            k += 1
            pre_lens.append(int(P[g]))
            caps.append(s)
            parts.append(np.concatenate([pre, np.arange(cur, cur + s)]))
            cur += s
        start = cur
    gather = np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)
    m = len(pre_lens)
    return Unpacked(np.asarray(pre_lens, dtype=np.int32), np.ones(m, dtype=np.int32),
                    np.asarray(caps, dtype=np.int32), gather.astype(np.int64))
