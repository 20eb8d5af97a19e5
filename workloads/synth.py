"""Workload recipes and seeded tensor draws.

Five workloads stand in for the datasets and serving traces the pages measure
on (preference-optimisation data in "Preference Packing", abstract; batched
inference traces in "PackInfer", abstract). None of those data are used; every
length and every tensor here is synthetic.

Random streams (numpy PCG64):
  * ``default_rng([cfg, 0])``       lengths of workload ``cfg``
  * ``default_rng([cfg, 1|2|3])``   Q | K | V, drawn as float32 N(0, 1) in
    ``[T, H, d]`` C order, in token chunks (identical to one monolithic draw)
A non-default ``seed`` appends itself to each key: ``[cfg, stream, seed]``.

bf16 inputs are the float32 draws rounded to nearest-even bf16; the bits are
returned as uint16 so both sides read exactly the same values.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, Optional, Sequence

import numpy as np

WORKLOAD_NAMES = (
    "tiny-fp32",
    "dpo-bf16",
    "grpo-bf16",
    "heterogeneous-bf16",
    "long-prefix-bf16",
)


@dataclasses.dataclass
class Workload:
    index: int                 # -1 for custom shapes
    name: str
    prefix_lens: np.ndarray    # int32 [G]
    suffix_counts: np.ndarray  # int32 [G]
    suffix_lens: np.ndarray    # int32 [sum(suffix_counts)], group-major order
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                 # "f32" or "bf16"
    rope_theta: float
    softmax_scale: float
    seed: Optional[int] = None

    @property
    def num_groups(self) -> int:
        return int(self.prefix_lens.shape[0])

    @property
    def total_tokens(self) -> int:
        return int(self.prefix_lens.sum() + self.suffix_lens.sum())

    def groups(self):
        """Yield (prefix_len, [suffix lens]) per group, in input order."""
        off = 0
        for g in range(self.num_groups):
            n = int(self.suffix_counts[g])
            yield int(self.prefix_lens[g]), [int(s) for s in self.suffix_lens[off:off + n]]
            off += n

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "groups": self.num_groups,
            "tokens": self.total_tokens,
            "num_q_heads": self.num_q_heads,
            "num_kv_heads": self.num_kv_heads,
            "head_dim": self.head_dim,
            "dtype": self.dtype,
            "rope_theta": self.rope_theta,
            "seed": self.seed,
        }


def _rng(cfg: int, stream: int, seed: Optional[int]) -> np.random.Generator:
    key = [cfg, stream] if seed is None else [cfg, stream, seed]
    return np.random.default_rng(key)


def _lognormal_int(rng, median, sigma, n, lo, hi):
    x = rng.lognormal(mean=math.log(median), sigma=sigma, size=n)
    return np.clip(np.rint(x), lo, hi).astype(np.int32)


def _arr(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def make_workload(index: int, seed: Optional[int] = None) -> Workload:
    """Lengths and shapes of workload ``index`` (0..4).

    Integer draws are inclusive ranges; lognormal lengths are rounded to the
    nearest integer, then clamped.
    """
    rng = _rng(index, 0, seed)
    inv = 1.0 / math.sqrt(128.0)
    if index == 0:
        # Fixed tiny case: two groups, fp32, one head, d = 64.
        return Workload(0, WORKLOAD_NAMES[0], _arr([5, 9]), _arr([2, 3]),
                        _arr([3, 4, 2, 6, 1]), 1, 1, 64, "f32", 1.0e4,
                        1.0 / 8.0, seed)
    if index == 1:
        # DPO-style: 8 prompts, each with a chosen and a rejected response.
        p = rng.integers(256, 1024, size=8, endpoint=True)
        s = rng.integers(64, 512, size=16, endpoint=True)
        return Workload(1, WORKLOAD_NAMES[1], _arr(p), _arr([2] * 8), _arr(s),
                        32, 8, 128, "bf16", 5.0e5, inv, seed)
    if index == 2:
        # GRPO-style: 16 prompts x 8 sampled responses.
        p = rng.integers(512, 2048, size=16, endpoint=True)
        s = _lognormal_int(rng, 400.0, 0.6, 128, 32, 2048)
        return Workload(2, WORKLOAD_NAMES[2], _arr(p), _arr([8] * 16), _arr(s),
                        32, 8, 128, "bf16", 5.0e5, inv, seed)
    if index == 3:
        # Heterogeneous serving batch: 64 requests; the first 19 (30 %) sit in
        # share-groups of 2-4 on a per-group 1024-token prefix and keep their
        # own drawn length as the suffix; the rest are unshared (prefix only).
        n_req = 64
        lens = _lognormal_int(rng, 600.0, 1.0, n_req, 32, 8192)
        n_shared = int(round(0.3 * n_req))
        sizes = []
        left = n_shared
        while left > 0:
            ok = [s for s in (2, 3, 4) if s <= left and left - s != 1]
            s = int(rng.choice(ok))
            sizes.append(s)
            left -= s
        p, c, s = [], [], []
        cur = 0
        for gs in sizes:
            p.append(1024)
            c.append(gs)
            s.extend(int(x) for x in lens[cur:cur + gs])
            cur += gs
        for i in range(n_shared, n_req):
            p.append(int(lens[i]))
            c.append(0)
        return Workload(3, WORKLOAD_NAMES[3], _arr(p), _arr(c), _arr(s),
                        32, 8, 128, "bf16", 5.0e5, inv, seed)
    if index == 4:
        # Long shared prefix (image+text prompt shape), 64/8 heads.
        s = rng.integers(256, 2048, size=16, endpoint=True)
        return Workload(4, WORKLOAD_NAMES[4], _arr([16384] * 4), _arr([4] * 4),
                        _arr(s), 64, 8, 128, "bf16", 5.0e5, inv, seed)
    raise ValueError(f"no workload {index}")


def make_custom(prefix_lens: Sequence[int], suffix_lens: Sequence[Sequence[int]],
                num_q_heads: int = 4, num_kv_heads: int = 1, head_dim: int = 128,
                dtype: str = "bf16", rope_theta: float = 5.0e5,
                softmax_scale: Optional[float] = None, seed: int = 0,
                name: str = "custom") -> Workload:
    """A workload with explicit lengths (edge cases: P = 0, n = 0, S = 0)."""
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"dtype must be 'f32' or 'bf16', not {dtype!r}")
    if len(prefix_lens) != len(suffix_lens):
        raise ValueError("one suffix list per group")
    flat = [int(x) for grp in suffix_lens for x in grp]
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(head_dim)
    return Workload(-1, name, _arr(prefix_lens), _arr([len(s) for s in suffix_lens]),
                    _arr(flat), num_q_heads, num_kv_heads, head_dim, dtype,
                    float(rope_theta), float(softmax_scale), seed)


# ----------------------------------------------------------------- tensors --

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16 (ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


_STREAM = {"q": 1, "k": 2, "v": 3, "do": 4}   # "do": upstream gradient of O (backward)
_DECODE_STREAM = 5                                # decode step: current lengths, then queries


def draw_tensor(w: Workload, which: str, chunk_tokens: int = 4096) -> np.ndarray:
    """Draw Q, K, V or the upstream gradient dO ("do", shaped like Q) of
    workload ``w`` as ``[T, H, d]``.

    Returns float32 for fp32 workloads and uint16 bf16 bits for bf16 ones.
    """
    heads = w.num_q_heads if which in ("q", "do") else w.num_kv_heads
    if w.index >= 0:
        rng = _rng(w.index, _STREAM[which], w.seed)
    else:
        rng = np.random.default_rng([1000, _STREAM[which], int(w.seed or 0)])
    T, d = w.total_tokens, w.head_dim
    row = heads * d
    if w.dtype == "f32":
        out = np.empty((T, heads, d), dtype=np.float32)
    else:
        out = np.empty((T, heads, d), dtype=np.uint16)
    flat = out.reshape(T, row)
    for t0 in range(0, T, chunk_tokens):
        t1 = min(T, t0 + chunk_tokens)
        x = rng.standard_normal((t1 - t0) * row, dtype=np.float32).reshape(t1 - t0, row)
        flat[t0:t1] = x if w.dtype == "f32" else f32_to_bf16_bits(x)
    return out


def draw_decode(w: Workload) -> Dict[str, np.ndarray]:
    """Inputs of one decode step over workload ``w``'s layout taken as a KV
    cache whose response segments are at capacity (the drawn suffix lengths).

    cur_lens: int32 [N], uniform on [min(1, cap), cap] per response (the step
    falls anywhere in generation); q: [N, Hq, d], one query per response, drawn
    like Q (float32 N(0,1); uint16 bf16 bits for bf16 workloads).
    """
    if w.index >= 0:
        rng = _rng(w.index, _DECODE_STREAM, w.seed)
    else:
        rng = np.random.default_rng([1000, _DECODE_STREAM, int(w.seed or 0)])
    caps = np.asarray(w.suffix_lens, dtype=np.int64)
    lo = np.minimum(caps, 1)
    cur = (lo + np.floor(rng.random(len(caps)) * (caps - lo + 1))).astype(np.int32)
    n, hq, d = len(caps), w.num_q_heads, w.head_dim
    x = rng.standard_normal(n * hq * d, dtype=np.float32).reshape(n, hq, d)
    q = x if w.dtype == "f32" else f32_to_bf16_bits(x)
    return {"cur_lens": cur, "q": q}


def draw_qkv(w: Workload) -> Dict[str, np.ndarray]:
    return {name: draw_tensor(w, name) for name in ("q", "k", "v")}


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
