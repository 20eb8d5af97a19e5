"""fp64 CPU oracle for packed shared-prefix causal attention.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The HIP library never calls it and
shares no code with it; the two meet only through the seeded inputs of the
``workloads`` package.

What is computed, and where the pages fix it
--------------------------------------------
"Preference Packing: Efficient Preference Optimization for LLMs" (core idea,
technical framework): samples that share a prompt are packed as the prompt once
followed by each response; prompt attention is computed once and reused for
every response, and the model itself is unchanged (key innovation).
The verl ``prefix_grouper_utils.py`` page (section 1, building position ids,
and the prefix-sharing diagram) fixes that every response continues the
prefix independently and that its position ids restart at the prefix length.

Hence the packed result has a plain definition: every packed row equals the
row of textbook causal attention over the unpacked sequence prefix || response
it belongs to. ``attention`` is that definition written out. ``attention_masked``
is the packed form with an explicit key set per token, ``attention_dense`` the
same with a dense T x T mask; tests tie all three together.

Readings where the pages are silent:
  * RoPE is never defined on the pages: rotate-half convention on Q and K,
    omega_i = theta^(-2i/d), i < d/2.
  * softmax scale is an input (1/sqrt(d) in the workloads).
  * GQA: query head h reads KV head h // (Hq / Hkv).
  * lse is the natural log of the sum of exp of the *scaled* scores.
  * zero-length suffixes occupy no tokens; P = 0 and n = 0 are legal.

The backward (``attention_backward``) is the chain rule of that definition
written out for an upstream gradient of O; tests/test_oracle_backward.py pins it.
``decode_attention`` is one generation step over a group-contiguous cache;
tests/test_oracle_decode.py pins it.

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (hand-derived values, closed forms, a library routine, brute
force); the pins are listed beside each function.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Sequence, Tuple

import numpy as np

# ------------------------------------------------------------------ layout --


def layout(prefix_lens: Sequence[int], suffix_counts: Sequence[int],
           suffix_lens: Sequence[int]) -> Dict[str, np.ndarray]:
    """Token layout of the packed batch.

    "Preference Packing" (technical framework, step 2): each group is stored as
    its prompt once, then each of its responses. Groups and responses keep
    input order (reading). Segments are listed per group as
    [prefix, suffix_1, ..., suffix_n]; zero-length ones are kept in the list
    and occupy no tokens (verl page, section 1: empty suffixes are skipped).

    Per token t: g0 = first token of its group, pe = end of its group's prefix,
    ss = start of its own segment (the group start for prefix tokens).

    Pinned by: hand-derived offsets of the tiny workload (tests/golden).
    """
    P = [int(x) for x in prefix_lens]
    n = [int(x) for x in suffix_counts]
    S = [int(x) for x in suffix_lens]
    if len(P) != len(n) or sum(n) != len(S):
        raise ValueError("inconsistent lengths")
    if min(P + n + S + [0]) < 0:
        raise ValueError("negative length")
    group_off = [0]
    seg_off = [0]
    g0: List[int] = []
    pe: List[int] = []
    ss: List[int] = []
    k = 0
    for g in range(len(P)):
        start = group_off[-1]
        pend = start + P[g]
        seg_off.append(pend)
        for t in range(start, pend):
            g0.append(start)
            pe.append(pend)
            ss.append(start)
        cur = pend
        for _ in range(n[g]):
            s_len = S[k]
            k += 1
            for t in range(cur, cur + s_len):
                g0.append(start)
                pe.append(pend)
                ss.append(cur)
            cur += s_len
            seg_off.append(cur)
        group_off.append(cur)
    return {
        "prefix_lens": np.asarray(P, dtype=np.int64),
        "suffix_counts": np.asarray(n, dtype=np.int64),
        "suffix_lens": np.asarray(S, dtype=np.int64),
        "group_off": np.asarray(group_off, dtype=np.int64),
        "seg_off": np.asarray(seg_off, dtype=np.int64),
        "g0": np.asarray(g0, dtype=np.int64),
        "pe": np.asarray(pe, dtype=np.int64),
        "ss": np.asarray(ss, dtype=np.int64),
        "total_tokens": group_off[-1],
    }


def sequences(lay) -> Iterable[Tuple[int, int, int, int]]:
    """The unpacked sequences: (group, prefix start, prefix len, suffix span).

    Yields (g, p0, P, (s0, s1)) per suffix; a group with no suffix yields once
    with an empty suffix span, so its prefix still forms a sequence.
    """
    k = 0
    for g in range(len(lay["prefix_lens"])):
        p0 = int(lay["group_off"][g])
        P = int(lay["prefix_lens"][g])
        cur = p0 + P
        n = int(lay["suffix_counts"][g])
        if n == 0:
            yield g, p0, P, (cur, cur)
        for _ in range(n):
            s = int(lay["suffix_lens"][k])
            k += 1
            yield g, p0, P, (cur, cur + s)
            cur += s


# --------------------------------------------------------------- positions --


def positions(lay) -> np.ndarray:
    """int64 position id per packed token.

    verl page, section 1 (building position ids) and the prefix-sharing
    diagram: every response continues the prompt independently, as if
    prompt || response were its own sequence, so a token's position is its
    index in that unpacked sequence. In terms of the layout's per-token
    descriptors (g0 = group start, pe = prompt end, ss = own segment start):
    a prompt token t has position t - g0; a response token has the prompt
    length pe - g0 plus its index t - ss in its own response.

    Pinned by: hand-derived ids of the tiny workload; equality with
    arange(P+S) of each unpacked sequence.
    """
    T = int(lay["total_tokens"])
    t = np.arange(T, dtype=np.int64)
    g0 = np.asarray(lay["g0"], dtype=np.int64)
    pe = np.asarray(lay["pe"], dtype=np.int64)
    ss = np.asarray(lay["ss"], dtype=np.int64)
    return np.where(t < pe, t - g0, (pe - g0) + (t - ss)).astype(np.int64)


# -------------------------------------------------------------------- rope --


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding (rotate-half convention) in fp64.

    The pages never define RoPE; they only fix the positions it is applied at
    (verl page, section 1). Reading: for i < d/2, omega_i = theta^(-2i/d),
    phi = pos * omega_i, and the pair (x_i, x_{i+d/2}) is rotated by phi.

    x: [T, H, d] (any float dtype); pos: int [T]. Returns fp64 [T, H, d].
    Pinned by: complex-multiplication form, pos = 0 identity, pair norms,
    dependence of <R(a)q, R(b)k> on b - a only.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    omega = float(theta) ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    phi = np.asarray(pos, dtype=np.float64)[:, None] * omega[None, :]   # [T, d/2]
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    lo = x[..., :half]
    hi = x[..., half:]
    out = np.empty_like(x)
    out[..., :half] = lo * c - hi * s
    out[..., half:] = hi * c + lo * s
    return out


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even) of fp64 input, returned as fp64.

    bf16 keeps 8 significant bits; x = m * 2^e with 0.5 <= |m| < 1, so the
    rounded value is rint(m * 2^8) * 2^(e - 8) (rint rounds ties to even).
    Valid for normal numbers, which is all the workloads produce.
    Pinned by: tie cases 1 + 2^-8 -> 1 and 1 + 3*2^-8 -> 1 + 2^-6.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def storage_round(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to the storage dtype of a workload (fp64 out)."""
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------- attention --


def _kv_head(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """GQA reading: consecutive query heads share a KV head."""
    return h // (num_q_heads // num_kv_heads)


def _causal_rows(q_rows: np.ndarray, k_seq: np.ndarray, v_seq: np.ndarray,
                 row_index: np.ndarray, scale: float):
    """Textbook causal softmax attention for selected rows of one sequence.

    Row i of the sequence attends keys 0..i. q_rows: [R, d] (rows with
    sequence indices ``row_index``), k_seq/v_seq: [L, d]. Returns (o [R, d],
    lse [R]) with lse = max + ln(sum exp(s - max)) of the scaled scores.
    """
    s = scale * (q_rows @ k_seq.T)                               # [R, L]
    cols = np.arange(k_seq.shape[0])[None, :]
    s = np.where(cols <= row_index[:, None], s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ v_seq) / l
    return o, (m + np.log(l))[:, 0]


def attention(q, k, v, lay, scale: float, num_q_heads: int, num_kv_heads: int,
              row_chunk: int = 1024):
    """Packed attention output by its definition: causal attention of each
    unpacked sequence.

    "Preference Packing" (core idea) and the verl prefix-sharing diagram: the
    prompt's attention is computed once and each response continues it, as if
    prompt || response were its own sequence. So prefix rows are the causal
    attention of the prefix alone (they cannot see any suffix), and the rows of
    suffix k are the suffix rows of causal attention over prefix || suffix_k.

    q: [T, Hq, d], k/v: [T, Hkv, d] (any float dtype; computed in fp64).
    Returns o fp64 [T, Hq, d] and lse fp64 [Hq, T].
    Pinned by: equality with ``attention_masked`` and ``attention_dense`` and
    with torch's float64 SDPA (library routine); special cases (first token,
    constant V, identical keys, n = 1, P = 0, GQA vs repeated MHA).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, Hq, d = q.shape
    o = np.zeros((T, Hq, d), dtype=np.float64)
    lse = np.zeros((Hq, T), dtype=np.float64)
    done_prefix = set()
    for g, p0, P, (s0, s1) in sequences(lay):
        tok = np.concatenate([np.arange(p0, p0 + P), np.arange(s0, s1)])
        todo = [] if g in done_prefix else list(range(P))
        todo += list(range(P, len(tok)))
        done_prefix.add(g)
        if not todo:
            continue
        rows = np.asarray(todo)
        for h in range(Hq):
            hk = _kv_head(h, Hq, num_kv_heads)
            ks = k[tok, hk]
            vs = v[tok, hk]
            for c0 in range(0, len(rows), row_chunk):
                r = rows[c0:c0 + row_chunk]
                oo, ll = _causal_rows(q[tok[r], h], ks, vs, r, scale)
                o[tok[r], h] = oo
                lse[h, tok[r]] = ll
    return o, lse


def allowed_keys(lay, t: int) -> np.ndarray:
    """Key set K(t) of packed token t (reading of the mask, never written as a
    formula on the pages): keys of its own group up to itself, except keys of a
    sibling response. A prefix token sees its prefix causally; a response token
    sees the whole prefix and its own response causally.

    K(t) = { j : g0 <= j <= t and (j < pe or j >= ss) }.
    Pinned by: equality of ``attention_masked`` with ``attention``.
    """
    g0, pe, ss = int(lay["g0"][t]), int(lay["pe"][t]), int(lay["ss"][t])
    j = np.arange(g0, t + 1)
    return j[(j < pe) | (j >= ss)]


def attention_masked(q, k, v, lay, scale: float, num_q_heads: int,
                     num_kv_heads: int):
    """Packed attention over the packed row with the key set K(t) per token.

    This is the form a packed kernel evaluates (one pass over the packed row,
    PackInfer abstract: attention built directly over packed query-key
    regions). Returns (o [T, Hq, d], lse [Hq, T]) in fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, Hq, d = q.shape
    o = np.zeros((T, Hq, d))
    lse = np.zeros((Hq, T))
    for t in range(T):
        keys = allowed_keys(lay, t)
        for h in range(Hq):
            hk = _kv_head(h, Hq, num_kv_heads)
            s = scale * (k[keys, hk] @ q[t, h])
            m = s.max()
            p = np.exp(s - m)
            o[t, h] = (p @ v[keys, hk]) / p.sum()
            lse[h, t] = m + math.log(p.sum())
    return o, lse


def segment_ids(lay) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Per token: group id, segment id (0 = prefix, k = suffix k), and a flag
    for prefix tokens. Used only by the dense brute-force form."""
    T = int(lay["total_tokens"])
    grp = np.zeros(T, dtype=np.int64)
    seg = np.zeros(T, dtype=np.int64)
    k = 0
    for g in range(len(lay["prefix_lens"])):
        a, b = int(lay["group_off"][g]), int(lay["group_off"][g + 1])
        grp[a:b] = g
        cur = a + int(lay["prefix_lens"][g])
        for j in range(int(lay["suffix_counts"][g])):
            s = int(lay["suffix_lens"][k])
            k += 1
            seg[cur:cur + s] = j + 1
            cur += s
    return grp, seg, seg == 0


def dense_mask(lay) -> np.ndarray:
    """Dense T x T boolean mask from segment ids:
    M[i, j] = same group and j <= i and (j is a prefix token or same segment).
    """
    grp, seg, is_pre = segment_ids(lay)
    T = grp.shape[0]
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    return (grp[:, None] == grp[None, :]) & (j <= i) & (is_pre[None, :] | (seg[:, None] == seg[None, :]))


def attention_dense(q, k, v, lay, scale: float, num_q_heads: int,
                    num_kv_heads: int):
    """Brute force: one softmax per head over all T keys with the dense mask.
    For tiny inputs only (T <= a few hundred)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, Hq, d = q.shape
    M = dense_mask(lay)
    o = np.zeros((T, Hq, d))
    lse = np.zeros((Hq, T))
    for h in range(Hq):
        hk = _kv_head(h, Hq, num_kv_heads)
        s = np.where(M, scale * (q[:, h] @ k[:, hk].T), -np.inf)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        o[:, h] = (p @ v[:, hk]) / l
        lse[h] = (m + np.log(l))[:, 0]
    return o, lse


def attention_rows(q, k, v, lay, scale: float, num_q_heads: int,
                   num_kv_heads: int, tokens: Sequence[int], heads: Sequence[int]):
    """Selected outputs by the definition, one (token, head) at a time.

    For a prefix token at prefix index i: causal attention over prefix[0..i].
    For a token at index i of suffix k: attention over the whole prefix and
    suffix_k[0..i] (its unpacked sequence, causal). Returns o [n, d], lse [n]
    for the pairs zip(tokens, heads). Cheap enough for full-size workloads.
    """
    T, Hq, d = q.shape
    bounds = {}
    for g, p0, P, (s0, s1) in sequences(lay):
        for t in range(s0, s1):
            bounds[t] = (p0, P, s0)
    out_o = np.zeros((len(tokens), d))
    out_l = np.zeros(len(tokens))
    # rows of one token and KV head share their key rows: gather them once
    todo: Dict[Tuple[int, int], List[Tuple[int, int]]] = {}
    for n, (t, h) in enumerate(zip(tokens, heads)):
        t, h = int(t), int(h)
        todo.setdefault((t, _kv_head(h, Hq, num_kv_heads)), []).append((n, h))
    for (t, hk), rows in todo.items():
        if t in bounds:
            p0, P, s0 = bounds[t]
            keys = np.concatenate([np.arange(p0, p0 + P), np.arange(s0, t + 1)])
        else:  # prefix token
            g0 = int(lay["g0"][t])
            keys = np.arange(g0, t + 1)
        kk = np.asarray(k[keys, hk], dtype=np.float64)
        vv = np.asarray(v[keys, hk], dtype=np.float64)
        for n, h in rows:
            qq = np.asarray(q[t, h], dtype=np.float64)
            s = scale * (kk @ qq)
            m = s.max()
            p = np.exp(s - m)
            out_o[n] = (p @ vv) / p.sum()
            out_l[n] = m + math.log(p.sum())
    return out_o, out_l


# ------------------------------------------------------------------ backward --


def group_mask(lay, g: int) -> np.ndarray:
    """Allowed (query, key) pairs inside group g as an n_g x n_g boolean matrix
    (row = query, column = key, both indexed from the group's first token):
    key j is allowed for query i iff j <= i and (j is a prompt token or i and
    j lie in the same response). Same reading as ``allowed_keys``."""
    a, b = int(lay["group_off"][g]), int(lay["group_off"][g + 1])
    pe = int(lay["pe"][a]) if b > a else a
    ss = np.asarray(lay["ss"][a:b], dtype=np.int64)
    t = np.arange(a, b)
    i = t[:, None]
    j = t[None, :]
    return (j <= i) & ((j < pe) | (ss[:, None] == ss[None, :]))


def attention_backward(q, k, v, do, lay, scale: float, num_q_heads: int,
                       num_kv_heads: int, groups: Sequence[int] = None,
                       magnitudes: bool = False):
    """Gradients of the packed attention output, by the chain rule.

    The packed forward (``attention``) maps Q, K, V to O with one softmax per
    (token, head) over its key set. Its derivative, for an upstream gradient dO
    of O (the lse output is treated as carrying no gradient), is written out
    per group and query head in fp64:
      P  = softmax(scale * Q K^T) over the allowed keys (rows = queries),
      dV = P^T dO,           dP = dO V^T,
      D  = rowsum(P * dP) = rowsum(dO * O),
      dS = P * (dP - D),     dQ = scale * dS K,   dK = scale * dS^T Q.
    Under GQA a KV head's dK and dV sum the contributions of all its query
    heads. A prompt key therefore collects gradient from every response of its
    group, since the prompt is stored once (Preference Packing, core idea).

    q, do: [T, Hq, d]; k, v: [T, Hkv, d]. Returns (dq [T, Hq, d], dk, dv
    [T, Hkv, d]) in fp64, computed for ``groups`` (default: all) and zero
    elsewhere. Dense per group: for groups of up to a few thousand tokens.
    Pinned by: central finite differences of sum(dO * O) with ``attention``;
    torch's float64 SDPA autograd on the unpacked sequences (library routine);
    closed forms (constant V gives dQ = dK = 0; the keys' dV sum to the
    queries' dO sum; a group's first token has dQ = 0).

    With ``magnitudes`` it also returns, per output element, the root sum of
    squares of the terms of its defining sum (what a probabilistic rounding
    error bound scales with; not part of the gradient): for dV_j the terms
    p_ij dO_i, for dK_j the terms scale (|dS_ij| + p_ij delta_i) q_i and for
    dQ_i the terms scale (|dS_ij| + p_ij delta_i) k_j, where delta_i =
    ||dO_i * O_i||_2 is the size of the products D_i sums. Returned as a
    fourth item {"dq", "dk", "dv"} of arrays shaped like the gradients.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    T, Hq, d = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    if magnitudes:
        mq = np.zeros_like(dq)
        mk = np.zeros_like(dk)
        mv = np.zeros_like(dv)
    if groups is None:
        groups = range(len(lay["prefix_lens"]))
    for g in groups:
        a, b = int(lay["group_off"][g]), int(lay["group_off"][g + 1])
        if b == a:
            continue
        M = group_mask(lay, g)
        for h in range(Hq):
            hk = _kv_head(h, Hq, num_kv_heads)
            Q, K, V, dO = q[a:b, h], k[a:b, hk], v[a:b, hk], do[a:b, h]
            s = np.where(M, scale * (Q @ K.T), -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            P = e / e.sum(axis=1, keepdims=True)
            O = P @ V
            dP = dO @ V.T
            D = (dO * O).sum(axis=1, keepdims=True)
            dS = P * (dP - D)
            dq[a:b, h] = scale * (dS @ K)
            dk[a:b, hk] += scale * (dS.T @ Q)
            dv[a:b, hk] += P.T @ dO
            if magnitudes:
                delta = np.sqrt(((dO * O) ** 2).sum(axis=1, keepdims=True))
                A2 = (np.abs(dS) + P * delta) ** 2
                mq[a:b, h] = scale ** 2 * (A2 @ (K * K))
                mk[a:b, hk] += scale ** 2 * (A2.T @ (Q * Q))
                mv[a:b, hk] += (P * P).T @ (dO * dO)
    if magnitudes:
        return dq, dk, dv, {"dq": np.sqrt(mq), "dk": np.sqrt(mk), "dv": np.sqrt(mv)}
    return dq, dk, dv


def attention_backward_dq_rows(q, k, v, do, lay, scale: float, num_q_heads: int,
                               num_kv_heads: int, tokens: Sequence[int],
                               heads: Sequence[int], magnitudes: bool = False):
    """Selected rows of dQ by the same chain rule as ``attention_backward``,
    one (token, head) at a time over that row's key set (the keys of
    ``attention_rows``): with p the row's softmax over its keys,
      o = p V,  D = dO . o,  dp_j = dO . v_j,  dq = scale * sum_j p_j (dp_j - D) k_j.
    A query row's dQ needs only its own row of P, so this is cheap at full size.
    Returns [n, d] in fp64 for the pairs zip(tokens, heads). Pinned by:
    equality with ``attention_backward`` on every row of small workloads;
    closed forms (constant V gives dq = 0; a row with one key has dq = 0).
    With ``magnitudes`` it also returns the root sum of squares of the terms
    scale (|dS_j| + p_j delta) k_j per element, delta = ||dO * o||_2, as
    ``attention_backward`` defines them."""
    T, Hq, d = q.shape
    bounds = {}
    for g, p0, P, (s0, s1) in sequences(lay):
        for t in range(s0, s1):
            bounds[t] = (p0, P, s0)
    out = np.zeros((len(tokens), d))
    mag = np.zeros((len(tokens), d))
    for n, (t, h) in enumerate(zip(tokens, heads)):
        t, h = int(t), int(h)
        hk = _kv_head(h, Hq, num_kv_heads)
        if t in bounds:
            p0, P, s0 = bounds[t]
            keys = np.concatenate([np.arange(p0, p0 + P), np.arange(s0, t + 1)])
        else:  # prompt token
            keys = np.arange(int(lay["g0"][t]), t + 1)
        qq = np.asarray(q[t, h], dtype=np.float64)
        gg = np.asarray(do[t, h], dtype=np.float64)
        kk = np.asarray(k[keys, hk], dtype=np.float64)
        vv = np.asarray(v[keys, hk], dtype=np.float64)
        s = scale * (kk @ qq)
        e = np.exp(s - s.max())
        p = e / e.sum()
        o = p @ vv
        D = gg @ o
        dp = vv @ gg
        dS = p * (dp - D)
        out[n] = scale * (dS @ kk)
        if magnitudes:
            delta = math.sqrt(float(((gg * o) ** 2).sum()))
            mag[n] = scale * np.sqrt(((np.abs(dS) + p * delta) ** 2) @ (kk * kk))
    if magnitudes:
        return out, mag
    return out


def attention_backward_kv_rows(q, k, v, do, lay, scale: float, num_q_heads: int,
                               num_kv_heads: int, keys: Sequence[int],
                               kv_heads: Sequence[int], o=None, lse=None,
                               magnitudes: bool = False):
    """Selected rows of dK and dV by the same chain rule as
    ``attention_backward``, one (key token, KV head) at a time, summed over
    the query rows that read the key.

    Query token t reads key j iff j is in K(t) (``allowed_keys``): every later
    token of the group for a prompt key (the rest of the prompt and every
    response: "Preference Packing", core idea, the prompt is shared by all
    responses, so its gradient collects all of them), the rest of its own
    response for a response key. For each such t and each query head h of the
    KV head, with the row's own softmax p_tj = exp(scale q_t.k_j - lse_t) and
    D_t = dO_t . o_t:
      dV_j += p_tj dO_t,   dK_j += scale p_tj (dO_t . v_j - D_t) q_t.
    ``o`` [T, Hq, d] and ``lse`` [Hq, T] are the forward's output and
    logsumexp from ``attention`` (computed here over every row when not given;
    then only for small layouts); only the rows of the groups of the selected
    keys and the query heads of the selected KV heads are read.
    Returns (dk [n, d], dv [n, d]) for the pairs zip(keys, kv_heads), and with
    ``magnitudes`` also the root sum of squares of their terms as
    ``attention_backward`` defines them: (dk, dv, mag_dk, mag_dv).
    Pinned by: equality with ``attention_backward`` on every key row of small
    layouts; closed forms (constant V gives dk = 0; over a group's keys dV sums
    to the group's dO and dK to zero).
    """
    T, Hq, d = q.shape
    r = Hq // num_kv_heads
    if o is None or lse is None:
        o, lse = attention(q, k, v, lay, scale, num_q_heads, num_kv_heads)
    go = np.asarray(lay["group_off"], dtype=np.int64)
    ss_all = np.asarray(lay["ss"], dtype=np.int64)
    n = len(keys)
    dk = np.zeros((n, d))
    dv = np.zeros((n, d))
    mk = np.zeros((n, d))
    mv = np.zeros((n, d))
    for idx, (j, hk) in enumerate(zip(keys, kv_heads)):
        j, hk = int(j), int(hk)
        g0, pe = int(lay["g0"][j]), int(lay["pe"][j])
        g = int(np.searchsorted(go, g0, side="right")) - 1
        gend = int(go[g + 1])
        t = np.arange(j, gend)
        if j >= pe:   # response key: only the rest of its own response reads it
            t = t[ss_all[j:gend] == ss_all[j]]
        kj = np.asarray(k[j, hk], dtype=np.float64)
        vj = np.asarray(v[j, hk], dtype=np.float64)
        for h in range(hk * r, (hk + 1) * r):
            qt = np.asarray(q[t, h], dtype=np.float64)
            gt = np.asarray(do[t, h], dtype=np.float64)
            ot = np.asarray(o[t, h], dtype=np.float64)
            p = np.exp(scale * (qt @ kj) - np.asarray(lse[h, t], dtype=np.float64))
            D = (gt * ot).sum(axis=1)
            dS = p * (gt @ vj - D)
            dv[idx] += p @ gt
            dk[idx] += scale * (dS @ qt)
            if magnitudes:
                delta = np.sqrt(((gt * ot) ** 2).sum(axis=1))
                mv[idx] += (p * p) @ (gt * gt)
                mk[idx] += scale ** 2 * (((np.abs(dS) + p * delta) ** 2) @ (qt * qt))
    if magnitudes:
        return dk, dv, np.sqrt(mk), np.sqrt(mv)
    return dk, dv


def backward_flop(lay, head_dim: int, num_q_heads: int) -> int:
    """Algorithmic FLOP of the backward: five products over the allowed pairs
    (S = QK^T recomputed, dP = dO V^T, dV = P^T dO, dQ = dS K, dK = dS^T Q),
    2 d FLOP each per pair and query head: 10 d Hq per allowed pair."""
    return 10 * head_dim * num_q_heads * useful_pairs(lay)


# -------------------------------------------------------- pack and unpack --


def pack_rows(prefix: np.ndarray, suffix: np.ndarray, lay) -> np.ndarray:
    """Packed rows from right-padded per-group prompts and per-response rows.

    verl page, section 2 (building the grouped batch: the prompts selected once
    per group are concatenated with the responses, right padding): the packed
    row of group g is prompt_g followed by each of its responses, groups one
    after another. prefix: [G, Pmax, ...] (first prefix_lens[g] rows valid),
    suffix: [N, Smax, ...] (first suffix_lens[k] rows valid, responses in group
    order). Returns [T, ...], written out by concatenation.
    Pinned by: a hand-written example; unpack_rows(pack_rows(x)) gives the
    valid rows back.
    """
    parts = []
    k = 0
    for g in range(len(lay["prefix_lens"])):
        parts.append(prefix[g, :int(lay["prefix_lens"][g])])
        for _ in range(int(lay["suffix_counts"][g])):
            parts.append(suffix[k, :int(lay["suffix_lens"][k])])
            k += 1
    if not parts:
        return np.zeros((0,) + prefix.shape[2:], dtype=prefix.dtype)
    return np.concatenate(parts, axis=0)


def unpack_rows(packed: np.ndarray, lay, prefix_pad: int, suffix_pad: int):
    """Split packed rows back per group and per response, the last prompt row
    included in each response part.

    verl page, section 3 (forward: the output is split into prefix and suffix
    parts with the last prefix position included; the caller drops the last
    column): prefix_out[g, i] = packed row of prompt token i of group g;
    suffix_out[k, 0] = the group's last prompt row (its logit predicts the
    response's first token), suffix_out[k, 1 + j] = row of response token j.
    Reading where the pages are silent: padding rows are zero, and a group
    without a prompt gives a zero first row. Returns (prefix_out [G,
    prefix_pad, ...], suffix_out [N, suffix_pad + 1, ...]).
    """
    G = len(lay["prefix_lens"])
    N = len(lay["suffix_lens"])
    tail = packed.shape[1:]
    pre = np.zeros((G, prefix_pad) + tail, dtype=packed.dtype)
    suf = np.zeros((N, suffix_pad + 1) + tail, dtype=packed.dtype)
    k = 0
    for g in range(G):
        a = int(lay["group_off"][g])
        P = int(lay["prefix_lens"][g])
        pre[g, :P] = packed[a:a + P]
        cur = a + P
        for _ in range(int(lay["suffix_counts"][g])):
            S = int(lay["suffix_lens"][k])
            if P > 0:
                suf[k, 0] = packed[a + P - 1]
            suf[k, 1:1 + S] = packed[cur:cur + S]
            cur += S
            k += 1
    return pre, suf


# ------------------------------------------------------- padded form --


def group_lens(lay) -> np.ndarray:
    """Tokens of every group's packed row (prefix plus all its responses)."""
    return np.diff(np.asarray(lay["group_off"], dtype=np.int64))


def padded_positions(lay, max_len: int) -> np.ndarray:
    """Position ids of the right-padded form [G, max_len].

    verl page, section 1 (building position ids): the padded tensor starts
    zero-filled and row g holds group g's packed row, so its first n_g entries
    are the packed positions of the group's tokens (``positions``) and the
    right padding keeps 0.
    Pinned by: hand-derived rows of the tiny workload; real tokens equal
    ``positions`` (the packed form).
    """
    G = len(lay["prefix_lens"])
    out = np.zeros((G, max_len), dtype=np.int64)
    pos = positions(lay)
    go = np.asarray(lay["group_off"], dtype=np.int64)
    for g in range(G):
        out[g, :go[g + 1] - go[g]] = pos[go[g]:go[g + 1]]
    return out


def padding_mask(lay, max_len: int) -> np.ndarray:
    """1 on the real tokens of each padded row, 0 on right padding (uint8)."""
    n = group_lens(lay)
    return (np.arange(max_len)[None, :] < n[:, None]).astype(np.uint8)


def pad_rows(packed: np.ndarray, lay, max_len: int) -> np.ndarray:
    """Packed rows [T, ...] to the right-padded form [G, max_len, ...]: row g
    is its group's packed row, then zeros."""
    G = len(lay["prefix_lens"])
    out = np.zeros((G, max_len) + packed.shape[1:], dtype=packed.dtype)
    for g in range(G):
        a, b = int(lay["group_off"][g]), int(lay["group_off"][g + 1])
        out[g, :b - a] = packed[a:b]
    return out


def unpad_rows(padded: np.ndarray, lay) -> np.ndarray:
    """The right-padded form [G, max_len, ...] back to packed rows [T, ...]."""
    parts = [padded[g, :int(n)] for g, n in enumerate(group_lens(lay))]
    if not parts:
        return np.zeros((0,) + padded.shape[2:], dtype=padded.dtype)
    return np.concatenate(parts, axis=0)


# ------------------------------------------------------------------ decode --


def decode_key_rows(lay, cur_lens, k: int) -> np.ndarray:
    """Cache rows that response k's newest token attends to at a decode step.

    PackInfer abstract (I/O-aware grouping): requests that share a prefix are
    co-located and their KV cache is kept group-contiguous while generation
    proceeds, so the prompt's keys are stored, and read, once per group.
    Reading: the cache is the packed layout of ``lay`` with each response's
    segment at its capacity (``lay``'s suffix_lens); response k's valid rows
    are the first len_k = clamp(cur_lens[k], 0, capacity_k) of its segment, the
    last of them holding the token being decoded. Its key set is the group's
    prompt rows plus its own valid rows; a sibling's rows are never read.
    """
    g = int(response_group(lay)[k])
    a = int(lay["group_off"][g])
    P = int(lay["prefix_lens"][g])
    s0 = int(lay["seg_off"][g + k + 1])          # segments: per group prefix, then responses
    cap = int(lay["suffix_lens"][k])
    n = min(max(int(cur_lens[k]), 0), cap)
    return np.concatenate([np.arange(a, a + P), np.arange(s0, s0 + n)]).astype(np.int64)


def response_group(lay) -> np.ndarray:
    """Group of each response, responses in group order."""
    return np.repeat(np.arange(len(lay["prefix_lens"])), lay["suffix_counts"]).astype(np.int64)


def decode_attention(q, k_cache, v_cache, lay, cur_lens, scale: float,
                     num_q_heads: int, num_kv_heads: int, responses=None):
    """One decode step of shared-prefix attention: the newest token of every
    response attends to its group's prompt and its own rows so far.

    q: [N, Hq, d], one query per response (responses in group order);
    k_cache, v_cache: [T, Hkv, d] in the layout's order; cur_lens: [N].
    Written out by definition: softmax of the scaled scores over
    ``decode_key_rows``, times V, in fp64. An empty key set (no prompt and no
    valid row) gives o = 0 and lse = -inf (reading).
    Returns o [N, Hq, d] and lse [Hq, N] (natural log, scaled scores);
    with ``responses`` given, only those rows are computed (the rest stay 0).
    Pinned by: the forward oracle's last row of each response on the compacted
    layout (tests/test_oracle_decode.py), torch's float64 SDPA per response,
    closed forms (one key, constant V, empty set) and a planted sibling leak.
    """
    q = np.asarray(q, dtype=np.float64)
    N, Hq, d = q.shape
    o = np.zeros((N, Hq, d), dtype=np.float64)
    lse = np.full((Hq, N), -np.inf, dtype=np.float64)
    for k in (range(N) if responses is None else responses):
        rows = decode_key_rows(lay, cur_lens, k)
        if len(rows) == 0:
            continue
        kc = np.asarray(k_cache[rows], dtype=np.float64)
        vc = np.asarray(v_cache[rows], dtype=np.float64)
        for h in range(Hq):
            hk = _kv_head(h, Hq, num_kv_heads)
            s = scale * (kc[:, hk] @ q[k, h])
            m = s.max()
            p = np.exp(s - m)
            o[k, h] = (p @ vc[:, hk]) / p.sum()
            lse[h, k] = m + np.log(p.sum())
    return o, lse


def decode_bytes(lay, cur_lens, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V bytes one decode step must read: each group's prompt once plus
    every response's valid rows (the I/O PackInfer's grouping aims at)."""
    rows = 0
    for g in range(len(lay["prefix_lens"])):
        if int(lay["suffix_counts"][g]) > 0:
            rows += int(lay["prefix_lens"][g])
    caps = np.asarray(lay["suffix_lens"], dtype=np.int64)
    rows += int(np.clip(np.asarray(cur_lens, dtype=np.int64), 0, caps).sum())
    return rows * num_kv_heads * head_dim * elem_bytes * 2


# ---------------------------------------------------------- FLOP accounting --


def useful_pairs(lay) -> int:
    """Number of allowed (query, key) pairs of the packed layout (per head).

    Per group: P(P+1)/2 for the prompt plus S*P + S(S+1)/2 per response.
    Pinned by: count of the dense mask; hand-derived 217 for the tiny workload.
    """
    total = 0
    k = 0
    for g in range(len(lay["prefix_lens"])):
        P = int(lay["prefix_lens"][g])
        total += P * (P + 1) // 2
        for _ in range(int(lay["suffix_counts"][g])):
            S = int(lay["suffix_lens"][k])
            k += 1
            total += S * P + S * (S + 1) // 2
    return total


def unpacked_pairs(lay) -> int:
    """Pairs of causal attention over every unpacked sequence (the work that
    preference packing removes is the repeated prompt triangle)."""
    total = 0
    for g, p0, P, (s0, s1) in sequences(lay):
        L = P + (s1 - s0)
        total += L * (L + 1) // 2
    return total


def useful_flop(lay, num_q_heads: int, head_dim: int) -> int:
    """Useful FLOP: QK^T and PV multiply-adds over allowed pairs only."""
    return 4 * head_dim * num_q_heads * useful_pairs(lay)


# -------------------------------------------------------------- pipeline ----


def pipeline(q, k, v, lay, theta: float, scale: float, num_q_heads: int,
             num_kv_heads: int, dtype: str):
    """positions -> RoPE (fp64, then rounded to the storage dtype, as the
    RoPE step hands its result over in that dtype) -> attention."""
    pos = positions(lay)
    qr = storage_round(rope(q, pos, theta), dtype)
    kr = storage_round(rope(k, pos, theta), dtype)
    o, lse = attention(qr, kr, v, lay, scale, num_q_heads, num_kv_heads)
    return pos, qr, kr, o, lse
