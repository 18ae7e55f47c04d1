"""Pure-Python brute-force attention for tiny inputs (no numpy, no torch math).

A second route to the same definition as the oracle, used to pin it: the
softmax weight of key j is computed as 1 / sum_k exp(s_k - s_j), with no
row maximum and no two-pass structure, and visible sets are built as Python
sets from the positional rules.  Inputs are nested lists of floats that are
already bf16 values.
"""
import math


def visible_prefill(i, Lkv, q_pos0, window):
    p = q_pos0 + i
    return {j for j in range(Lkv) if j <= p and (window <= 0 or j > p - window)}


def _attend(qrow, keys, vals, scale):
    """keys/vals: dict key-index -> row.  Returns the output row."""
    D = len(qrow)
    if not keys:
        return [0.0] * D
    s = {j: scale * math.fsum(qrow[d] * keys[j][d] for d in range(D)) for j in keys}
    w = {j: 1.0 / math.fsum(math.exp(s[k] - s[j]) for k in keys) for j in keys}
    return [math.fsum(w[j] * vals[j][d] for j in keys) for d in range(D)]


def prefill(q, k, v, scale, q_pos0, window=0):
    """q [B][Hq][Lq][D], k/v [B][Hkv][Lkv][D] -> out [B][Hq][Lq][D]."""
    B, Hq, Lq = len(q), len(q[0]), len(q[0][0])
    Hkv, Lkv = len(k[0]), len(k[0][0])
    g = Hq // Hkv
    out = []
    for b in range(B):
        ob = []
        for h in range(Hq):
            hk = h // g
            oh = []
            for i in range(Lq):
                vis = visible_prefill(i, Lkv, q_pos0, window)
                oh.append(_attend(q[b][h][i], {j: k[b][hk][j] for j in vis},
                                  {j: v[b][hk][j] for j in vis}, scale))
            ob.append(oh)
        out.append(ob)
    return out


def ring_holds(R, kv_end):
    """Which positions a ring of R rows still holds after positions
    0 .. kv_end - 1 were written in order to rows position mod R: the set of
    positions x whose row was not overwritten by a later position."""
    last = {}
    for pos in range(kv_end):
        last[pos % R] = pos
    return {x for r, x in last.items()}


def varlen(q, ks, vs, seq_info, seg_attr, scale, stale=None):
    """q [T][Hq][D]; ks/vs [rows][cols][Hkv][D]; seq_info list of 4-tuples;
    seg_attr list of (causal, window, ring_rows) with ring_rows <= 0 meaning
    all rows.  All segments are assumed in range and disjoint.  A segment
    that would read a key its ring no longer holds (simulated by ring_holds)
    is not attended: its rows stay 0 and, when ``stale`` is a list, its
    index is appended to it."""
    T, Hq, D = len(q), len(q[0]), len(q[0][0])
    rows, Hkv = len(ks), len(ks[0][0])
    g = Hq // Hkv
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(T)]
    for n, ((q_start, q_len, col, kv_end), (causal, window, ring_rows)) in \
            enumerate(zip(seq_info, seg_attr)):
        R = ring_rows if ring_rows > 0 else rows
        held = ring_holds(R, kv_end)
        vis_rows = []
        for j in range(q_len):
            p = kv_end - q_len + j
            vis_rows.append({x for x in range(kv_end)
                             if (not causal or x <= p) and (window <= 0 or x > p - window)})
        if any(not vis <= held for vis in vis_rows):
            if stale is not None:
                stale.append(n)
            continue
        for j, vis in enumerate(vis_rows):
            for h in range(Hq):
                hk = h // g
                out[q_start + j][h] = _attend(
                    q[q_start + j][h],
                    {x: ks[x % R][col][hk] for x in vis},
                    {x: vs[x % R][col][hk] for x in vis}, scale)
    return out
