"""Seeded synthetic inputs shared by the tests and the benchmark.

This module holds no attention arithmetic: it only draws tensors and builds
segment tables.  Both the library's callers and the oracle's callers take
their inputs from here, so the two sides read identical bf16 bits.

Recipe: values are N(0,1) drawn in fp32 by a CPU ``torch.Generator`` seeded
per tensor, then rounded to bf16.  Seeds are 1001 (Q), 1002 (K), 1003 (V)
plus 100 x the workload id, unless a test passes its own.
"""
import math

import torch

SEED_Q, SEED_K, SEED_V = 1001, 1002, 1003


def randn_bf16(shape, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=0):
    """Contiguous [B,H,L,D] bf16 Q, K, V on the CPU."""
    q = randn_bf16((B, Hq, Lq, D), SEED_Q + 100 * wid)
    k = randn_bf16((B, Hkv, Lkv, D), SEED_K + 100 * wid)
    v = randn_bf16((B, Hkv, Lkv, D), SEED_V + 100 * wid)
    return q, k, v


# The prefill workloads (B, Hq, Hkv, D, Lq, Lkv, q_pos0 or None for end-aligned).
PREFILL_WORKLOADS = {
    "tiny": dict(wid=1, B=1, Hq=4, Hkv=1, D=64, Lq=256, Lkv=256, q_pos0=None),
    "d64_lq512_lkv16k": dict(wid=2, B=1, Hq=16, Hkv=2, D=64, Lq=512, Lkv=16384, q_pos0=None),
    # the same short chunk at D = 128 (a row of the pages' operator table)
    "d128_lq512_lkv16k": dict(wid=7, B=1, Hq=16, Hkv=2, D=128, Lq=512, Lkv=16384, q_pos0=None),
    "d128_lq1k_lkv128k": dict(wid=3, B=1, Hq=16, Hkv=2, D=128, Lq=1024, Lkv=131072, q_pos0=None),
    # the same, with key positions shifted past the first 16 query positions
    "d128_lq1k_lkv128k_masked16": dict(wid=3, B=1, Hq=16, Hkv=2, D=128, Lq=1024, Lkv=131072,
                                       q_pos0=-16),
    "d64_lq4k_lkv128k": dict(wid=4, B=1, Hq=16, Hkv=2, D=64, Lq=4096, Lkv=131072, q_pos0=None),
    "d128_lq4k_lkv128k": dict(wid=4, B=1, Hq=16, Hkv=2, D=128, Lq=4096, Lkv=131072, q_pos0=None),
    # head dimension 256 on the long-context shape
    "d256_lq1k_lkv128k": dict(wid=5, B=1, Hq=16, Hkv=2, D=256, Lq=1024, Lkv=131072, q_pos0=None),
    "d256_lq512_lkv16k": dict(wid=6, B=1, Hq=16, Hkv=2, D=256, Lq=512, Lkv=16384, q_pos0=None),
}

# The D=128 long-context chunk with keys that push every workgroup onto the
# exact softmax rerun (see rising_logits).
PREFILL_WORKLOADS["d128_lq1k_lkv128k_rising"] = dict(
    wid=3, B=1, Hq=16, Hkv=2, D=128, Lq=1024, Lkv=131072, q_pos0=None, logits="rising")


def rising_logits(q, k, scale, nats, period):
    """Q made positive and K moved along the all-ones direction so that the
    logit of key j against the mean query rises by nats * (j mod period) /
    period: a saw-tooth whose every period rises by `nats`.  Returns (q, k),
    bf16.  No attention arithmetic: a shift of the inputs only."""
    qpos = q.abs()
    qsum = qpos.float().sum(-1).mean().item()
    Lkv = k.shape[2]
    ramp = nats * (torch.arange(Lkv, dtype=torch.float32) % period) / period
    shift = (ramp / (scale * qsum)).view(1, 1, -1, 1)
    return qpos, (k.float() + shift).to(torch.bfloat16)


# Varlen column store of the segment-table workload: [rows, cols, Hkv, D];
# the last column is scratch.  Packed Q/out are [T, Hq, D].
VARLEN_STORE = dict(rows=8192, cols=9, Hkv=2, D=128, Hq=16)
RING_ROWS = 2048 + 511  # window + max_write - 1 with window 2048, max_write 512
RING_WINDOW = 2048


def pinned_varlen_table():
    """The pinned 8-segment table.

    Returns (seq_info [S,4], seg_attr [S,3], T) as int32 CPU tensors and an
    int.  Packed order s5, s0, s2, s7, s1, s4, s6, s3 with 3-row gaps and a
    17-row tail leaves 41 packed rows uncovered.
    Modes: s0-s3 causal flat; s4-s5 non-causal flat; s6-s7 causal with a
    2048-key window on a 2559-row ring.
    """
    # (q_start, q_len, col, kv_end), (causal, window, ring_rows)
    rows = [
        ((518, 1, 3, 8192), (1, 0, 0)),
        ((545, 512, 0, 700), (1, 0, 0)),
        ((522, 16, 5, 64), (1, 0, 0)),
        ((1582, 128, 1, 3000), (1, 0, 0)),
        ((1060, 4, 7, 5000), (0, 0, 0)),
        ((3, 512, 2, 512), (0, 0, 0)),
        ((1067, 512, 4, 8192), (1, RING_WINDOW, RING_ROWS)),
        ((541, 1, 6, 2000), (1, RING_WINDOW, RING_ROWS)),
    ]
    seq_info = torch.tensor([r[0] for r in rows], dtype=torch.int32)
    seg_attr = torch.tensor([r[1] for r in rows], dtype=torch.int32)
    T = 1727
    return seq_info, seg_attr, T


def random_varlen_table(seed, T_max=None, S=8, q_lens=(1, 4, 16, 128, 512),
                        kv_lo=64, kv_hi=8192):
    """A seeded 8-segment table in the pinned table's modes.

    q_len uniform over ``q_lens``; kv_end = floor(exp(U(ln kv_lo, ln kv_hi)))
    clamped to >= q_len; columns a random permutation of 0..S-1; segments
    packed in a random order with 0-3 row gaps.  Returns (seq_info, seg_attr, T).
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    idx = torch.randint(0, len(q_lens), (S,), generator=g)
    qlen = [q_lens[int(i)] for i in idx]
    u = torch.rand(S, generator=g, dtype=torch.float64)
    kv = [int(math.floor(math.exp(math.log(kv_lo) + float(x) * (math.log(kv_hi) - math.log(kv_lo)))))
          for x in u]
    kv = [min(max(kv_i, q), kv_hi) for kv_i, q in zip(kv, qlen)]
    colp = torch.randperm(S, generator=g).tolist()
    order = torch.randperm(S, generator=g).tolist()
    gaps = torch.randint(0, 4, (S + 1,), generator=g).tolist()
    attrs = []
    for s in range(S):
        if s < S // 2:
            attrs.append((1, 0, 0))
        elif s < 3 * S // 4:
            attrs.append((0, 0, 0))
        else:
            attrs.append((1, RING_WINDOW, RING_ROWS))
    info = [None] * S
    t = gaps[0]
    for n, s in enumerate(order):
        info[s] = (t, qlen[s], colp[s], kv[s])
        t += qlen[s] + gaps[n + 1]
    T = t
    if T_max is not None and T > T_max:
        raise ValueError("table exceeds T_max")
    return (torch.tensor(info, dtype=torch.int32), torch.tensor(attrs, dtype=torch.int32), T)


def varlen_inputs(T, rows=8192, cols=9, Hkv=2, D=128, Hq=16, wid=5):
    """Packed Q [T,Hq,D] and the K/V column stores [rows,cols,Hkv,D], bf16 CPU."""
    q = randn_bf16((T, Hq, D), SEED_Q + 100 * wid)
    k = randn_bf16((rows, cols, Hkv, D), SEED_K + 100 * wid)
    v = randn_bf16((rows, cols, Hkv, D), SEED_V + 100 * wid)
    return q, k, v
