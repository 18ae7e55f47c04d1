"""Seeded random shapes against the oracle: prefill (B, heads, GQA group,
ragged Lq/Lkv, start position, window, D = 64/128/256) and varlen tables
(store size, heads, D, segment modes), to the same tolerance as the fixed
cases."""
import math
import random

import pytest
import torch

import causal_gqa_prefill_flash_amd as attn
import oracle
from causal_gqa_prefill_flash_amd import synth
from gpu_util import compare, dev, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", range(64))
def test_random_prefill_shape(seed):
    rng = random.Random(9100 + seed)
    D = rng.choice([64, 128, 256])
    Hkv = rng.choice([1, 2, 4])
    g = rng.choice([1, 2, 3, 4, 8])
    Hq = Hkv * g
    if Hq > 16:
        Hq, g = Hkv * (16 // Hkv), 16 // Hkv
    B = rng.choice([1, 2])
    Lq = rng.randint(1, 200)
    Lkv = rng.randint(0, 1500)
    q_pos0 = rng.choice([Lkv - Lq, rng.randint(-60, max(Lkv, 1))])
    window = rng.choice([0, 0, rng.randint(1, 400)])
    scale = rng.choice([1.0 / math.sqrt(D), 0.2, -0.1])
    say("random prefill", seed, dict(B=B, Hq=Hq, Hkv=Hkv, Lq=Lq, Lkv=Lkv, D=D, q_pos0=q_pos0,
                                       window=window, scale=scale))
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=200 + seed)
    out = attn.causal_prefill(q.to(dev()), k.to(dev()), v.to(dev()), scale=scale, q_pos0=q_pos0,
                              window=window)
    ref = oracle.prefill(q, k, v, scale, q_pos0=q_pos0, window=window)
    compare(out, ref, "random prefill %d" % seed)


@pytest.mark.parametrize("seed", range(32))
def test_random_varlen_table(seed):
    rng = random.Random(9200 + seed)
    D = rng.choice([64, 128])
    Hkv = rng.choice([1, 2])
    Hq = Hkv * rng.choice([1, 2, 4, 8])
    rows = rng.choice([512, 1024, 3000])
    cols = rng.randint(3, 6)
    S = rng.randint(1, 2 * (cols - 1))
    info, attr, t = [], [], 0
    for _ in range(S):
        t += rng.randint(0, 3)
        q_len = rng.choice([1, 2, 4, 7, 16, 33, 100])
        col = rng.randint(0, cols - 2)
        causal = rng.choice([1, 1, 0])
        ring = rng.choice([0, 0, rng.randint(q_len + 8, rows)])
        R = ring if ring > 0 else rows
        kv_end = rng.randint(0, 3 * R) if ring else rng.randint(0, rows)
        # ring segments mostly with a window the ring holds (R - q_len + 1
        # keys at most), sometimes wider (flagged ATTN_SEG_SPAN)
        wmax = R - q_len + 1 if ring and rng.random() < 0.8 else R
        window = rng.choice([0, rng.randint(1, wmax)]) if (causal or rng.random() < 0.3) else 0
        info.append((t, q_len, col, kv_end))
        attr.append((causal, window, ring))
        t += q_len
    T = t + rng.randint(0, 5)
    say("random varlen", seed, dict(D=D, Hq=Hq, Hkv=Hkv, rows=rows, cols=cols, S=S, T=T))
    info = torch.tensor(info, dtype=torch.int32)
    attr = torch.tensor(attr, dtype=torch.int32)
    q, ks, vs = synth.varlen_inputs(T, rows, cols, Hkv, D, Hq, wid=300 + seed)
    out, ws = attn.sdpa_varlen(q.to(dev()), ks.to(dev()), vs.to(dev()), info.to(dev()),
                               seg_attr=attr.to(dev()))
    err = attn.varlen_read_error(ws, S, T)
    ref, flags = oracle.varlen(q, ks, vs, info, seg_attr=attr, return_flags=True)
    say("  flags", flags)
    assert err == flags and flags & ~attn.SEG_SPAN == 0
    compare(out, ref, "random varlen %d" % seed)


@pytest.mark.parametrize("seed", range(12))
def test_random_varlen_tables_with_long_segments(seed):
    """Seeded tables over an 8192-row store with q_len up to 640 and kv_end up
    to the store: enough q-block slots that the launch chooses the key-split
    size per table on the device (coarser splits than 512 keys for the larger
    tables), with causal, non-causal, windowed and ring segments."""
    rng = random.Random(9300 + seed)
    D = rng.choice([64, 128])
    Hkv = 2
    Hq = Hkv * rng.choice([2, 4, 8])
    rows, cols = 8192, 6
    S = rng.randint(3, 8)
    info, attr, t = [], [], 0
    for s_ in range(S):
        t += rng.randint(0, 3)
        q_len = rng.choice([1, 3, 40, 200, 640])
        col = s_ % (cols - 1)
        causal = rng.choice([1, 1, 0])
        ring = rng.choice([0, 0, 2559]) if causal else 0
        R = ring if ring else rows
        kv_end = rng.randint(q_len, 3 * R if ring else rows)
        window = (rng.choice([0, 2048]) if not ring else R - q_len + 1) if causal else 0
        info.append((t, q_len, col, kv_end))
        attr.append((causal, window, ring))
        t += q_len
    T = t + rng.randint(0, 5)
    say("random long varlen", seed, dict(D=D, Hq=Hq, S=S, T=T))
    info = torch.tensor(info, dtype=torch.int32)
    attr = torch.tensor(attr, dtype=torch.int32)
    q, ks, vs = synth.varlen_inputs(T, rows, cols, Hkv, D, Hq, wid=400 + seed)
    out, ws = attn.sdpa_varlen(q.to(dev()), ks.to(dev()), vs.to(dev()), info.to(dev()),
                               seg_attr=attr.to(dev()))
    err = attn.varlen_read_error(ws, S, T)
    ref, flags = oracle.varlen(q, ks, vs, info, seg_attr=attr, return_flags=True)
    assert err == flags == 0
    compare(out, ref, "random long varlen %d" % seed)
