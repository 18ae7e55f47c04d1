"""Pins of the oracle against what the pages and the mathematics fix.

None of these re-types the oracle's formula: they use closed forms with exact
rational answers (tests/golden), brute force by another route (tests/brute.py),
invariants, special cases that reduce to plainer attention, and torch's
float64 SDPA with an explicit boolean mask.
"""
import json
import math
import os
from fractions import Fraction

import pytest
import torch

import brute
import oracle
from causal_gqa_prefill_flash_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bf(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16)


def _lists(t):
    return t.to(torch.float64).tolist()


def _frac_tensor(nested):
    return torch.tensor([[[[float(Fraction(x)) for x in r] for r in h] for h in b] for b in nested],
                        dtype=torch.float64)


def _scale(s):
    return math.log(2.0) if s == "ln2" else float(s)


# ---------------------------------------------------------------- golden cases

def test_golden_causal_rational():
    g = json.load(open(os.path.join(GOLDEN, "causal_rational_3x3.json")))
    out = oracle.prefill(_bf(g["q"]), _bf(g["k"]), _bf(g["v"]), _scale(g["scale"]),
                         q_pos0=g["q_pos0"], window=g["window"])
    torch.testing.assert_close(out, _frac_tensor(g["out"]), rtol=1e-13, atol=1e-13)


def test_golden_window_rational():
    g = json.load(open(os.path.join(GOLDEN, "window_rational.json")))
    out = oracle.prefill(_bf(g["q"]), _bf(g["k"]), _bf(g["v"]), _scale(g["scale"]),
                         q_pos0=g["q_pos0"], window=g["window"])
    torch.testing.assert_close(out, _frac_tensor(g["out"]), rtol=1e-13, atol=1e-13)


def test_golden_ring_varlen_rational():
    g = json.load(open(os.path.join(GOLDEN, "ring_varlen_rational.json")))
    rows, cols = g["rows"], g["cols"]
    nan = float("nan")
    ks = torch.full((rows, cols, 1, 2), nan)
    vs = torch.full((rows, cols, 1, 2), nan)
    ks[:, 0, 0, :] = torch.tensor([[float(x) for x in r] for r in g["k_col0"]])
    vs[:, 0, 0, :] = torch.tensor([[float(x) for x in r] for r in g["v_col0"]])
    out, flags = oracle.varlen(_bf(g["q"]), ks.to(torch.bfloat16), vs.to(torch.bfloat16),
                               g["seq_info"], scale=_scale(g["scale"]), causal=g["causal"],
                               window=g["window"], ring_rows=g["ring_rows"], return_flags=True)
    assert flags == 0
    exp = torch.tensor([[[float(Fraction(x)) for x in h] for h in t] for t in g["out"]],
                       dtype=torch.float64)
    torch.testing.assert_close(out, exp, rtol=1e-13, atol=1e-13)


def test_golden_noncausal_window_rational():
    g = json.load(open(os.path.join(GOLDEN, "noncausal_window_rational.json")))
    rows, cols = g["rows"], g["cols"]
    nan = float("nan")
    ks = torch.full((rows, cols, 1, 2), nan)
    vs = torch.full((rows, cols, 1, 2), nan)
    ks[:, 0, 0, :] = torch.tensor([[float(x) for x in r] for r in g["k_col0"]])
    vs[:, 0, 0, :] = torch.tensor([[float(x) for x in r] for r in g["v_col0"]])
    out, flags = oracle.varlen(_bf(g["q"]), ks.to(torch.bfloat16), vs.to(torch.bfloat16),
                               g["seq_info"], seg_attr=g["seg_attr"], scale=_scale(g["scale"]),
                               return_flags=True)
    assert flags == 0
    exp = torch.tensor([[[float(Fraction(x)) for x in h] for h in t] for t in g["out"]],
                       dtype=torch.float64)
    torch.testing.assert_close(out, exp, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("Lq,Lkv,q_pos0,window", [
    (16, 16, 0, 0),      # the tiny workload cut to 16 rows
    (5, 16, 11, 0),      # end-aligned chunk, Lq != Lkv
    (7, 12, 5, 4),       # sliding window
    (6, 9, -2, 0),       # first two rows see nothing
    (4, 0, 0, 0),        # no keys at all
])
def test_prefill_vs_brute(Lq, Lkv, q_pos0, window):
    B, Hq, Hkv, D = 2, 4, 2, 8
    q = synth.randn_bf16((B, Hq, Lq, D), 11)
    k = synth.randn_bf16((B, Hkv, Lkv, D), 12)
    v = synth.randn_bf16((B, Hkv, Lkv, D), 13)
    scale = 1.0 / math.sqrt(D)
    got = oracle.prefill(q, k, v, scale, q_pos0=q_pos0, window=window)
    ref = torch.tensor(brute.prefill(_lists(q), _lists(k), _lists(v), scale, q_pos0, window),
                       dtype=torch.float64).reshape(B, Hq, Lq, D)
    torch.testing.assert_close(got, ref, rtol=1e-12, atol=1e-12)


def test_varlen_vs_brute_wrapped_ring():
    rows, cols, Hkv, D, Hq = 9, 4, 1, 8, 2
    R, W = 7, 4
    ks = synth.randn_bf16((rows, cols, Hkv, D), 21)
    vs = synth.randn_bf16((rows, cols, Hkv, D), 22)
    # (q_start, q_len, col, kv_end): a wrapped ring, a fresh ring, a flat one
    seq_info = [(1, 4, 0, 11), (6, 2, 2, 3), (9, 3, 1, 9)]
    seg_attr = [(1, W, R), (1, W, R), (1, 0, 0)]
    T = 13
    q = synth.randn_bf16((T, Hq, D), 23)
    scale = 0.37
    got, flags = oracle.varlen(q, ks, vs, seq_info, seg_attr=seg_attr, scale=scale,
                               return_flags=True)
    assert flags == 0
    ref = brute.varlen(_lists(q), _lists(ks), _lists(vs), seq_info, seg_attr, scale)
    torch.testing.assert_close(got, torch.tensor(ref, dtype=torch.float64), rtol=1e-12, atol=1e-12)
    # rows 0, 5, 8, 12 are covered by no segment
    for t in (0, 5, 8, 12):
        assert torch.count_nonzero(got[t]) == 0


def test_varlen_noncausal_vs_brute():
    rows, cols, Hkv, D, Hq = 12, 3, 2, 4, 4
    ks = synth.randn_bf16((rows, cols, Hkv, D), 31)
    vs = synth.randn_bf16((rows, cols, Hkv, D), 32)
    seq_info = [(0, 3, 1, 10), (3, 2, 0, 2)]
    seg_attr = [(0, 0, 0), (0, 3, 0)]  # second: non-causal with a lower bound
    q = synth.randn_bf16((5, Hq, D), 33)
    got = oracle.varlen(q, ks, vs, seq_info, seg_attr=seg_attr, scale=0.5)
    ref = brute.varlen(_lists(q), _lists(ks), _lists(vs), seq_info, seg_attr, 0.5)
    torch.testing.assert_close(got, torch.tensor(ref, dtype=torch.float64), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ closed forms

def test_one_key_row_returns_that_value():
    q, k, v = synth.prefill_inputs(1, 4, 1, 8, 8, 16, wid=7)
    out = oracle.prefill(q, k, v, 0.25, q_pos0=0)
    # row 0 sees key 0 alone: its output is exactly v[0] for every head
    for h in range(4):
        assert torch.equal(out[0, h, 0], v[0, 0, 0].double())
    # with a window of one key every row returns its own value row
    out1 = oracle.prefill(q, k, v, 0.25, q_pos0=0, window=1)
    for h in range(4):
        assert torch.equal(out1[0, h], v[0, 0].double())


@pytest.mark.parametrize("zero_q", [True, False])
def test_uniform_weights_give_mean_of_visible_values(zero_q):
    B, Hq, Hkv, Lq, Lkv, D = 1, 2, 1, 6, 10, 8
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=8)
    if zero_q:
        q = torch.zeros_like(q)
        scale = 0.125
    else:
        scale = 0.0
    out = oracle.prefill(q, k, v, scale)
    for i in range(Lq):
        p = Lkv - Lq + i
        mean = v[0, 0, : p + 1].double().mean(0)
        torch.testing.assert_close(out[0, 0, i], mean, rtol=1e-13, atol=1e-13)


def test_equal_keys_give_mean_of_values():
    q, k, v = synth.prefill_inputs(1, 2, 1, 4, 4, 8, wid=9)
    k = k[:, :, :1].expand(1, 1, 4, 8).contiguous()
    out = oracle.prefill(q, k, v, 0.3, q_pos0=0)
    for i in range(4):
        torch.testing.assert_close(out[0, 1, i], v[0, 0, : i + 1].double().mean(0),
                                   rtol=1e-13, atol=1e-13)


def test_fully_masked_rows_are_exact_zeros():
    q, k, v = synth.prefill_inputs(1, 4, 2, 20, 20, 8, wid=10)
    out = oracle.prefill(q, k, v, 0.35, q_pos0=-16)
    assert torch.count_nonzero(out[:, :, :16]) == 0
    # row 16 sits at position 0 and sees key 0 alone
    assert torch.equal(out[0, 0, 16], v[0, 0, 0].double())
    assert torch.isfinite(out).all()


def test_single_two_key_ln3():
    # scores 0 and ln 3: weights 1/4, 3/4
    q = _bf([[[[1.0, 0.0]]]])
    k = _bf([[[[0.0, 0.0], [1.0, 0.0]]]])
    v = _bf([[[[4.0, 0.0], [0.0, 8.0]]]])
    out = oracle.prefill(q, k, v, math.log(3.0))
    torch.testing.assert_close(out[0, 0, 0], torch.tensor([1.0, 6.0], dtype=torch.float64),
                               rtol=1e-14, atol=1e-14)


def test_saturated_scores_stay_finite_and_pick_the_largest():
    """Scores in the thousands: without the exact row maximum as the softmax
    reference the exponentials overflow; with it the weights saturate onto
    the best-scoring visible key, whose value row comes back."""
    B, Hq, Hkv, Lq, Lkv, D = 1, 2, 1, 5, 9, 16
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=18)
    out = oracle.prefill(q, k, v, 2000.0)
    assert torch.isfinite(out).all()
    s = q.double() @ k.double().repeat_interleave(2, 1).transpose(-1, -2)
    for h in range(Hq):
        for i in range(Lq):
            p = Lkv - Lq + i
            j = int(torch.argmax(s[0, h, i, : p + 1]))
            torch.testing.assert_close(out[0, h, i], v[0, 0, j].double(), rtol=0, atol=1e-12)


# ------------------------------------------------------------ invariants

def test_probability_rows_sum_to_one():
    q, k, v = synth.prefill_inputs(1, 4, 2, 12, 40, 16, wid=11)
    _, p = oracle.prefill(q, k, v, 0.25, window=9, return_probs=True)
    s = p.sum(-1)
    torch.testing.assert_close(s, torch.ones_like(s), rtol=0, atol=1e-12)
    # and the weights vanish exactly outside the visible band
    for i in range(12):
        pos = 40 - 12 + i
        assert torch.count_nonzero(p[..., i, pos + 1:]) == 0
        assert torch.count_nonzero(p[..., i, : pos - 9 + 1]) == 0


def test_masked_keys_do_not_matter_and_the_boundary_key_does():
    B, Hq, Hkv, Lq, Lkv, D = 1, 4, 2, 8, 32, 16
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=12)
    W = 6
    base = oracle.prefill(q, k, v, 0.25, window=W)
    i = 3
    p = Lkv - Lq + i
    # future keys and keys before the window, including NaN
    for j in (p + 1, Lkv - 1, p - W, 0):
        k2, v2 = k.clone(), v.clone()
        k2[:, :, j] = float("nan")
        v2[:, :, j] = float("nan")
        out = oracle.prefill(q, k2, v2, 0.25, window=W)
        assert torch.equal(out[:, :, i], base[:, :, i]), j
    # the newest and the oldest visible key both change the row
    for j in (p, p - W + 1):
        v2 = v.clone()
        v2[:, :, j] += 1.0
        out = oracle.prefill(q, k, v2, 0.25, window=W)
        assert not torch.equal(out[:, :, i], base[:, :, i]), j


def test_window_covering_everything_equals_global_causal():
    q, k, v = synth.prefill_inputs(1, 4, 2, 10, 30, 16, wid=13)
    a = oracle.prefill(q, k, v, 0.2)
    b = oracle.prefill(q, k, v, 0.2, window=31)
    assert torch.equal(a, b)


def test_gqa_equals_mha_with_repeated_heads():
    B, Hq, Hkv, Lq, Lkv, D = 2, 8, 2, 6, 14, 16
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=14)
    gqa = oracle.prefill(q, k, v, 0.25)
    g = Hq // Hkv
    mha = oracle.prefill(q, k.repeat_interleave(g, dim=1), v.repeat_interleave(g, dim=1), 0.25)
    assert torch.equal(gqa, mha)


def test_strided_views_read_through_real_strides():
    B, Hq, Hkv, Lq, Lkv, D = 1, 4, 2, 6, 12, 16
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=15)
    ref = oracle.prefill(q, k, v, 0.25)
    # BSHD storage viewed as BHSD, and a padded L-stride
    qb = q.transpose(1, 2).contiguous().transpose(1, 2)
    kp = torch.zeros(B, Hkv, Lkv, D + 8, dtype=torch.bfloat16)
    kp[..., :D] = k
    out = oracle.prefill(qb, kp[..., :D], v, 0.25)
    assert torch.equal(out, ref)
    # a non-unit innermost stride is still read correctly by the oracle
    vt = v.transpose(2, 3).contiguous().transpose(2, 3)
    assert torch.equal(oracle.prefill(q, k, vt, 0.25), ref)
    qt = q.transpose(2, 3).contiguous().transpose(2, 3)
    assert torch.equal(oracle.prefill(qt, k, v, 0.25), ref)


def test_matches_torch_sdpa_float64_with_explicit_mask():
    B, Hq, Hkv, Lq, Lkv, D = 1, 4, 2, 24, 64, 32
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=16)
    for q_pos0, W in ((Lkv - Lq, 0), (Lkv - Lq, 7), (3, 0)):
        out = oracle.prefill(q, k, v, 1.0 / math.sqrt(D), q_pos0=q_pos0, window=W)
        pos = torch.arange(Lq)[:, None] + q_pos0
        j = torch.arange(Lkv)[None, :]
        mask = j <= pos
        if W > 0:
            mask &= j > pos - W
        g = Hq // Hkv
        ref = torch.nn.functional.scaled_dot_product_attention(
            q.double(), k.double().repeat_interleave(g, 1), v.double().repeat_interleave(g, 1),
            attn_mask=mask)
        torch.testing.assert_close(out, ref, rtol=1e-12, atol=1e-12)


def test_row_selection_matches_full():
    q, k, v = synth.prefill_inputs(1, 4, 2, 20, 50, 16, wid=17)
    full = oracle.prefill(q, k, v, 0.25)
    sel = [0, 7, 19]
    part = oracle.prefill(q, k, v, 0.25, rows=sel)
    assert torch.equal(part, full[:, :, sel])


# ------------------------------------------------------------ varlen special cases

def _store(rows, cols, Hkv, D, seed):
    return synth.randn_bf16((rows, cols, Hkv, D), seed), synth.randn_bf16((rows, cols, Hkv, D), seed + 1)


def test_varlen_single_causal_segment_equals_prefill_on_the_column():
    rows, cols, Hkv, D, Hq = 64, 3, 2, 16, 8
    ks, vs = _store(rows, cols, Hkv, D, 41)
    q_len, kv_end, col = 5, 37, 1
    q = synth.randn_bf16((q_len + 2, Hq, D), 43)
    out = oracle.varlen(q, ks, vs, [(1, q_len, col, kv_end)], scale=0.25)
    # the column as a [1, Hkv, kv_end, D] strided view
    kcol = ks[:kv_end, col].permute(1, 0, 2).unsqueeze(0)
    vcol = vs[:kv_end, col].permute(1, 0, 2).unsqueeze(0)
    qv = q[1:1 + q_len].permute(1, 0, 2).unsqueeze(0)
    ref = oracle.prefill(qv, kcol, vcol, 0.25, q_pos0=kv_end - q_len)
    assert torch.equal(out[1:1 + q_len], ref[0].permute(1, 0, 2))
    assert torch.count_nonzero(out[0]) == 0 and torch.count_nonzero(out[-1]) == 0


def test_varlen_noncausal_full_block_is_bidirectional_attention():
    rows, cols, Hkv, D, Hq = 16, 2, 1, 8, 2
    ks, vs = _store(rows, cols, Hkv, D, 51)
    q = synth.randn_bf16((6, Hq, D), 53)
    out = oracle.varlen(q, ks, vs, [(0, 6, 0, 6)], causal=0, scale=0.3)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.double().permute(1, 0, 2), ks[:6, 0].double().permute(1, 0, 2).repeat_interleave(2, 0),
        vs[:6, 0].double().permute(1, 0, 2).repeat_interleave(2, 0), scale=0.3)
    torch.testing.assert_close(out, ref.permute(1, 0, 2), rtol=1e-12, atol=1e-12)


def test_varlen_ring_before_wrap_equals_flat():
    rows, cols, Hkv, D, Hq = 40, 3, 1, 8, 2
    ks, vs = _store(rows, cols, Hkv, D, 61)
    q = synth.randn_bf16((4, Hq, D), 63)
    seg = [(0, 4, 1, 20)]
    a = oracle.varlen(q, ks, vs, seg, seg_attr=[(1, 6, 25)], scale=0.3)
    b = oracle.varlen(q, ks, vs, seg, seg_attr=[(1, 6, 0)], scale=0.3)
    assert torch.equal(a, b)


def test_ring_of_window_plus_max_write_minus_one_rows_holds_every_visible_key():
    """The ring size rule on the pages fixes the window convention.

    A ring of W + q_len - 1 rows, written in position order, must reproduce
    the attention over the same keys stored flat at their true positions.
    Under the reading 'W keys including the query's own position' it does;
    a window of W + 1 keys would alias the oldest key onto the newest row.
    """
    W, q_len, kv_end = 6, 4, 23
    R = W + q_len - 1
    Hkv, D, Hq = 1, 8, 2
    flat_k = synth.randn_bf16((kv_end, 2, Hkv, D), 71)
    flat_v = synth.randn_bf16((kv_end, 2, Hkv, D), 72)
    ring_k = torch.zeros((R, 2, Hkv, D), dtype=torch.bfloat16)
    ring_v = torch.zeros((R, 2, Hkv, D), dtype=torch.bfloat16)
    for pos in range(kv_end):  # later positions overwrite earlier ones
        ring_k[pos % R] = flat_k[pos]
        ring_v[pos % R] = flat_v[pos]
    q = synth.randn_bf16((q_len, Hq, D), 73)
    seg = [(0, q_len, 0, kv_end)]
    a = oracle.varlen(q, ring_k, ring_v, seg, seg_attr=[(1, W, R)], scale=0.3)
    b = oracle.varlen(q, flat_k, flat_v, seg, seg_attr=[(1, W, 0)], scale=0.3)
    assert torch.equal(a, b)
    # one more key per window (W + 1): the first query would reach a position
    # the ring has overwritten, so the segment is flagged and not attended
    a1, f1 = oracle.varlen(q, ring_k, ring_v, seg, seg_attr=[(1, W + 1, R)], scale=0.3,
                           return_flags=True)
    b1 = oracle.varlen(q, flat_k, flat_v, seg, seg_attr=[(1, W + 1, 0)], scale=0.3)
    assert f1 == oracle.SEGF_SPAN and torch.count_nonzero(a1) == 0
    assert torch.count_nonzero(b1) > 0


@pytest.mark.parametrize("causal,W,q_len,kv_end,R,stale", [
    (1, 6, 4, 23, 9, False),    # W + q_len - 1 = R: every visible key is held
    (1, 7, 4, 23, 9, True),     # one key more than the ring holds
    (1, 0, 1, 9, 9, False),     # no window, ring not yet wrapped
    (1, 0, 1, 10, 9, True),     # no window, wrapped: key 0 was overwritten
    (0, 6, 4, 23, 9, False),    # non-causal: the window is the lower bound only
    (0, 7, 4, 23, 9, True),
    (1, 6, 4, 7, 9, False),     # fewer keys than rows
    (1, 3, 0, 50, 9, False),    # no queries: nothing is read
    (1, 30, 2, 2, 9, False),    # window past position 0
])
def test_ring_span_flag_matches_the_simulated_ring(causal, W, q_len, kv_end, R, stale):
    """A ring segment is attended only when every key its queries see is still
    held by the ring (positions written in order, later ones overwriting the
    row of earlier ones); otherwise it is flagged SEGF_SPAN and its rows are 0.
    Expected answers come from the written-in-order simulation in brute.py and
    are checked against the hand-derived column above."""
    rows, cols, Hkv, D, Hq = 12, 2, 1, 4, 1
    ks, vs = _store(rows, cols, Hkv, D, 101)
    q = synth.randn_bf16((max(q_len, 1), Hq, D), 103)
    info, attr = [(0, q_len, 0, kv_end)], [(causal, W, R)]
    got, f = oracle.varlen(q, ks, vs, info, seg_attr=attr, scale=0.5, return_flags=True)
    found = []
    ref = brute.varlen(_lists(q), _lists(ks), _lists(vs), info, attr, 0.5, stale=found)
    assert bool(found) == stale
    assert f == (oracle.SEGF_SPAN if stale else 0)
    torch.testing.assert_close(got, torch.tensor(ref, dtype=torch.float64), rtol=1e-12,
                               atol=1e-12)
    # flat storage of the same rows never sets the flag
    _, f2 = oracle.varlen(q, ks, vs, [(0, q_len, 0, min(kv_end, rows))],
                          seg_attr=[(causal, W, 0)], scale=0.5, return_flags=True)
    assert f2 == 0


def test_varlen_segment_order_and_foreign_columns_do_not_matter():
    rows, cols, Hkv, D, Hq = 32, 5, 2, 8, 4
    ks, vs = _store(rows, cols, Hkv, D, 81)
    q = synth.randn_bf16((20, Hq, D), 83)
    info = [(0, 3, 2, 10), (5, 6, 0, 30), (12, 1, 3, 1), (14, 4, 1, 4)]
    attr = [(1, 0, 0), (0, 0, 0), (1, 0, 0), (1, 3, 7)]
    base = oracle.varlen(q, ks, vs, info, seg_attr=attr, scale=0.3)
    perm = [2, 0, 3, 1]
    out = oracle.varlen(q, ks, vs, [info[i] for i in perm], seg_attr=[attr[i] for i in perm],
                        scale=0.3)
    assert torch.equal(out, base)
    # NaN in the scratch column, in rows past every kv_end of flat segments
    ks2, vs2 = ks.clone(), vs.clone()
    ks2[:, cols - 1] = float("nan")
    vs2[:, cols - 1] = float("nan")
    ks2[30:, 0] = float("nan")
    vs2[10:, 2] = float("nan")
    out2 = oracle.varlen(q, ks2, vs2, info, seg_attr=attr, scale=0.3)
    assert torch.equal(out2, base)
    # uncovered packed rows are exact zeros
    for t in (3, 4, 11, 13, 18, 19):
        assert torch.count_nonzero(base[t]) == 0


def test_varlen_query_before_first_key_is_zero():
    rows, cols, Hkv, D, Hq = 16, 2, 1, 8, 1
    ks, vs = _store(rows, cols, Hkv, D, 91)
    q = synth.randn_bf16((4, Hq, D), 93)
    out = oracle.varlen(q, ks, vs, [(0, 4, 0, 2)], scale=0.3)  # positions -2, -1, 0, 1
    assert torch.count_nonzero(out[:2]) == 0
    assert torch.equal(out[2, 0], vs[0, 0, 0].double())


def test_varlen_invalid_segments_are_flagged_and_skipped():
    rows, cols, Hkv, D, Hq = 16, 3, 1, 8, 1
    ks, vs = _store(rows, cols, Hkv, D, 95)
    q = synth.randn_bf16((10, Hq, D), 97)
    cases = [
        ((0, 4, 2, 8), oracle.SEGF_COL),     # the scratch column
        ((0, 4, -1, 8), oracle.SEGF_COL),
        ((8, 4, 0, 8), oracle.SEGF_QRANGE),  # runs past T
        ((0, -1, 0, 8), oracle.SEGF_QRANGE),
        ((0, 4, 0, 17), oracle.SEGF_KVEND),  # flat storage holds 16 rows
        ((0, 4, 0, -3), oracle.SEGF_KVEND),
    ]
    for seg, flag in cases:
        out, f = oracle.varlen(q, ks, vs, [seg, (5, 2, 1, 6)], scale=0.3, return_flags=True)
        assert f == flag, (seg, f)
        assert torch.count_nonzero(out[:5]) == 0
        assert torch.count_nonzero(out[5:7]) > 0
    out, f = oracle.varlen(q, ks, vs, [(0, 4, 0, 8)], seg_attr=[(1, 0, 17)], scale=0.3,
                           return_flags=True)
    assert f == oracle.SEGF_ATTR and torch.count_nonzero(out) == 0
    with pytest.raises(oracle.OracleInvalid):
        oracle.varlen(q, ks, vs, [(0, 4, 0, 8), (3, 2, 1, 6)], scale=0.3)
    with pytest.raises(oracle.OracleInvalid):  # more segments than 2 x (cols - 1)
        oracle.varlen(q, ks, vs, [(i, 1, 0, 4) for i in range(5)], scale=0.3)


# ------------------------------------------------------------------ slot write

def _kv_step(T, rows, cols, Hkv, D, wid):
    ks = synth.randn_bf16((rows, cols, Hkv, D), 9000 + wid)
    vs = synth.randn_bf16((rows, cols, Hkv, D), 9100 + wid)
    kn = synth.randn_bf16((T, Hkv, D), 9200 + wid)
    vn = synth.randn_bf16((T, Hkv, D), 9300 + wid)
    return ks, vs, kn, vn


def test_kv_write_matches_index_copy_on_the_flattened_slots():
    """Distinct slots: the write is index_copy_ over the [rows*cols] slot axis
    with slot = (position mod rows) * cols + column."""
    rows, cols, Hkv, D = 40, 5, 2, 16
    ks, vs, kn, vn = _kv_step(12, rows, cols, Hkv, D, 1)
    pos = torch.tensor([0, 1, 2, 39, 40, 41, 7, 80, 5, 6, 119, 3], dtype=torch.int64)
    col = torch.tensor([0, 0, 0, 1, 1, 1, 2, 2, 3, 3, 4, 4], dtype=torch.int32)
    k2, v2, f = oracle.kv_write(ks, vs, kn, vn, pos, col)
    assert f == 0
    slots = (pos % rows) * cols + col.to(torch.int64)
    assert len(set(slots.tolist())) == len(slots)
    kr = ks.clone().view(rows * cols, Hkv, D).index_copy_(0, slots, kn).view_as(ks)
    vr = vs.clone().view(rows * cols, Hkv, D).index_copy_(0, slots, vn).view_as(vs)
    assert torch.equal(k2.view(torch.int16), kr.view(torch.int16))
    assert torch.equal(v2.view(torch.int16), vr.view(torch.int16))


def test_kv_write_ring_modulus_and_untouched_slots():
    """Per-token ring rows: position p lands at row p mod R; every other slot
    keeps its bits; gathering the written slots returns the new rows."""
    rows, cols, Hkv, D = 32, 4, 1, 8
    ks, vs, kn, vn = _kv_step(6, rows, cols, Hkv, D, 2)
    pos = torch.tensor([10, 11, 12, 25, 26, 31], dtype=torch.int64)
    col = torch.tensor([1, 1, 1, 2, 2, 3], dtype=torch.int32)
    R = torch.tensor([7, 7, 7, 0, 0, 32], dtype=torch.int32)
    k2, v2, f = oracle.kv_write(ks, vs, kn, vn, pos, col, slot_rows=R)
    assert f == 0
    expect_rows = [3, 4, 5, 25, 26, 31]
    touched = set()
    for i, r in enumerate(expect_rows):
        assert torch.equal(k2[r, col[i]], kn[i]) and torch.equal(v2[r, col[i]], vn[i])
        touched.add((r, int(col[i])))
    for r in range(rows):
        for c in range(cols):
            if (r, c) not in touched:
                assert torch.equal(k2[r, c], ks[r, c]) and torch.equal(v2[r, c], vs[r, c])


def test_kv_write_flags_and_skips_invalid_tokens():
    rows, cols, Hkv, D = 16, 3, 1, 8
    ks, vs, kn, vn = _kv_step(4, rows, cols, Hkv, D, 3)
    pos = torch.tensor([1, -1, 2, 3], dtype=torch.int64)
    col = torch.tensor([3, 0, -1, 1], dtype=torch.int32)
    R = torch.tensor([0, 0, 0, 17], dtype=torch.int32)
    k2, v2, f = oracle.kv_write(ks, vs, kn, vn, pos, col, slot_rows=R)
    assert f == oracle.KVF_COL | oracle.KVF_POS | oracle.KVF_ROWS
    assert torch.equal(k2.view(torch.int16), ks.view(torch.int16))
    assert torch.equal(v2.view(torch.int16), vs.view(torch.int16))


def test_kv_write_later_token_wins_a_shared_slot():
    rows, cols, Hkv, D = 8, 2, 1, 8
    ks, vs, kn, vn = _kv_step(3, rows, cols, Hkv, D, 4)
    pos = torch.tensor([2, 10, 18], dtype=torch.int64)   # all row 2
    col = torch.tensor([1, 1, 1], dtype=torch.int32)
    k2, v2, _ = oracle.kv_write(ks, vs, kn, vn, pos, col)
    assert torch.equal(k2[2, 1], kn[2]) and torch.equal(v2[2, 1], vn[2])


def test_kv_write_then_attend_reads_the_written_key():
    """Write convention = read convention: after a step writes position p of
    a sequence, a one-query segment that sees only key p (window 1) returns
    exactly the written V row, and a segment ending at p + 1 attends over the
    written key with the stored ones."""
    rows, cols, Hkv, D, Hq = 24, 3, 2, 16, 4
    ks, vs, kn, vn = _kv_step(2, rows, cols, Hkv, D, 5)
    R = 10
    pos = torch.tensor([23, 23], dtype=torch.int64)       # row 3 of a 10-row ring
    col = torch.tensor([0, 1], dtype=torch.int32)
    k2, v2, f = oracle.kv_write(ks, vs, kn, vn, pos, col,
                                slot_rows=torch.tensor([R, 0], dtype=torch.int32))
    assert f == 0
    q = synth.randn_bf16((2, Hq, D), 9400)
    info = torch.tensor([(0, 1, 0, 24), (1, 1, 1, 24)], dtype=torch.int32)
    attr = torch.tensor([(1, 1, R), (1, 1, 0)], dtype=torch.int32)   # window 1: only key 23
    out = oracle.varlen(q, k2, v2, info, seg_attr=attr)
    g = Hq // Hkv
    for t in range(2):
        for h in range(Hq):
            assert torch.equal(out[t, h], vn[t, h // g].double())
    # a causal segment with the widest window its ring holds (R keys) sees
    # the new key at its own position as well
    full = oracle.varlen(q[:1], k2, v2, info[:1], seg_attr=torch.tensor([(1, R, R)],
                                                                     dtype=torch.int32))
    stale = oracle.varlen(q[:1], ks, vs, info[:1], seg_attr=torch.tensor([(1, R, R)],
                                                                      dtype=torch.int32))
    assert torch.count_nonzero(full) > 0
    assert not torch.allclose(full, stale)


# ------------------------------------------------------- randomised brute force

from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as hst  # noqa: E402


@settings(max_examples=40, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow])
@given(Hkv=hst.integers(1, 2), g=hst.integers(1, 3), Lq=hst.integers(1, 7),
       Lkv=hst.integers(0, 9), q_pos0=hst.integers(-4, 10), window=hst.integers(0, 6),
       D=hst.sampled_from([2, 4, 8]), seed=hst.integers(0, 10 ** 6))
def test_prefill_vs_brute_random(Hkv, g, Lq, Lkv, q_pos0, window, D, seed):
    """Random tiny prefill shapes (GQA groups, rows before the first key,
    windows, no keys): the oracle equals the brute force to 1e-12."""
    Hq = Hkv * g
    q = synth.randn_bf16((1, Hq, Lq, D), seed)
    k = synth.randn_bf16((1, Hkv, Lkv, D), seed + 1)
    v = synth.randn_bf16((1, Hkv, Lkv, D), seed + 2)
    scale = 1.0 / math.sqrt(D)
    got = oracle.prefill(q, k, v, scale, q_pos0=q_pos0, window=window)
    ref = torch.tensor(brute.prefill(_lists(q), _lists(k), _lists(v), scale, q_pos0, window),
                       dtype=torch.float64).reshape(1, Hq, Lq, D)
    torch.testing.assert_close(got, ref, rtol=1e-12, atol=1e-12)


@settings(max_examples=40, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow])
@given(data=hst.data())
def test_varlen_vs_brute_random(data):
    """Random tiny tables of disjoint segments over a small store: causal or
    not, windows, ring moduli (wrapped or not), queries before the first key;
    the oracle equals the brute force to 1e-12, uncovered rows are zero, and
    exactly the segments that would read a position their ring no longer
    holds are flagged."""
    rows = data.draw(hst.integers(2, 10))
    cols = data.draw(hst.integers(2, 4))
    Hkv = data.draw(hst.integers(1, 2))
    Hq = Hkv * data.draw(hst.integers(1, 2))
    D = data.draw(hst.sampled_from([2, 4]))
    nseg = data.draw(hst.integers(0, 2 * (cols - 1)))
    info, attr, t = [], [], 0
    for _ in range(nseg):
        t += data.draw(hst.integers(0, 2))
        q_len = data.draw(hst.integers(0, 4))
        col = data.draw(hst.integers(0, cols - 2))
        causal = data.draw(hst.integers(0, 1))
        ring = data.draw(hst.integers(0, rows))  # 0: flat storage
        R = ring if ring > 0 else rows
        kv_end = data.draw(hst.integers(0, 3 * R if ring > 0 else rows))
        window = data.draw(hst.integers(0, 4))
        info.append((t, q_len, col, kv_end))
        attr.append((causal, window, ring))
        t += q_len
    T = max(1, t + data.draw(hst.integers(0, 2)))  # the brute force needs one packed row
    seed = data.draw(hst.integers(0, 10 ** 6))
    ks = synth.randn_bf16((rows, cols, Hkv, D), seed)
    vs = synth.randn_bf16((rows, cols, Hkv, D), seed + 1)
    q = synth.randn_bf16((T, Hq, D), seed + 2)
    scale = 0.5
    got, flags = oracle.varlen(q, ks, vs, info, seg_attr=attr or None, scale=scale,
                               return_flags=True)
    stale = []
    ref = brute.varlen(_lists(q), _lists(ks), _lists(vs), info, attr, scale, stale=stale)
    assert flags == (oracle.SEGF_SPAN if stale else 0)
    torch.testing.assert_close(got, torch.tensor(ref, dtype=torch.float64).reshape(T, Hq, D),
                               rtol=1e-12, atol=1e-12)
