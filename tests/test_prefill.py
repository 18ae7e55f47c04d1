"""Parity of attn_causal_prefill (HIP, through the C ABI) with the fp64 oracle."""
import math
import os

import pytest
import torch

import causal_gqa_prefill_flash_amd as attn
import oracle
from causal_gqa_prefill_flash_amd import synth
from gpu_util import compare, dev, sample_rows, say

pytestmark = pytest.mark.gpu


def _run(q, k, v, **kw):
    out = attn.causal_prefill(q.to(dev()), k.to(dev()), v.to(dev()), **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("B,Hq,Hkv,Lq,Lkv,D,q_pos0,window", [
    (1, 4, 1, 256, 256, 64, 0, 0),        # the tiny workload
    (2, 8, 2, 300, 1000, 64, None, 0),    # ragged Lq and Lkv, end-aligned
    (2, 8, 2, 300, 1000, 128, None, 0),
    (1, 16, 2, 77, 3001, 128, None, 0),
    (1, 6, 2, 130, 700, 64, None, 0),     # g = 3: rows of a block are 3 heads x 42 positions
    (1, 4, 4, 200, 333, 128, 0, 0),       # MHA (g = 1)
    (1, 16, 2, 300, 1000, 256, None, 0),  # D = 256: ragged, several q-blocks
    (2, 8, 2, 129, 700, 256, 0, 0),       # D = 256: queries from position 0
    (1, 8, 2, 200, 900, 256, None, 150),  # D = 256 with a window
    (1, 32, 1, 40, 500, 64, None, 0),     # g = 32
    (1, 300, 1, 3, 200, 64, None, 0),     # g = 300: head chunks of 256 and 44 rows
    (1, 600, 2, 2, 130, 128, None, 0),    # the same over two KV heads
    (1, 150, 1, 5, 300, 256, None, 0),    # D = 256, g = 150: chunks of 128 and 22
    (1, 8, 2, 257, 900, 128, None, 100),  # sliding window
    (1, 8, 2, 129, 129, 64, 0, 1),        # window of one key: returns V rows
    (1, 8, 2, 100, 400, 128, 37, 0),      # q_pos0 inside the prefix: late keys unseen
    (1, 8, 2, 64, 200, 64, -20, 0),       # 20 rows see nothing
    (1, 8, 2, 1, 5000, 128, None, 0),     # a single query row
    (1, 8, 2, 33, 0, 64, None, 0),        # no keys
    (1, 8, 2, 64, 200, 256, -20, 0),      # D = 256: 20 rows see nothing
    (1, 8, 2, 33, 0, 256, None, 0),       # D = 256: no keys
])
def test_prefill_matches_oracle(B, Hq, Hkv, Lq, Lkv, D, q_pos0, window):
    say("prefill", B, Hq, Hkv, Lq, Lkv, D, q_pos0, window)
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=20)
    scale = 1.0 / math.sqrt(D)
    if q_pos0 is None:
        q_pos0 = Lkv - Lq
    out = _run(q, k, v, scale=scale, q_pos0=q_pos0, window=window)
    ref = oracle.prefill(q, k, v, scale, q_pos0=q_pos0, window=window)
    compare(out, ref, "B%d Hq%d Hkv%d Lq%d Lkv%d D%d" % (B, Hq, Hkv, Lq, Lkv, D))
    if q_pos0 < 0:
        assert torch.count_nonzero(out[:, :, :-q_pos0]) == 0


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16])
def test_forced_splits_match_oracle(D, splits, monkeypatch):
    monkeypatch.setenv("ATTN_FORCE_SPLITS", str(splits))
    B, Hq, Hkv, Lq, Lkv = 1, 16, 2, 96, 4100
    say("forced splits", splits, "D", D)
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=21)
    out = _run(q, k, v)
    ref = oracle.prefill(q, k, v, 1.0 / math.sqrt(D))
    compare(out, ref, "splits %d D %d" % (splits, D))


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("Lkv", [1, 64, 65, 128, 191, 192, 250, 320, 449])
def test_key_tile_counts(D, Lkv, monkeypatch):
    """One split over 1..8 key tiles, ragged and exact: the key loop runs in
    steps of three tiles with one- and two-tile tails, and the last PV product
    reads the stage of the last tile."""
    monkeypatch.setenv("ATTN_FORCE_SPLITS", "1")
    B, Hq, Hkv, Lq = 1, 8, 2, 32
    say("key tiles", D, Lkv)
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=27)
    q_pos0 = Lkv - Lq
    out = _run(q, k, v, q_pos0=q_pos0)
    ref = oracle.prefill(q, k, v, 1.0 / math.sqrt(D), q_pos0=q_pos0)
    compare(out, ref, "D %d Lkv %d" % (D, Lkv))
    if q_pos0 < 0:
        assert torch.count_nonzero(out[:, :, :-q_pos0]) == 0


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.5])
def test_scale_sign_and_zero(scale):
    say("scale", scale)
    q, k, v = synth.prefill_inputs(1, 8, 2, 70, 300, 64, wid=22)
    out = _run(q, k, v, scale=scale)
    ref = oracle.prefill(q, k, v, scale)
    compare(out, ref, "scale %g" % scale)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("mult", [1.0, -1.0, 1.01, -2.0])
@pytest.mark.parametrize("splits", [1, 3])
def test_both_scale_paths(D, mult, splits, monkeypatch):
    """|scale| <= 1/sqrt(D) runs the kernel that carries the scale in Q and
    starts the scores from the negated references; a larger |scale| runs the
    one that keeps Q exact.  Both, with either sign, split or not, with a
    window and edge tiles, against the oracle."""
    monkeypatch.setenv("ATTN_FORCE_SPLITS", str(splits))
    scale = mult / math.sqrt(D)
    say("scale paths D=%d scale=%g splits=%d" % (D, scale, splits))
    q, k, v = synth.prefill_inputs(1, 8, 2, 150, 1300, D, wid=24)
    out = _run(q, k, v, scale=scale, window=700)
    ref = oracle.prefill(q, k, v, scale, window=700)
    compare(out, ref, "scale %g D %d splits %d" % (scale, D, splits))


def test_output_through_real_strides_and_canary():
    B, Hq, Hkv, Lq, Lkv, D = 2, 8, 2, 90, 600, 128
    say("strided outputs")
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=23)
    ref = oracle.prefill(q, k, v, 1.0 / math.sqrt(D))
    # BSHD storage viewed as BHSD
    bshd = torch.full((B, Lq, Hq, D), 7.0, dtype=torch.bfloat16, device=dev())
    attn.causal_prefill(q.to(dev()), k.to(dev()), v.to(dev()), out=bshd.transpose(1, 2))
    torch.cuda.synchronize()
    compare(bshd.transpose(1, 2), ref, "BSHD output")
    # padded L-stride: the padding must keep its canary
    pad = torch.full((B, Hq, Lq, D + 64), 3.0, dtype=torch.bfloat16, device=dev())
    attn.causal_prefill(q.to(dev()), k.to(dev()), v.to(dev()), out=pad[..., :D])
    torch.cuda.synchronize()
    compare(pad[..., :D], ref, "padded output")
    assert torch.all(pad[..., D:] == 3.0)
    # strided inputs: Q as a BSHD view, K/V with padded rows
    qb = q.transpose(1, 2).contiguous().to(dev()).transpose(1, 2)
    kp = torch.zeros(B, Hkv, Lkv, D + 8, dtype=torch.bfloat16)
    kp[..., :D] = k
    out = attn.causal_prefill(qb, kp.to(dev())[..., :D], v.to(dev()))
    torch.cuda.synchronize()
    compare(out, ref, "strided inputs")


def test_deterministic_and_masked_keys_do_not_matter():
    B, Hq, Hkv, Lq, Lkv, D = 1, 8, 2, 128, 2000, 128
    say("determinism / masked keys")
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=24)
    qd, kd, vd = q.to(dev()), k.to(dev()), v.to(dev())
    q_pos0 = 1000  # rows sit at 1000..1127: keys from 1128 on are never visible
    a = attn.causal_prefill(qd, kd, vd, q_pos0=q_pos0).clone()
    b = attn.causal_prefill(qd, kd, vd, q_pos0=q_pos0).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # NaN in keys no row can see
    k2, v2 = kd.clone(), vd.clone()
    k2[:, :, 1128:] = float("nan")
    v2[:, :, 1128:] = float("nan")
    c = attn.causal_prefill(qd, k2, v2, q_pos0=q_pos0)
    # finite changes to a key that only later rows of a block see
    k3, v3 = kd.clone(), vd.clone()
    k3[:, :, 1127] += 5.0
    v3[:, :, 1127] -= 3.0
    d = attn.causal_prefill(qd, k3, v3, q_pos0=q_pos0)
    torch.cuda.synchronize()
    assert torch.equal(c, a)
    assert torch.equal(d[:, :, :127], a[:, :, :127])
    assert not torch.equal(d[:, :, 127], a[:, :, 127])


# ------------------------------------------------------------- full-size workloads

FULL = ["d64_lq512_lkv16k", "d128_lq512_lkv16k", "d128_lq1k_lkv128k", "d128_lq1k_lkv128k_masked16",
        "d64_lq4k_lkv128k", "d128_lq4k_lkv128k", "d256_lq512_lkv16k", "d256_lq1k_lkv128k"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_on_sampled_rows(name):
    w = synth.PREFILL_WORKLOADS[name]
    B, Hq, Hkv, D, Lq, Lkv = w["B"], w["Hq"], w["Hkv"], w["D"], w["Lq"], w["Lkv"]
    q_pos0 = w["q_pos0"] if w["q_pos0"] is not None else Lkv - Lq
    say("full size", name)
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=w["wid"])
    out = _run(q, k, v, q_pos0=q_pos0)
    rows = sample_rows(Lq, head=24, tail=24, every=211)
    ref = oracle.prefill(q, k, v, 1.0 / math.sqrt(D), q_pos0=q_pos0, rows=rows)
    compare(out[:, :, rows], ref, name)
    if q_pos0 < 0:
        z = out[:, :, : -q_pos0]
        assert torch.count_nonzero(z) == 0 and torch.isfinite(out).all()


def test_full_size_strided_output():
    w = synth.PREFILL_WORKLOADS["d128_lq4k_lkv128k"]
    B, Hq, Hkv, D, Lq, Lkv = w["B"], w["Hq"], w["Hkv"], w["D"], w["Lq"], w["Lkv"]
    say("full size, BSHD output")
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=w["wid"])
    bshd = torch.empty((B, Lq, Hq, D), dtype=torch.bfloat16, device=dev())
    attn.causal_prefill(q.to(dev()), k.to(dev()), v.to(dev()), out=bshd.transpose(1, 2))
    torch.cuda.synchronize()
    rows = sample_rows(Lq, head=8, tail=8, every=509)
    ref = oracle.prefill(q, k, v, 1.0 / math.sqrt(D), rows=rows)
    compare(bshd.transpose(1, 2)[:, :, rows], ref, "BSHD full size")


# ------------------------------------------- the fixed-reference pass and its rerun

def _shifted_keys(k, q, scale, logit_of_key):
    """K with each key moved along the all-ones direction so that its logit
    against the mean query rises by logit_of_key[j] nats (q made positive, so
    the shift is the same sign for every row)."""
    qpos = q.abs()
    qsum = qpos.float().sum(-1).mean().item()
    shift = (logit_of_key / (scale * qsum)).view(1, 1, -1, 1)
    return qpos, (k.float() + shift).to(torch.bfloat16)


def _count_redone(fn):
    """(fn(), (attention workgroups, how many of them redid their key range
    with the exact running maximum)), from the profiling aid around fn."""
    attn.timing_begin()
    try:
        out = fn()
        torch.cuda.synchronize()
    finally:
        attn.timing_end()
    return out, attn.timing_reruns()


@pytest.mark.parametrize("B,Hq,Hkv,Lq,Lkv,D,q_pos0,window,wid", [
    (2, 16, 4, 59, 1262, 256, 1203, 370, 297),
    (2, 16, 2, 88, 763, 256, 146, 368, 394),
    (1, 16, 2, 178, 427, 256, 230, 0, 274),
    (1, 8, 2, 119, 1326, 128, 76, 0, 401),
])
def test_sharp_softmax_rounds_like_its_weights(B, Hq, Hkv, Lq, Lkv, D, q_pos0, window, wid):
    """Scale 0.2, 2.3-3.2 times the standard scale: logits with a standard
    deviation near 3, so a row's output is close to one V row.  With a fixed
    reference the largest weight is not 1 and its bf16 rounding would move
    such an output by up to 2^-9 of that V value on top of the output's own
    rounding (max-abs up to 2e-2 on these shapes); the kernels' row sums add
    the rounded weights there, which cancels it."""
    say("sharp softmax", B, Hq, Hkv, Lq, Lkv, D, q_pos0, window)
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=wid)
    out = _run(q, k, v, scale=0.2, q_pos0=q_pos0, window=window)
    ref = oracle.prefill(q, k, v, 0.2, q_pos0=q_pos0, window=window)
    compare(out, ref, "sharp softmax D=%d" % D)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("direction", ["rising", "falling"])
def test_logits_far_from_the_first_tile(D, direction):
    """Logits that rise along the keys by ~150 nats overflow the reference
    taken from the first tile unless it is refreshed (D = 128); at D = 64 and
    256 the workgroups redo the range exactly.  Falling logits stay on the
    fast pass with tiny P.  All match the oracle."""
    B, Hq, Hkv, Lq, Lkv = 1, 8, 2, 64, 2000
    say("logits", direction, "D", D)
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=25)
    scale = 1.0 / math.sqrt(D)
    ramp = torch.linspace(0.0, 150.0, Lkv)
    if direction == "falling":
        ramp = ramp.flip(0)
    q, k = _shifted_keys(k, q, scale, ramp)
    out = _run(q, k, v, scale=scale)
    ref = oracle.prefill(q, k, v, scale)
    compare(out, ref, "logits %s D %d" % (direction, D))


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("splits", [1, 3])
def test_rising_logits_refresh_the_reference(D, splits, monkeypatch):
    """Logits rising by 150 nats over 2000 keys (0.11 in log2 units per key):
    at D = 128 the periodic refresh of the fixed references keeps every sum
    in range, so no workgroup redoes its range; at D = 64 and 256, which have
    no refresh, some do.  Split or not, the output matches the oracle."""
    monkeypatch.setenv("ATTN_FORCE_SPLITS", str(splits))
    B, Hq, Hkv, Lq, Lkv = 1, 8, 2, 64, 2000
    say("refresh, D", D, "splits", splits)
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=28)
    scale = 1.0 / math.sqrt(D)
    q, k = _shifted_keys(k, q, scale, torch.linspace(0.0, 150.0, Lkv))
    out, (wg, redone) = _count_redone(lambda: _run(q, k, v, scale=scale))
    say("  workgroups", wg, "redone", redone)
    ref = oracle.prefill(q, k, v, scale)
    compare(out, ref, "refresh D %d splits %d" % (D, splits))
    assert wg > 0
    assert (redone > 0) == (D != 128)


@pytest.mark.parametrize("Hq", [8, 4])
@pytest.mark.parametrize("splits", [1, 2])
def test_rising_logits_in_a_window(Hq, splits, monkeypatch):
    """Logits rising 0.12 nats per key (84 nats over a 700-key window: sums
    far past 2^64 with a fixed reference) under a sliding window.  At g = 4
    every row of a q-block (64 positions) sees keys of its range's first
    tile, and the refresh keeps every sum in range: no workgroup reruns.  At
    g = 2 a q-block spans 128 positions, so some rows see nothing in that
    tile and keep the reference 0; their first visible logits (about 360 in
    log2 units) overflow P, and their workgroups redo the range with the
    exact running maximum.  Both match the oracle."""
    monkeypatch.setenv("ATTN_FORCE_SPLITS", str(splits))
    B, Hkv, Lq, Lkv, D, window = 1, 2, 192, 3000, 128, 700
    say("rising logits in a window, Hq", Hq, "splits", splits)
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=29)
    scale = 1.0 / math.sqrt(D)
    q, k = _shifted_keys(k, q, scale, torch.linspace(0.0, 0.12 * Lkv, Lkv))
    out, (wg, redone) = _count_redone(lambda: _run(q, k, v, scale=scale, window=window))
    say("  workgroups", wg, "redone", redone)
    ref = oracle.prefill(q, k, v, scale, window=window)
    compare(out, ref, "rising logits, window %d, Hq %d, splits %d" % (window, Hq, splits))
    assert wg > 0 and (redone > 0) == (Hq == 4)


@pytest.mark.parametrize("splits", [1, 3])
def test_rising_logits_with_splits(splits, monkeypatch):
    """Each split keeps its own reference; a split whose logits rise faster
    than the refresh follows (200 nats over its last 1000 keys) is redone
    exactly, and the merge combines both kinds of partials."""
    monkeypatch.setenv("ATTN_FORCE_SPLITS", str(splits))
    B, Hq, Hkv, Lq, Lkv, D = 1, 8, 2, 96, 3000, 128
    say("rising logits, splits", splits)
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=26)
    scale = 1.0 / math.sqrt(D)
    ramp = torch.zeros(Lkv)
    ramp[2000:] = torch.linspace(0.0, 200.0, Lkv - 2000)  # only the last split outgrows
    q, k = _shifted_keys(k, q, scale, ramp)
    out, (wg, redone) = _count_redone(lambda: _run(q, k, v, scale=scale))
    say("  workgroups", wg, "redone", redone)
    ref = oracle.prefill(q, k, v, scale)
    compare(out, ref, "rising logits, splits %d" % splits)
    assert 0 < redone < wg if splits > 1 else redone == wg


def test_windowed_rows_with_very_negative_logits():
    """Rows whose window starts past the first tile keep the reference 0; with
    every logit near -150 nats their sums underflow and the workgroup redoes
    the range exactly."""
    B, Hq, Hkv, Lq, Lkv, D = 1, 8, 2, 128, 1000, 64
    say("windowed, very negative logits")
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=27)
    scale = 1.0 / math.sqrt(D)
    q, k = _shifted_keys(k, q, scale, torch.full((Lkv,), -150.0))
    out = _run(q, k, v, scale=scale, window=64)
    ref = oracle.prefill(q, k, v, scale, window=64)
    compare(out, ref, "windowed negative logits")
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("shift", [-20, 20])
def test_split_partials_hold_any_magnitude(D, shift, monkeypatch):
    """Split partials are kept in fp16 with a per-row power-of-two scale: V
    scaled by 2^shift (beyond fp16's range either way) gives the unscaled
    result scaled by 2^shift, within the bar once scaled back, with five
    forced key splits."""
    monkeypatch.setenv("ATTN_FORCE_SPLITS", "5")
    B, Hq, Hkv, Lq, Lkv = 1, 8, 2, 150, 2500
    say("split partials, V x 2^%d, D %d" % (shift, D))
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=28)
    vs = (v.float() * 2.0 ** shift).to(torch.bfloat16)  # exact: a power of two
    out = _run(q, k, vs)
    ref = oracle.prefill(q, k, v, 1.0 / math.sqrt(D))
    compare(out.float() * 2.0 ** -shift, ref, "V x 2^%d D %d" % (shift, D))
