"""Parity of attn_causal_prefill_dev, the prefill with a device-resident
(q_pos0, kv_len) bound, with the oracle and with the host-bound call."""
import pytest
import torch

import causal_gqa_prefill_flash_amd as attn
import oracle
from causal_gqa_prefill_flash_amd import synth
from gpu_util import compare, dev, say

pytestmark = pytest.mark.gpu


def _bounds(q_pos0, kv_len):
    return torch.tensor([q_pos0, kv_len], dtype=torch.int64, device=dev())


@pytest.mark.parametrize("D", [64, 128, 256])
def test_device_bound_equal_to_the_host_bound_gives_the_same_bits(D):
    say("prefill dev bound == host bound, D", D)
    B, Hq, Hkv, Lq, Lkv = 1, 16, 2, 300, 5000
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=70)
    qd, kd, vd = q.to(dev()), k.to(dev()), v.to(dev())
    host = attn.causal_prefill(qd, kd, vd, q_pos0=Lkv - Lq)
    out, ws = attn.causal_prefill_dev(qd, kd, vd, _bounds(Lkv - Lq, Lkv))
    assert attn.prefill_read_error(ws) == 0
    assert torch.equal(out.view(torch.int16), host.view(torch.int16))
    compare(out, oracle.prefill(q, k, v, 1.0 / D ** 0.5, q_pos0=Lkv - Lq), "dev bound D%d" % D)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_chunked_prefill_replays_one_graph(D):
    """A 4096-key cache filled chunk by chunk: one captured graph, replayed
    for each 512-row chunk with the chunk's queries and (start, start + 512)
    written into the device buffers; keys past the bound are NaN."""
    say("chunked prefill graph, D", D)
    B, Hq, Hkv, Lq, cap = 1, 16, 2, 512, 4096
    _, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, cap, D, wid=71)
    kd, vd = k.to(dev()), v.to(dev())
    kd_nan, vd_nan = kd.clone(), vd.clone()
    qd = torch.zeros((B, Hq, Lq, D), dtype=torch.bfloat16, device=dev())
    bd = _bounds(0, Lq)
    out = torch.zeros_like(qd)
    ws = torch.empty(attn.prefill_dev_workspace_bytes(B, Hq, Hkv, Lq, cap, D), dtype=torch.uint8,
                     device=dev())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        attn.causal_prefill_dev(qd, kd_nan, vd_nan, bd, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        attn.causal_prefill_dev(qd, kd_nan, vd_nan, bd, out=out, workspace=ws)
    torch.cuda.synchronize()
    for c, start in enumerate(range(0, cap, Lq)):
        say("  chunk", c, "start", start)
        qc = synth.randn_bf16((B, Hq, Lq, D), 7300 + c)
        end = start + Lq
        # the cache holds the keys up to this chunk's end; later ones are NaN
        kd_nan.copy_(kd)
        vd_nan.copy_(vd)
        kd_nan[:, :, end:] = float("nan")
        vd_nan[:, :, end:] = float("nan")
        qd.copy_(qc)
        bd.copy_(torch.tensor([start, end], dtype=torch.int64))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert attn.prefill_read_error(ws) == 0
        ref = oracle.prefill(qc, k[:, :, :end], v[:, :, :end], 1.0 / D ** 0.5, q_pos0=start)
        compare(out, ref, "chunk %d" % c)


def test_out_of_range_bounds_are_clamped_and_flagged():
    say("prefill dev bound out of range")
    B, Hq, Hkv, Lq, cap, D = 1, 8, 2, 128, 1000, 128
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, cap, D, wid=72)
    qd, kd, vd = q.to(dev()), k.to(dev()), v.to(dev())
    scale = 1.0 / D ** 0.5
    out, ws = attn.causal_prefill_dev(qd, kd, vd, _bounds(900, cap + 77))
    assert attn.prefill_read_error(ws) == attn.BOUND_KV
    compare(out, oracle.prefill(q, k, v, scale, q_pos0=900), "kv_len above capacity")
    out, ws = attn.causal_prefill_dev(qd, kd, vd, _bounds(900, -5))
    assert attn.prefill_read_error(ws) == attn.BOUND_KV
    assert torch.count_nonzero(out) == 0
    out, ws = attn.causal_prefill_dev(qd, kd, vd, _bounds(-(1 << 63), cap))
    assert attn.prefill_read_error(ws) == attn.BOUND_QPOS
    assert torch.count_nonzero(out) == 0


def test_rows_before_the_first_key_and_a_short_bound():
    """q_pos0 = -40: the first 40 rows see nothing (zeros); kv_len = 300 of a
    2000-key capacity whose tail is NaN."""
    say("prefill dev bound: negative start, short bound")
    B, Hq, Hkv, Lq, cap, D = 1, 8, 2, 256, 2000, 64
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, cap, D, wid=73)
    kd, vd = k.to(dev()), v.to(dev())
    kd[:, :, 300:] = float("nan")
    vd[:, :, 300:] = float("nan")
    out, ws = attn.causal_prefill_dev(q.to(dev()), kd, vd, _bounds(-40, 300), window=100)
    assert attn.prefill_read_error(ws) == 0
    ref = oracle.prefill(q, k[:, :, :300], v[:, :, :300], 1.0 / D ** 0.5, q_pos0=-40, window=100)
    compare(out, ref, "negative start, window, short bound")
    assert torch.count_nonzero(out[:, :, :40]) == 0
