"""Large sizes: a 2M-key prefix (key indices and tile counts far past the
benchmark shapes), element offsets past 2^31 through the output strides, and
a million-row varlen store; each checked against the oracle on sampled rows."""
import math

import pytest
import torch

import causal_gqa_prefill_flash_amd as attn
import oracle
from causal_gqa_prefill_flash_amd import synth
from gpu_util import compare, dev, say

pytestmark = pytest.mark.gpu


def test_two_million_keys():
    B, Hq, Hkv, Lq, Lkv, D = 1, 8, 1, 64, 1 << 21, 64
    say("prefill over 2M keys")
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=400)
    out = attn.causal_prefill(q.to(dev()), k.to(dev()), v.to(dev()))
    rows = [0, 31, 63]
    ref = oracle.prefill(q, k, v, 1.0 / math.sqrt(D), rows=rows)
    compare(out[:, :, rows], ref, "2M keys")


def test_output_offsets_past_two_to_the_31():
    """The second batch of the output starts 2^31 + 1024 elements into its
    buffer; every address of it needs 64-bit arithmetic."""
    B, Hq, Hkv, Lq, Lkv, D = 2, 4, 2, 96, 700, 128
    say("output offsets past 2^31")
    q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=401)
    bstride = (1 << 31) + 1024
    buf = torch.empty(bstride + Hq * Lq * D, dtype=torch.bfloat16, device=dev())
    out = buf.as_strided((B, Hq, Lq, D), (bstride, Lq * D, D, 1))
    out.fill_(float("nan"))
    attn.causal_prefill(q.to(dev()), k.to(dev()), v.to(dev()), out=out)
    ref = oracle.prefill(q, k, v, 1.0 / math.sqrt(D))
    compare(out, ref, "offsets past 2^31")
    del buf


def test_million_row_store():
    """A varlen store of 2^20 rows: a decode step and a 100-row chunk at the
    end of a million-key column, a ring column, against the oracle."""
    rows, cols, Hkv, D, Hq = 1 << 20, 3, 1, 64, 8
    say("varlen over 2^20 rows")
    info = torch.tensor([(0, 1, 0, rows), (2, 100, 1, rows - 5)], dtype=torch.int32)
    attr = torch.tensor([(1, 0, 0), (1, 4096, 8191)], dtype=torch.int32)
    q, ks, vs = synth.varlen_inputs(110, rows, cols, Hkv, D, Hq, wid=402)
    out, ws = attn.sdpa_varlen(q.to(dev()), ks.to(dev()), vs.to(dev()), info.to(dev()),
                               seg_attr=attr.to(dev()))
    assert attn.varlen_read_error(ws, 2, 110) == 0
    ref = oracle.varlen(q, ks, vs, info, seg_attr=attr)
    compare(out, ref, "million-row store")
