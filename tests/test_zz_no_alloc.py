"""attn_causal_prefill_noalloc (the entry point that allocates nothing)
against attn_causal_prefill, through the C ABI: the same bits, on two calls in
a row (the second smaller), both within the parity bar of the oracle; and a
call whose partials exceed the static buffer is refused."""
import ctypes
import math

import pytest
import torch

import causal_gqa_prefill_flash_amd as attn
import oracle
from causal_gqa_prefill_flash_amd import synth
from gpu_util import compare, dev, sample_rows, say

pytestmark = pytest.mark.gpu


def _s(t):
    return (ctypes.c_int64 * 4)(*t.stride())


def _noalloc(q, k, v, out, q_pos0):
    B, Hq, Lq, D = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    st = attn.lib().attn_causal_prefill_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
        ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(out.data_ptr()), B, Hq, Hkv, Lq, Lkv, D,
        1.0 / math.sqrt(D), _s(q), _s(k), _s(v), _s(out), q_pos0, 0,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


@pytest.mark.parametrize("case", [
    # (B, Hq, Hkv, Lq, Lkv, D): a split launch with ~34 MB of partials, then a
    # smaller one that reuses the start of the same buffer
    [(1, 16, 2, 512, 16384, 128), (1, 16, 2, 96, 4100, 64)],
])
def test_noalloc_matches_the_workspace_entry_point(case):
    for n, (B, Hq, Hkv, Lq, Lkv, D) in enumerate(case):
        say("noalloc call", n, dict(B=B, Hq=Hq, Hkv=Hkv, Lq=Lq, Lkv=Lkv, D=D))
        need = attn.prefill_workspace_bytes(B, Hq, Hkv, Lq, Lkv, D)
        assert 0 < need <= attn.NOALLOC_SCRATCH_BYTES  # the buffer is really used
        q, k, v = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=700 + n)
        qd, kd, vd = q.to(dev()), k.to(dev()), v.to(dev())
        ref_out = attn.causal_prefill(qd, kd, vd)
        out = torch.full_like(qd, float("nan"))
        torch.cuda.synchronize()
        assert _noalloc(qd, kd, vd, out, Lkv - Lq) == attn.ATTN_OK, attn.last_error()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        rows = sample_rows(Lq, head=16, tail=16, every=61)
        ref = oracle.prefill(q, k, v, 1.0 / math.sqrt(D), rows=rows)
        compare(out[:, :, rows], ref, "noalloc call %d" % n)


def test_noalloc_refuses_partials_larger_than_the_buffer(monkeypatch):
    """Sixteen forced key splits of the long-context D=128 chunk need ~136 MB
    of partials: refused before any launch, with the reason.  The tensors are
    real and full size all the same."""
    monkeypatch.setenv("ATTN_FORCE_SPLITS", "16")
    B, Hq, Hkv, Lq, Lkv, D = 1, 16, 2, 1024, 131072, 128
    need = attn.prefill_workspace_bytes(B, Hq, Hkv, Lq, Lkv, D)
    say("noalloc refusal, partials", need)
    assert need > attn.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, Hq, Lq, D), dtype=torch.bfloat16, device=dev())
    k = torch.zeros((B, Hkv, Lkv, D), dtype=torch.bfloat16, device=dev())
    out = torch.full_like(q, 7.0)
    assert _noalloc(q, k, k, out, Lkv - Lq) == attn.ATTN_ERR_WORKSPACE
    assert "static scratch buffer" in attn.last_error()
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())  # nothing was launched
