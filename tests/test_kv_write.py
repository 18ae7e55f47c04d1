"""Parity of attn_kv_write (HIP, through the C ABI) with the oracle: a pure
copy, so bit-exact; and the write followed by attn_sdpa_varlen, eagerly and
as one captured graph, against the oracle's write then attention."""
import pytest
import torch

import causal_gqa_prefill_flash_amd as attn
import oracle
from causal_gqa_prefill_flash_amd import synth
from gpu_util import compare, dev, say

pytestmark = pytest.mark.gpu


def _bits_equal(a, b):
    return torch.equal(a.detach().cpu().view(torch.int16), b.detach().cpu().view(torch.int16))


def _step_tokens(info, attr):
    """The tokens of a step: every packed row of every segment, at position
    kv_end - q_len + j of its column, with the segment's ring rows."""
    pos, col, srows, rows_t = [], [], [], []
    for s in range(info.shape[0]):
        q_start, q_len, c, kv_end = (int(x) for x in info[s])
        for j in range(q_len):
            rows_t.append(q_start + j)
            pos.append(kv_end - q_len + j)
            col.append(c)
            srows.append(int(attr[s][2]))
    return (torch.tensor(pos, dtype=torch.int64), torch.tensor(col, dtype=torch.int32),
            torch.tensor(srows, dtype=torch.int32), torch.tensor(rows_t, dtype=torch.int64))


def _run(ks, vs, kn, vn, pos, col, srows=None):
    kd, vd = ks.to(dev()), vs.to(dev())
    ws = attn.kv_write(kn.to(dev()), vn.to(dev()), kd, vd, pos.to(dev()), col.to(dev()),
                       srows.to(dev()) if srows is not None else None)
    err = attn.kv_write_read_error(ws, kn.shape[0])
    return kd.cpu(), vd.cpu(), err


@pytest.mark.parametrize("D", [64, 128, 256])
def test_pinned_step_write_is_bit_exact(D):
    """The pinned table's 1686 step tokens (flat and ring columns)."""
    say("kv_write pinned step D", D)
    st = synth.VARLEN_STORE
    info, attr, T = synth.pinned_varlen_table()
    pos, col, srows, _ = _step_tokens(info, attr)
    n = pos.shape[0]
    ks = synth.randn_bf16((st["rows"], st["cols"], st["Hkv"], D), 8100)
    vs = synth.randn_bf16((st["rows"], st["cols"], st["Hkv"], D), 8101)
    kn = synth.randn_bf16((n, st["Hkv"], D), 8102)
    vn = synth.randn_bf16((n, st["Hkv"], D), 8103)
    kd, vd, err = _run(ks, vs, kn, vn, pos, col, srows)
    kr, vr, flags = oracle.kv_write(ks, vs, kn, vn, pos, col, srows)
    assert err == flags == 0
    assert _bits_equal(kd, kr) and _bits_equal(vd, vr)


def test_strided_new_rows_from_a_packed_qkv_buffer():
    """K and V of the step as views into a packed [T, Hq + 2 Hkv, D] buffer,
    into a padded store (row stride larger than cols x Hkv x D)."""
    say("kv_write strided views")
    T, Hq, Hkv, D, rows, cols = 37, 8, 2, 128, 300, 5
    qkv = synth.randn_bf16((T, Hq + 2 * Hkv, D), 8200)
    kn, vn = qkv[:, Hq:Hq + Hkv], qkv[:, Hq + Hkv:]
    big_k = synth.randn_bf16((rows, cols + 1, Hkv, D + 64), 8201)
    big_v = synth.randn_bf16((rows, cols + 1, Hkv, D + 64), 8202)
    g = torch.Generator().manual_seed(8203)
    pos = torch.randperm(rows * 3, generator=g)[:T].to(torch.int64)
    col = torch.randint(0, cols, (T,), generator=g, dtype=torch.int32)
    # distinct slots
    slots = set()
    keep = []
    for i in range(T):
        key = (int(pos[i]) % rows, int(col[i]))
        if key not in slots:
            slots.add(key)
            keep.append(i)
    keep = torch.tensor(keep)
    qkv = qkv[keep].contiguous()
    kn, vn, pos, col = qkv[:, Hq:Hq + Hkv], qkv[:, Hq + Hkv:], pos[keep], col[keep]
    kd, vd = big_k.to(dev()), big_v.to(dev())
    ksv, vsv = kd[:, :cols, :, :D], vd[:, :cols, :, :D]
    qkv_d = qkv.to(dev())
    kvd, vvd = qkv_d[:, Hq:Hq + Hkv], qkv_d[:, Hq + Hkv:]
    assert not kvd.is_contiguous() and kvd.stride(0) == (Hq + 2 * Hkv) * D
    ws = attn.kv_write(kvd, vvd, ksv, vsv, pos.to(dev()), col.to(dev()))
    assert attn.kv_write_read_error(ws, kn.shape[0]) == 0
    kr, vr, _ = oracle.kv_write(big_k[:, :cols, :, :D], big_v[:, :cols, :, :D], kn, vn, pos, col)
    assert _bits_equal(ksv, kr) and _bits_equal(vsv, vr)
    # the padding and the extra column are untouched
    assert _bits_equal(kd[:, :, :, D:], big_k[:, :, :, D:])
    assert _bits_equal(kd[:, cols:], big_k[:, cols:])


def test_invalid_tokens_are_flagged_and_skipped():
    say("kv_write invalid tokens")
    rows, cols, Hkv, D = 64, 4, 2, 64
    ks = synth.randn_bf16((rows, cols, Hkv, D), 8300)
    vs = synth.randn_bf16((rows, cols, Hkv, D), 8301)
    kn = synth.randn_bf16((9, Hkv, D), 8302)
    vn = synth.randn_bf16((9, Hkv, D), 8303)
    pos = torch.tensor([5, -3, 6, 7, 8, 100, 9, 10, 11], dtype=torch.int64)
    col = torch.tensor([0, 0, 4, -1, 1, 1, 2, 2, 3], dtype=torch.int32)
    srows = torch.tensor([0, 0, 0, 0, 65, 20, 0, 0, 0], dtype=torch.int32)
    kd, vd, err = _run(ks, vs, kn, vn, pos, col, srows)
    kr, vr, flags = oracle.kv_write(ks, vs, kn, vn, pos, col, srows)
    assert err == flags == (attn.KV_COL | attn.KV_POS | attn.KV_ROWS)
    assert _bits_equal(kd, kr) and _bits_equal(vd, vr)


def test_padded_writes_to_the_scratch_column_keep_one_of_them():
    """Padded tokens of a static-width step all go to the scratch column at
    one position: the slot holds one of their rows, every other slot is the
    oracle's."""
    say("kv_write scratch column")
    rows, cols, Hkv, D = 128, 3, 2, 128
    ks = synth.randn_bf16((rows, cols, Hkv, D), 8400)
    vs = synth.randn_bf16((rows, cols, Hkv, D), 8401)
    kn = synth.randn_bf16((12, Hkv, D), 8402)
    vn = synth.randn_bf16((12, Hkv, D), 8403)
    pos = torch.tensor([3, 4, 5, 6, 9, 10] + [0] * 6, dtype=torch.int64)
    col = torch.tensor([0, 0, 0, 0, 1, 1] + [cols - 1] * 6, dtype=torch.int32)
    kd, vd, err = _run(ks, vs, kn, vn, pos, col)
    kr, vr, _ = oracle.kv_write(ks, vs, kn, vn, pos, col)
    assert err == 0
    assert _bits_equal(kd[:, :cols - 1], kr[:, :cols - 1])
    assert _bits_equal(kd[1:], kr[1:]) and _bits_equal(vd[1:], vr[1:])
    cand = [i for i in range(6, 12)]
    assert any(_bits_equal(kd[0, cols - 1], kn[i]) and _bits_equal(vd[0, cols - 1], vn[i])
               for i in cand)


def test_large_step_sampled():
    """A 16384-token prefill-sized step into a 65536-row store: bit-exact on
    the whole store (a copy is cheap to compare)."""
    say("kv_write 16384 tokens")
    T, rows, cols, Hkv, D = 16384, 65536, 3, 2, 128
    ks = torch.zeros((rows, cols, Hkv, D), dtype=torch.bfloat16)
    vs = torch.zeros((rows, cols, Hkv, D), dtype=torch.bfloat16)
    kn = synth.randn_bf16((T, Hkv, D), 8500)
    vn = synth.randn_bf16((T, Hkv, D), 8501)
    pos = torch.arange(T, dtype=torch.int64) + 40000
    col = torch.full((T,), 1, dtype=torch.int32)
    kd, vd, err = _run(ks, vs, kn, vn, pos, col)
    assert err == 0
    assert _bits_equal(kd[40000:40000 + T, 1], kn) and _bits_equal(vd[40000:40000 + T, 1], vn)
    assert torch.count_nonzero(kd[:40000]) == 0 and torch.count_nonzero(kd[:, 0]) == 0


def _pinned_step_inputs(wid):
    st = synth.VARLEN_STORE
    info, attr, T = synth.pinned_varlen_table()
    pos, col, srows, rows_t = _step_tokens(info, attr)
    q, ks, vs = synth.varlen_inputs(T, st["rows"], st["cols"], st["Hkv"], st["D"], st["Hq"],
                                    wid=wid)
    n = pos.shape[0]
    kn = synth.randn_bf16((n, st["Hkv"], st["D"]), 8600 + wid)
    vn = synth.randn_bf16((n, st["Hkv"], st["D"]), 8700 + wid)
    return info, attr, T, pos, col, srows, q, ks, vs, kn, vn


def test_write_then_attend_matches_the_oracle():
    """One decode/prefill step: write the step's K/V, then attend over the
    store; the oracle does the same two steps."""
    say("kv_write + varlen step")
    info, attr, T, pos, col, srows, q, ks, vs, kn, vn = _pinned_step_inputs(61)
    kd, vd = ks.to(dev()), vs.to(dev())
    ws = attn.kv_write(kn.to(dev()), vn.to(dev()), kd, vd, pos.to(dev()), col.to(dev()),
                       srows.to(dev()))
    out, vws = attn.sdpa_varlen(q.to(dev()), kd, vd, info.to(dev()), seg_attr=attr.to(dev()))
    assert attn.kv_write_read_error(ws, pos.shape[0]) == 0
    assert attn.varlen_read_error(vws, info.shape[0], T) == 0
    k2, v2, _ = oracle.kv_write(ks, vs, kn, vn, pos, col, srows)
    ref = oracle.varlen(q, k2, v2, info, seg_attr=attr)
    compare(out, ref, "write then attend")


def test_write_and_attend_in_one_graph():
    """The write and the attention captured as one graph; replays with new
    step rows, positions and tables written into the same buffers match the
    oracle, and the store accumulates the writes of every replay."""
    say("kv_write + varlen graph")
    st = synth.VARLEN_STORE
    info0, attr0, T, pos0, col0, srows0, q0, ks, vs, kn0, vn0 = _pinned_step_inputs(62)
    n = pos0.shape[0]
    S = info0.shape[0]
    kd, vd = ks.to(dev()), vs.to(dev())
    qd = q0.to(dev())
    knd, vnd = kn0.to(dev()), vn0.to(dev())
    posd, cold, srd = pos0.to(dev()), col0.to(dev()), srows0.to(dev())
    si, sa = info0.to(dev()), attr0.to(dev())
    out = torch.zeros((T, st["Hq"], st["D"]), dtype=torch.bfloat16, device=dev())
    kws = torch.empty(attn.kv_write_workspace_bytes(n), dtype=torch.uint8, device=dev())
    vws = torch.empty(attn.varlen_workspace_bytes(S, T, st["Hq"], st["Hkv"], st["D"], st["rows"],
                                                  st["cols"]), dtype=torch.uint8, device=dev())
    scratch_k, scratch_v = kd.clone(), vd.clone()  # warm-up writes go to a copy

    def step(kst, vst):
        attn.kv_write(knd, vnd, kst, vst, posd, cold, srd, workspace=kws)
        attn.sdpa_varlen(qd, kst, vst, si, seg_attr=sa, out=out, workspace=vws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(scratch_k, scratch_v)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(kd, vd)
    torch.cuda.synchronize()

    k_ref, v_ref = ks.clone(), vs.clone()
    gen = torch.Generator().manual_seed(8800)
    for rep in range(3):
        say("graph replay", rep)
        # the next step: the same table advanced by 0, 1, 2 positions per segment
        info = info0.clone()
        info[:, 3] = torch.clamp(info0[:, 3] + rep, max=st["rows"])
        pos, col, srows, _ = _step_tokens(info, attr0)
        kn = synth.randn_bf16((n, st["Hkv"], st["D"]), 8900 + rep)
        vn = synth.randn_bf16((n, st["Hkv"], st["D"]), 8950 + rep)
        qn = synth.randn_bf16(tuple(q0.shape), 8990 + rep)
        si.copy_(info)
        posd.copy_(pos)
        cold.copy_(col)
        srd.copy_(srows)
        knd.copy_(kn)
        vnd.copy_(vn)
        qd.copy_(qn)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert attn.kv_write_read_error(kws, n) == 0
        assert attn.varlen_read_error(vws, S, T) == 0
        k_ref, v_ref, _ = oracle.kv_write(k_ref, v_ref, kn, vn, pos, col, srows)
        ref = oracle.varlen(qn, k_ref, v_ref, info, seg_attr=attr0)
        compare(out, ref, "graph replay %d" % rep)
        assert _bits_equal(kd, k_ref) and _bits_equal(vd, v_ref)
    del gen
