"""One captured graph of attn_sdpa_varlen serves any lengths written into the
same seq_info buffer: launch geometry never depends on its contents."""
import pytest
import torch

import causal_gqa_prefill_flash_amd as attn
import oracle
from causal_gqa_prefill_flash_amd import synth
from gpu_util import compare, dev, say

pytestmark = pytest.mark.gpu


def test_graph_replays_with_new_tables():
    st = synth.VARLEN_STORE
    T = 4200
    q, ks, vs = synth.varlen_inputs(T, st["rows"], st["cols"], st["Hkv"], st["D"], st["Hq"],
                                    wid=50)
    qd, kd, vd = q.to(dev()), ks.to(dev()), vs.to(dev())
    S = 8
    si = torch.zeros((S, 4), dtype=torch.int32, device=dev())
    sa = torch.zeros((S, 3), dtype=torch.int32, device=dev())
    out = torch.zeros((T, st["Hq"], st["D"]), dtype=torch.bfloat16, device=dev())
    need = attn.varlen_workspace_bytes(S, T, st["Hq"], st["Hkv"], st["D"], st["rows"], st["cols"])
    ws = torch.empty(need, dtype=torch.uint8, device=dev())

    tables = [synth.pinned_varlen_table()[:2]]
    for seed in (6001, 6002, 6003):
        info, attr, Tn = synth.random_varlen_table(seed)
        assert Tn <= T
        tables.append((info, attr))

    si.copy_(tables[0][0])
    sa.copy_(tables[0][1])
    torch.cuda.synchronize()
    say("graph: warm-up and capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        attn.sdpa_varlen(qd, kd, vd, si, seg_attr=sa, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        attn.sdpa_varlen(qd, kd, vd, si, seg_attr=sa, out=out, workspace=ws)
    torch.cuda.synchronize()

    for rep in range(2):
        for n, (info, attr) in enumerate(tables):
            say("graph replay", rep, "table", n)
            si.copy_(info)
            sa.copy_(attr)
            out.fill_(float("nan"))  # every row must be rewritten by the replay
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert attn.varlen_read_error(ws, S, T) == 0
            ref = oracle.varlen(q, ks, vs, info, seg_attr=attr, T=T)
            compare(out, ref, "replay %d table %d" % (rep, n))
            # the eager call on the same buffers gives the same bits
            eager = torch.empty_like(out)
            attn.sdpa_varlen(qd, kd, vd, si, seg_attr=sa, out=eager)
            torch.cuda.synchronize()
            assert torch.equal(eager.view(torch.int16), out.view(torch.int16))
