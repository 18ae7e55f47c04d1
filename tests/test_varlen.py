"""Parity of attn_sdpa_varlen (HIP, through the C ABI) with the fp64 oracle."""
import math

import pytest
import torch

import causal_gqa_prefill_flash_amd as attn
import oracle
from causal_gqa_prefill_flash_amd import synth
from gpu_util import compare, dev, say

pytestmark = pytest.mark.gpu


def _gpu_varlen(q, ks, vs, seq_info, seg_attr=None, canary=float("nan"), **kw):
    out = torch.full(q.shape, canary, dtype=torch.bfloat16, device=dev())
    sa = seg_attr.to(dev()) if seg_attr is not None else None
    si = seq_info.to(dev())
    out, ws = attn.sdpa_varlen(q.to(dev()), ks.to(dev()), vs.to(dev()), si, seg_attr=sa,
                               out=out, **kw)
    err = attn.varlen_read_error(ws, si.shape[0], q.shape[0])
    return out, err


def test_pinned_table_matches_oracle():
    say("varlen pinned table")
    st = synth.VARLEN_STORE
    info, attr, T = synth.pinned_varlen_table()
    q, ks, vs = synth.varlen_inputs(T, st["rows"], st["cols"], st["Hkv"], st["D"], st["Hq"])
    out, err = _gpu_varlen(q, ks, vs, info, attr)
    ref, flags = oracle.varlen(q, ks, vs, info, seg_attr=attr, return_flags=True)
    assert err == flags == 0
    compare(out, ref, "pinned table")
    covered = torch.zeros(T, dtype=torch.bool)
    for s in range(info.shape[0]):
        covered[info[s, 0]: info[s, 0] + info[s, 1]] = True
    assert int((~covered).sum()) == 41
    assert torch.count_nonzero(out[(~covered).to(dev())]) == 0


@pytest.mark.parametrize("seed", range(5001, 5011))
def test_seeded_tables_match_oracle(seed):
    say("varlen seeded table", seed)
    st = synth.VARLEN_STORE
    info, attr, T = synth.random_varlen_table(seed)
    q, ks, vs = synth.varlen_inputs(T, st["rows"], st["cols"], st["Hkv"], st["D"], st["Hq"],
                                    wid=seed)
    out, err = _gpu_varlen(q, ks, vs, info, attr)
    ref = oracle.varlen(q, ks, vs, info, seg_attr=attr)
    assert err == 0
    compare(out, ref, "seed %d" % seed)


@pytest.mark.parametrize("Hq,Hkv,D,seed", [(4, 4, 128, 5101), (6, 2, 64, 5102), (32, 1, 128, 5103),
                                             (40, 8, 64, 5104)])
def test_gqa_ratios_match_oracle(Hq, Hkv, D, seed):
    """Seeded tables at other query heads per KV head (g = 1, 3, 32, 5): the
    q-block holds 256 / g positions of g heads (85 positions at g = 3), and
    a segment takes the decode items while q_len * g <= 32."""
    say("varlen GQA ratio", Hq, Hkv, D, seed)
    info, attr, T = synth.random_varlen_table(seed)
    q, ks, vs = synth.varlen_inputs(T, 8192, 9, Hkv, D, Hq, wid=seed)
    out, err = _gpu_varlen(q, ks, vs, info, attr)
    ref = oracle.varlen(q, ks, vs, info, seg_attr=attr)
    assert err == 0
    compare(out, ref, "Hq %d Hkv %d D %d seed %d" % (Hq, Hkv, D, seed))


@pytest.mark.parametrize("Hq,Hkv,D", [(300, 1, 64), (600, 2, 128)])
def test_head_chunks_match_oracle(Hq, Hkv, D):
    """g = 300 query heads per KV head: more than the 256 rows of a q-block,
    so each q-block holds one position of 256 heads and a second head chunk
    holds the other 44 (a partly filled row block)."""
    say("varlen head chunks", Hq, Hkv, D)
    rows, cols = 2048, 4
    info = torch.tensor([(0, 5, 0, 700), (6, 1, 1, 1500), (8, 3, 2, 64)], dtype=torch.int32)
    attr = torch.tensor([(1, 0, 0), (1, 256, 0), (0, 0, 0)], dtype=torch.int32)
    T = 11
    q, ks, vs = synth.varlen_inputs(T, rows, cols, Hkv, D, Hq, wid=5106)
    out, err = _gpu_varlen(q, ks, vs, info, attr)
    ref = oracle.varlen(q, ks, vs, info, seg_attr=attr)
    assert err == 0
    compare(out, ref, "head chunks Hq %d Hkv %d D %d" % (Hq, Hkv, D))


@pytest.mark.parametrize("D", [64, 128])
def test_short_query_steps_split_keys(D):
    """Every segment a decode-like step over a full column (the split path)."""
    say("varlen short steps D", D)
    rows, cols, Hkv, Hq = 8192, 9, 2, 16
    qlens = [1, 4, 16, 1, 4, 16, 1, 16]
    info, t = [], 0
    for s, ql in enumerate(qlens):
        info.append((t, ql, s, 8192 - 37 * s))
        t += ql + 1
    T = t
    info = torch.tensor(info, dtype=torch.int32)
    q, ks, vs = synth.varlen_inputs(T, rows, cols, Hkv, D, Hq, wid=40)
    out, err = _gpu_varlen(q, ks, vs, info)
    ref = oracle.varlen(q, ks, vs, info)
    assert err == 0
    compare(out, ref, "short steps D%d" % D)


@pytest.mark.parametrize("split_keys,cap", [(64, None), (200, None), (64, 3), (100000, None)])
def test_split_sizes_match_oracle(split_keys, cap, monkeypatch):
    """Every q-block splits its visible keys into chunks of about split_keys
    (at most 16, or the cap); any split size merges to the oracle."""
    monkeypatch.setenv("ATTN_VARLEN_SPLIT_KEYS", str(split_keys))
    if cap is not None:
        monkeypatch.setenv("ATTN_FORCE_SPLITS", str(cap))
    say("varlen split keys", split_keys, "cap", cap)
    st = synth.VARLEN_STORE
    info, attr, T = synth.pinned_varlen_table()
    q, ks, vs = synth.varlen_inputs(T, st["rows"], st["cols"], st["Hkv"], st["D"], st["Hq"],
                                    wid=46)
    out, err = _gpu_varlen(q, ks, vs, info, attr)
    ref = oracle.varlen(q, ks, vs, info, seg_attr=attr)
    assert err == 0
    compare(out, ref, "split keys %d cap %s" % (split_keys, cap))


@pytest.mark.parametrize("D", [64, 128])
def test_long_segment_rising_logits_split(D):
    """Logits that rise by ~200 nats over the last keys of a long segment make
    the later splits of each q-block redo their ranges exactly; the merge takes
    fast-pass and exact partials together."""
    say("varlen long segment, rising logits, D", D)
    rows, cols, Hkv, Hq = 4096, 3, 2, 16
    q_len, kv_end = 200, 4000
    q, ks, vs = synth.varlen_inputs(q_len + 8, rows, cols, Hkv, D, Hq, wid=47)
    scale = 1.0 / math.sqrt(D)
    q = q.abs()
    qsum = q.float().sum(-1).mean().item()
    ramp = torch.zeros(rows)
    ramp[2500:kv_end] = torch.linspace(0.0, 200.0, kv_end - 2500)
    ks = (ks.float() + (ramp / (scale * qsum)).view(rows, 1, 1, 1)).to(torch.bfloat16)
    info = torch.tensor([(4, q_len, 1, kv_end)], dtype=torch.int32)
    out, err = _gpu_varlen(q, ks, vs, info, scale=scale)
    ref = oracle.varlen(q, ks, vs, info, scale=scale)
    assert err == 0
    compare(out, ref, "long segment rising logits D%d" % D)
    assert torch.count_nonzero(out[:4]) == 0 and torch.count_nonzero(out[4 + q_len:]) == 0


@pytest.mark.parametrize("D,Hq", [(128, 16), (64, 16), (128, 8)])
def test_decode_items_of_every_row_count(D, Hq):
    """Segments of 1..128 rows (q_len x g) run as decode items with 1, 2 or 4
    row blocks per key stream; flat, ring and windowed, next to one another."""
    say("varlen decode rows D", D, "Hq", Hq)
    rows, cols, Hkv = 8192, 9, 2
    g = Hq // Hkv
    qlens = [1, 3, 4, 5, 8, 12, 16, 128 // g]
    info, attr, t = [], [], 0
    for s, ql in enumerate(qlens):
        kv_end = 8192 - 301 * s if s % 3 else 6000 + 77 * s
        ring = 2559 if s % 4 == 3 else 0
        window = 2048 if ring else (700 if s == 5 else 0)
        info.append((t, ql, s, kv_end))
        attr.append((1, window, ring))
        t += ql + 2
    T = t + 3
    info = torch.tensor(info, dtype=torch.int32)
    attr = torch.tensor(attr, dtype=torch.int32)
    q, ks, vs = synth.varlen_inputs(T, rows, cols, Hkv, D, Hq, wid=48)
    out, err = _gpu_varlen(q, ks, vs, info, attr)
    ref = oracle.varlen(q, ks, vs, info, seg_attr=attr)
    assert err == 0
    compare(out, ref, "decode rows D%d Hq%d" % (D, Hq))


def test_two_segments_of_one_sequence():
    """A sequence's owner rows (causal) and its draft block (non-causal) as
    two segments over the same column, next to other sequences (up to
    2 x (cols - 1) segments)."""
    say("varlen two segments per sequence")
    rows, cols, Hkv, D, Hq = 4096, 3, 2, 128, 16
    info = torch.tensor([(0, 4, 1, 1000), (6, 16, 1, 1016), (24, 40, 0, 500), (70, 1, 0, 501)],
                        dtype=torch.int32)
    attr = torch.tensor([(1, 0, 0), (0, 0, 0), (1, 0, 0), (1, 0, 0)], dtype=torch.int32)
    q, ks, vs = synth.varlen_inputs(72, rows, cols, Hkv, D, Hq, wid=49)
    out, err = _gpu_varlen(q, ks, vs, info, attr)
    ref, flags = oracle.varlen(q, ks, vs, info, seg_attr=attr, return_flags=True)
    assert err == flags == 0
    compare(out, ref, "two segments per sequence")


@pytest.mark.parametrize("S", [64, 65, 150])
def test_tables_past_64_segments(S):
    """Up to 64 segments each wave of the attention kernel and of the finish
    pass plans the table on its own (a lane per segment); past that both go
    through LDS.  Tables of 64, 65 and 150 segments (decode rows, 256-row
    blocks, split and unsplit keys, rings, an invalid segment, gaps) match
    the oracle either way."""
    import random
    rng = random.Random(7000 + S)
    rows, Hkv, D, Hq = 1536, 2, 64, 8
    cols = S // 2 + 2
    info, attr, t = [], [], 0
    for s in range(S):
        t += rng.randint(0, 2)
        q_len = rng.choice([1, 2, 3, 5, 40])
        col = s // 2
        ring = rng.choice([0, 0, 0, 700])
        kv_end = rng.randint(q_len, rows if not ring else 2 * ring)
        window = ring - q_len + 1 if ring else rng.choice([0, 0, 100])
        info.append((t, q_len, col, kv_end))
        attr.append((1, window, ring))
        t += q_len
    info[S // 3] = (info[S // 3][0], info[S // 3][1], cols - 1, 5)  # the scratch column: invalid
    T = t + 3
    say("varlen table of", S, "segments, T", T)
    info = torch.tensor(info, dtype=torch.int32)
    attr = torch.tensor(attr, dtype=torch.int32)
    q, ks, vs = synth.varlen_inputs(T, rows, cols, Hkv, D, Hq, wid=70 + S)
    out, err = _gpu_varlen(q, ks, vs, info, attr)
    ref, flags = oracle.varlen(q, ks, vs, info, seg_attr=attr, return_flags=True)
    assert err == flags == attn.SEG_COL
    compare(out, ref, "%d segments" % S)


@pytest.mark.parametrize("q_len,kv_end", [(2048, 8192), (4096, 8192), (300, 6000)])
def test_long_segments_take_longer_splits(q_len, kv_end):
    """The split size is chosen per table on the device: a segment with many
    q-blocks takes longer key splits so that its items fit the launch (2048
    rows of 8192 keys at g = 2: 1728-key splits; 4096 rows: 3888-key ones, on
    a launch of 256 workgroups), and a decode segment beside it takes the
    same; a short segment keeps 512-key splits.  All match the oracle."""
    rows, cols, Hkv, D, Hq = 8192, 3, 2, 64, 4
    say("varlen long segment", q_len, kv_end)
    info = torch.tensor([(0, q_len, 0, kv_end), (q_len + 2, 1, 1, 8000)], dtype=torch.int32)
    T = q_len + 3
    q, ks, vs = synth.varlen_inputs(T, rows, cols, Hkv, D, Hq, wid=80)
    out, err = _gpu_varlen(q, ks, vs, info)
    assert err == 0
    ref = oracle.varlen(q, ks, vs, info)
    compare(out, ref, "long segment %d x %d" % (q_len, kv_end))


def test_single_segment_equals_prefill_on_the_column_view():
    say("varlen vs prefill on a strided column")
    rows, cols, Hkv, D, Hq = 4096, 5, 2, 128, 16
    q_len, kv_end, col = 200, 3333, 2
    q, ks, vs = synth.varlen_inputs(q_len, rows, cols, Hkv, D, Hq, wid=41)
    info = torch.tensor([(0, q_len, col, kv_end)], dtype=torch.int32)
    out, err = _gpu_varlen(q, ks, vs, info)
    assert err == 0
    kd, vd, qd = ks.to(dev()), vs.to(dev()), q.to(dev())
    kcol = kd[:kv_end, col].permute(1, 0, 2).unsqueeze(0)
    vcol = vd[:kv_end, col].permute(1, 0, 2).unsqueeze(0)
    pre = attn.causal_prefill(qd.permute(1, 0, 2).unsqueeze(0), kcol, vcol,
                              q_pos0=kv_end - q_len)
    torch.cuda.synchronize()
    ref = oracle.varlen(q, ks, vs, info)
    compare(out, ref, "varlen single segment")
    compare(pre[0].permute(1, 0, 2), ref, "prefill on the column view")


def test_unread_storage_does_not_matter():
    """NaN in the scratch column, other columns, rows past kv_end and stale
    ring rows leaves every output bit unchanged."""
    say("varlen unread storage")
    st = synth.VARLEN_STORE
    info, attr, T = synth.pinned_varlen_table()
    q, ks, vs = synth.varlen_inputs(T, st["rows"], st["cols"], st["Hkv"], st["D"], st["Hq"])
    base, _ = _gpu_varlen(q, ks, vs, info, attr)
    ks2, vs2 = ks.clone(), vs.clone()
    nan = float("nan")
    ks2[:, st["cols"] - 1] = nan            # scratch column
    vs2[:, st["cols"] - 1] = nan
    ks2[700:, 0] = nan                      # s1 (col 0) holds 700 keys
    vs2[3000:, 1] = nan                     # s3 (col 1) holds 3000 keys
    ks2[64:, 5] = nan                       # s2 (col 5) holds 64 keys
    ks2[2559:, 4] = nan                     # ring column of s6: rows past the ring
    vs2[2559:, 4] = nan
    ks2[2000:, 6] = nan                     # s7's ring (col 6) holds positions 0..1999
    ks2[:, 8] = nan
    out, err = _gpu_varlen(q, ks2, vs2, info, attr)
    assert err == 0
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))


def test_invalid_segments_are_flagged_and_zeroed():
    say("varlen invalid segments")
    rows, cols, Hkv, D, Hq = 1024, 4, 2, 64, 8
    T = 64
    q, ks, vs = synth.varlen_inputs(T, rows, cols, Hkv, D, Hq, wid=42)
    info = torch.tensor([(0, 8, 3, 100),      # scratch column
                         (8, 8, 0, 2000),     # more keys than flat rows
                         (60, 8, 1, 100),     # runs past T
                         (20, 10, 2, 500),    # valid
                         (40, 4, 1, 64)],     # valid
                        dtype=torch.int32)
    out, err = _gpu_varlen(q, ks, vs, info)
    ref, flags = oracle.varlen(q, ks, vs, info, return_flags=True)
    assert err == flags == (attn.SEG_COL | attn.SEG_KVEND | attn.SEG_QRANGE)
    compare(out, ref, "invalid segments")
    assert torch.count_nonzero(out[:20]) == 0


def test_overlapping_segments_are_flagged():
    say("varlen overlap flag")
    rows, cols, Hkv, D, Hq = 256, 3, 1, 64, 4
    q, ks, vs = synth.varlen_inputs(16, rows, cols, Hkv, D, Hq, wid=43)
    info = torch.tensor([(0, 8, 0, 100), (4, 8, 1, 100)], dtype=torch.int32)
    _, err = _gpu_varlen(q, ks, vs, info)
    assert err & attn.SEG_OVERLAP


def test_empty_table_zeroes_every_row():
    say("varlen empty table")
    rows, cols, Hkv, D, Hq = 64, 2, 1, 128, 2
    q, ks, vs = synth.varlen_inputs(9, rows, cols, Hkv, D, Hq, wid=44)
    info = torch.zeros((0, 4), dtype=torch.int32)
    out, err = _gpu_varlen(q, ks, vs, info)
    assert err == 0 and torch.count_nonzero(out) == 0


def test_call_level_modes_without_seg_attr():
    say("varlen call-level ring/window")
    rows, cols, Hkv, D, Hq = 600, 4, 2, 64, 8
    q, ks, vs = synth.varlen_inputs(80, rows, cols, Hkv, D, Hq, wid=45)
    info = torch.tensor([(0, 30, 0, 1500), (35, 1, 2, 900), (40, 33, 1, 33)], dtype=torch.int32)
    out, err = _gpu_varlen(q, ks, vs, info, causal=1, window=200, ring_rows=300)
    ref = oracle.varlen(q, ks, vs, info, causal=1, window=200, ring_rows=300)
    assert err == 0
    compare(out, ref, "call-level ring")
    out2, _ = _gpu_varlen(q, ks, vs, info, causal=0)
    ref2 = oracle.varlen(q, ks, vs, info, causal=0)
    compare(out2, ref2, "call-level non-causal")


@pytest.mark.parametrize("D", [64, 128])
def test_small_rings_wrap_inside_a_tile(D):
    """Ring storage of fewer rows than a 64-key tile (5, 37, 63) and around it
    (64, 65): one tile's keys wrap the ring several times; compute-path and
    decode-path segments, each with the widest window its ring holds
    (R - q_len + 1 keys)."""
    say("varlen small rings D=%d" % D)
    rows, cols, Hkv, Hq = 200, 6, 2, 8
    info = torch.tensor([(0, 20, 0, 300), (24, 3, 1, 500), (30, 10, 2, 129),
                         (45, 8, 3, 1000), (60, 2, 4, 777)], dtype=torch.int32)
    attr = torch.tensor([(1, 18, 37), (1, 3, 5), (1, 54, 63), (1, 57, 64), (1, 64, 65)],
                        dtype=torch.int32)
    q, ks, vs = synth.varlen_inputs(70, rows, cols, Hkv, D, Hq, wid=46)
    out, err = _gpu_varlen(q, ks, vs, info, attr)
    ref, flags = oracle.varlen(q, ks, vs, info, seg_attr=attr, return_flags=True)
    assert err == flags == 0
    compare(out, ref, "small rings")


@pytest.mark.parametrize("D", [64, 128])
def test_ring_segments_past_their_span_are_flagged(D):
    """Ring segments whose queries would see a position the ring has
    overwritten (no window with kv_end > R; a window wider than R - q_len + 1;
    the same on a non-causal segment) are flagged ATTN_SEG_SPAN and zeroed,
    next to valid ring and flat segments that are attended."""
    say("varlen ring span flag D", D)
    rows, cols, Hkv, Hq = 3000, 8, 2, 16
    info = torch.tensor([(0, 16, 0, 5000),   # ring 2559, no window: stale
                         (20, 512, 1, 8000), # window 2049 + 512 - 1 > 2559: stale
                         (540, 4, 2, 6000),  # non-causal, window 2557: stale
                         (550, 512, 3, 8000),  # window 2048: exactly the ring
                         (1070, 16, 4, 2500),  # ring not yet wrapped, no window
                         (1090, 33, 5, 2900)],  # flat
                        dtype=torch.int32)
    attr = torch.tensor([(1, 0, 2559), (1, 2049, 2559), (0, 2557, 2559), (1, 2048, 2559),
                         (1, 0, 2559), (1, 0, 0)], dtype=torch.int32)
    T = 1130
    q, ks, vs = synth.varlen_inputs(T, rows, cols, Hkv, D, Hq, wid=51)
    out, err = _gpu_varlen(q, ks, vs, info, attr)
    ref, flags = oracle.varlen(q, ks, vs, info, seg_attr=attr, return_flags=True)
    assert err == flags == attn.SEG_SPAN
    compare(out, ref, "ring span D%d" % D)
    assert torch.count_nonzero(out[:544]) == 0
    assert torch.count_nonzero(out[550:1062]) > 0


@pytest.mark.parametrize("shift", [-20, 20])
def test_split_partials_hold_any_magnitude(shift):
    """Varlen split partials (compute and decode items) are fp16 with a
    per-row power-of-two scale: V scaled by 2^shift, beyond fp16's range
    either way, gives the unscaled result scaled by 2^shift."""
    say("varlen split partials, V x 2^%d" % shift)
    rows, cols, Hkv, D, Hq = 8192, 5, 2, 128, 16
    info = torch.tensor([(0, 1, 0, 8192), (3, 4, 1, 6000), (10, 16, 2, 7000), (30, 64, 3, 5000)],
                        dtype=torch.int32)
    q, ks, vs = synth.varlen_inputs(96, rows, cols, Hkv, D, Hq, wid=52)
    vsc = (vs.float() * 2.0 ** shift).to(torch.bfloat16)  # exact: a power of two
    out, err = _gpu_varlen(q, ks, vsc, info)
    ref = oracle.varlen(q, ks, vs, info)
    assert err == 0
    compare(out.float() * 2.0 ** -shift, ref, "varlen V x 2^%d" % shift)
