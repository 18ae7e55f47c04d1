"""The C ABI on the CPU: the library loads, exports what include/attn.h
declares, and validates its arguments before touching the GPU.

No call here reaches a kernel: every case is rejected by host validation
(or is a no-op), so these run without a GPU.  Where a case is INVALID for
the library it must also be rejected by the oracle: both apply the same
written rules, each with its own code.
"""
import ctypes
import os
import re

import pytest
import torch

import causal_gqa_prefill_flash_amd as attn
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

A = 0x10000  # a 16-byte aligned fake device address; never dereferenced here


def _lib():
    if not os.path.exists(attn.LIB_PATH):
        from causal_gqa_prefill_flash_amd import build
        build.build()
    return attn.lib()


def _s(*v):
    return (ctypes.c_int64 * len(v))(*v)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = _lib()
    names = declared_functions()
    assert len(names) == 18, names
    for n in names:
        assert hasattr(L, n), n
    assert L.attn_abi_version() == 1


def test_library_exports_nothing_else():
    """Only the declared entry points have external linkage."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm is not installed")
    _lib()
    out = subprocess.run([nm, "-D", "--defined-only", attn.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    funcs = sorted(ln.split()[-1] for ln in out.splitlines() if " T " in ln)
    assert funcs == declared_functions(), funcs


def _prefill(q=A, k=A, v=A, out=A, B=1, Hq=4, Hkv=2, Lq=8, Lkv=16, D=64, scale=0.125,
             qs=None, ks=None, vs=None, os_=None, q_pos0=8, window=0):
    L = _lib()
    qs = qs or _s(Hq * Lq * D, Lq * D, D, 1)
    ks = ks or _s(Hkv * Lkv * D, Lkv * D, D, 1)
    vs = vs or _s(Hkv * Lkv * D, Lkv * D, D, 1)
    os_ = os_ or _s(Hq * Lq * D, Lq * D, D, 1)
    return L.attn_causal_prefill(q, k, v, out, B, Hq, Hkv, Lq, Lkv, D, scale, qs, ks, vs, os_,
                                 q_pos0, window, None, 0, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), attn.ATTN_ERR_INVALID),
    (dict(out=None), attn.ATTN_ERR_INVALID),
    (dict(B=0), attn.ATTN_ERR_INVALID),
    (dict(Hq=0), attn.ATTN_ERR_INVALID),
    (dict(Lq=-1), attn.ATTN_ERR_INVALID),
    (dict(Lkv=-5), attn.ATTN_ERR_INVALID),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_INVALID),
    (dict(scale=float("nan")), attn.ATTN_ERR_INVALID),
    (dict(scale=float("inf")), attn.ATTN_ERR_INVALID),
    (dict(D=96), attn.ATTN_ERR_UNSUPPORTED),
    (dict(D=512), attn.ATTN_ERR_UNSUPPORTED),
    (dict(qs=_s(4 * 8 * 64, 8 * 64, 64, 2)), attn.ATTN_ERR_UNSUPPORTED),   # inner stride
    (dict(ks=_s(2 * 16 * 64, 16 * 64, 68, 1)), attn.ATTN_ERR_UNSUPPORTED),  # row not 16 B
    (dict(vs=_s(2 * 16 * 64, -16 * 64, 64, 1)), attn.ATTN_ERR_UNSUPPORTED),  # negative
    (dict(ks=_s(2 * 16 << 24, 16 << 24, 1 << 24, 1)), attn.ATTN_ERR_UNSUPPORTED),  # row 2^24
    (dict(vs=_s(2 * 16 << 25, 16 << 25, 1 << 25, 1)), attn.ATTN_ERR_UNSUPPORTED),
    (dict(out=A + 8), attn.ATTN_ERR_UNSUPPORTED),                           # misaligned
    (dict(k=A + 2), attn.ATTN_ERR_UNSUPPORTED),
])
def test_prefill_validation(kw, code):
    assert _prefill(**kw) == code
    assert attn.last_error() != ""


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), attn.ATTN_ERR_INVALID),
    (dict(B=0), attn.ATTN_ERR_INVALID),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_INVALID),
    (dict(D=96), attn.ATTN_ERR_UNSUPPORTED),
    (dict(qs=_s(4 * 8 * 64, 8 * 64, 64, 2)), attn.ATTN_ERR_UNSUPPORTED),
    (dict(out=A + 8), attn.ATTN_ERR_UNSUPPORTED),
    (dict(Lq=0), attn.ATTN_OK),
])
def test_prefill_noalloc_validates_like_prefill(kw, code):
    """The allocation-free entry point runs the same host validation before
    any HIP call (and Lq == 0 enqueues nothing)."""
    L = _lib()
    a = dict(q=A, k=A, v=A, out=A, B=1, Hq=4, Hkv=2, Lq=8, Lkv=16, D=64)
    a.update({n: kw[n] for n in a if n in kw})
    Hq, Hkv, Lq, Lkv, D = a["Hq"], a["Hkv"], a["Lq"], a["Lkv"], a["D"]
    qs = kw.get("qs") or _s(Hq * Lq * D, Lq * D, D, 1)
    ks = _s(Hkv * Lkv * D, Lkv * D, D, 1)
    rc = L.attn_causal_prefill_noalloc(a["q"], a["k"], a["v"], a["out"], a["B"], Hq, Hkv, Lq,
                                       Lkv, D, 0.125, qs, ks, ks, qs, Lkv - Lq, 0, None)
    assert rc == code, attn.last_error()
    assert "ATTN_NOALLOC_SCRATCH_BYTES (64u << 20)" in open(HEADER).read()
    assert attn.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_error_messages_are_per_thread():
    """attn_last_error is thread-local: threads that fail validation in
    different ways, and one whose calls succeed, each read back their own
    result while the others run (ctypes drops the GIL inside the calls)."""
    import threading
    _lib()
    cases = [(dict(D=96), attn.ATTN_ERR_UNSUPPORTED, "head dim 96"),
             (dict(B=0), attn.ATTN_ERR_INVALID, "sizes must satisfy"),
             (dict(Lq=0), attn.ATTN_OK, "")]
    bad = []

    def run(kw, code, msg):
        for _ in range(3000):
            rc = _prefill(**kw)
            err = attn.last_error()
            if rc != code or (msg not in err if msg else err != ""):
                bad.append((kw, rc, err))
                return

    threads = [threading.Thread(target=run, args=c) for c in cases for _ in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not bad, bad[:3]


def test_prefill_empty_query_is_a_noop():
    assert _prefill(Lq=0) == attn.ATTN_OK
    assert attn.last_error() == ""
    # empty tensors may arrive as null pointers
    assert _prefill(Lq=0, q=None, out=None) == attn.ATTN_OK
    assert _prefill(Lkv=0, k=None, v=None, Lq=0) == attn.ATTN_OK
    assert _prefill(Lkv=8, k=None) == attn.ATTN_ERR_INVALID


@pytest.mark.parametrize("kw", [dict(B=0), dict(Lq=-1), dict(Hq=6, Hkv=4), dict(Lkv=-5)])
def test_oracle_rejects_what_the_library_calls_invalid(kw):
    assert _prefill(**kw) == attn.ATTN_ERR_INVALID
    L = oracle._load()
    B, Hq, Hkv, Lq, Lkv, D = (kw.get(n, d) for n, d in
                              (("B", 1), ("Hq", 4), ("Hkv", 2), ("Lq", 8), ("Lkv", 16), ("D", 64)))
    buf = torch.zeros(1 << 16, dtype=torch.int16).numpy()
    out = torch.zeros(1 << 16, dtype=torch.float64).numpy()
    st = (ctypes.c_int64 * 4)(64, 64, 64, 1)
    p = buf.ctypes.data_as(ctypes.c_void_p)
    rc = L.oracle_prefill(p, p, p, out.ctypes.data_as(ctypes.c_void_p), B, Hq, Hkv, Lq, Lkv, D,
                          0.1, st, st, st, 0, 0, None, 0, None)
    assert rc == 1


def _varlen(S=2, T=16, Hq=4, Hkv=2, D=64, rows=32, cols=3, causal=1, window=0, ring_rows=0,
            seq_info=A, seg_attr=None, ws=A, ws_bytes=None, q=A, qs=None, ks=None):
    L = _lib()
    if ws_bytes is None:
        ws_bytes = L.attn_sdpa_varlen_workspace(max(S, 0), max(T, 0), Hq, max(Hkv, 1), D,
                                                max(rows, 1), max(cols, 2)) or 1 << 20
    qs = qs or _s(Hq * D, D, 1)
    ks = ks or _s(cols * Hkv * D, Hkv * D, D, 1)
    return L.attn_sdpa_varlen(q, A, A, A, seq_info, S, seg_attr, T, Hq, Hkv, D, rows, cols,
                              0.125, causal, window, ring_rows, qs, ks, ks, _s(Hq * D, D, 1),
                              ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), attn.ATTN_ERR_INVALID),
    (dict(seq_info=None), attn.ATTN_ERR_INVALID),
    (dict(S=-1), attn.ATTN_ERR_INVALID),
    (dict(T=-1), attn.ATTN_ERR_INVALID),
    (dict(cols=1), attn.ATTN_ERR_INVALID),
    (dict(rows=0), attn.ATTN_ERR_INVALID),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_INVALID),
    (dict(S=5, cols=3), attn.ATTN_ERR_INVALID),          # > 2 x (cols - 1)
    (dict(ring_rows=33), attn.ATTN_ERR_INVALID),         # ring larger than the store
    (dict(causal=0, window=4), attn.ATTN_ERR_INVALID),   # window without causality
    (dict(D=32), attn.ATTN_ERR_UNSUPPORTED),
    (dict(D=256), attn.ATTN_ERR_UNSUPPORTED),            # varlen: 64 and 128 only
    (dict(qs=_s(4 * 64, 64, 2)), attn.ATTN_ERR_UNSUPPORTED),
    (dict(ks=_s(3 * 2 * 64, 2 * 64, 60, 1)), attn.ATTN_ERR_UNSUPPORTED),
    (dict(ws=None), attn.ATTN_ERR_WORKSPACE),
    (dict(ws_bytes=16), attn.ATTN_ERR_WORKSPACE),
    (dict(ws=A + 64), attn.ATTN_ERR_WORKSPACE),          # not 256-byte aligned
])
def test_varlen_validation(kw, code):
    assert _varlen(**kw) == code
    assert attn.last_error() != ""


@pytest.mark.parametrize("kw", [dict(S=5, cols=3), dict(ring_rows=33), dict(causal=0, window=4),
                                dict(cols=1)])
def test_oracle_rejects_what_the_library_calls_invalid_varlen(kw):
    assert _varlen(**kw) == attn.ATTN_ERR_INVALID
    S = kw.get("S", 2)
    cols = kw.get("cols", 3)
    rows = 32
    q = torch.zeros(16, 4, 64, dtype=torch.bfloat16)
    st = torch.zeros(rows, max(cols, 1), 2, 64, dtype=torch.bfloat16)
    info = [(2 * i, 1, 0, 4) for i in range(S)]
    with pytest.raises(oracle.OracleInvalid):
        oracle.varlen(q, st, st, info, causal=kw.get("causal", 1), window=kw.get("window", 0),
                      ring_rows=kw.get("ring_rows", 0))


def test_varlen_workspace_follows_rows_and_packed_rows():
    """Error words for T rows, then split partials per packed row: nsplit =
    min(16, ceil(rows / 512)) splits of D fp16 values and a 4-float record for
    each of Hq heads."""
    L = _lib()

    def al(n):
        return (n + 255) // 256 * 256

    def expect(T, Hq, D, rows):
        ns = min(16, (rows + 511) // 512)
        part = al(T * Hq * ns * D * 2) + al(T * Hq * ns * 4 * 4) if ns > 1 else 0
        return al(max(T, 1) * 4) + part

    a = L.attn_sdpa_varlen_workspace(8, 1727, 16, 2, 128, 8192, 9)
    assert a == expect(1727, 16, 128, 8192) and a % 256 == 0
    assert L.attn_sdpa_varlen_workspace(16, 1727, 16, 2, 128, 8192, 17) == a  # not S
    assert L.attn_sdpa_varlen_workspace(8, 4000, 16, 2, 128, 8192, 9) == expect(4000, 16, 128, 8192)
    assert L.attn_sdpa_varlen_workspace(8, 1727, 16, 2, 64, 3000, 9) == expect(1727, 16, 64, 3000)
    assert L.attn_sdpa_varlen_workspace(8, 100, 8, 2, 64, 512, 9) == expect(100, 8, 64, 512)
    assert L.attn_sdpa_varlen_workspace(8, 1727, 16, 2, 96, 8192, 9) == 0


def test_binding_refuses_cpu_tensors():
    q = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attn.causal_prefill(q, q[:, :1], q[:, :1])


def test_binding_checks_out_shapes_before_any_call():
    """A too-small out would let a kernel write past it, so every entry point
    checks it against q (prefill [B,Hq,Lq,D], varlen [T,Hq,D])."""
    q = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    kv = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    small = torch.zeros(1, 2, 3, 64, dtype=torch.bfloat16)
    bounds = torch.zeros(2, dtype=torch.int64)
    with pytest.raises(ValueError, match="out has shape"):
        attn.causal_prefill(q, kv, kv, out=small)
    with pytest.raises(ValueError, match="out has shape"):
        attn.causal_prefill_dev(q, kv, kv, bounds, out=small)
    qv = torch.zeros(10, 4, 64, dtype=torch.bfloat16)
    store = torch.zeros(16, 3, 2, 64, dtype=torch.bfloat16)
    info = torch.zeros(1, 4, dtype=torch.int32)
    with pytest.raises(ValueError, match="out has shape"):
        attn.sdpa_varlen(qv, store, store, info, out=torch.zeros(9, 4, 64, dtype=torch.bfloat16))


def test_binding_checks_that_every_tensor_is_on_one_device():
    q = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    kv = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    meta = torch.empty(1, 1, 8, 64, dtype=torch.bfloat16, device="meta")
    with pytest.raises(ValueError, match="one device"):
        attn.causal_prefill(q, kv, meta)
    with pytest.raises(ValueError, match="one device"):
        attn.causal_prefill_dev(q, kv, kv, torch.zeros(2, dtype=torch.int64, device="meta"))
    qv = torch.zeros(10, 4, 64, dtype=torch.bfloat16)
    store = torch.zeros(16, 3, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="one device"):
        attn.sdpa_varlen(qv, store, store, torch.zeros(1, 4, dtype=torch.int32, device="meta"))
    with pytest.raises(ValueError, match="one device"):
        attn.kv_write(torch.zeros(2, 2, 64, dtype=torch.bfloat16),
                      torch.zeros(2, 2, 64, dtype=torch.bfloat16), store, store,
                      torch.zeros(2, dtype=torch.int64, device="meta"),
                      torch.zeros(2, dtype=torch.int32))


def test_span_flag_bits_match_the_oracle():
    assert (attn.SEG_QRANGE, attn.SEG_COL, attn.SEG_KVEND, attn.SEG_ATTR, attn.SEG_OVERLAP,
            attn.SEG_SPAN) == (oracle.SEGF_QRANGE, oracle.SEGF_COL, oracle.SEGF_KVEND,
                               oracle.SEGF_ATTR, oracle.SEGF_OVERLAP, oracle.SEGF_SPAN)


def test_binding_fails_loudly_without_the_library(monkeypatch):
    monkeypatch.setattr(attn, "_lib", None)
    monkeypatch.setattr(attn, "LIB_PATH", "/nonexistent/libattn.so")
    with pytest.raises(ImportError):
        attn.lib()


def test_timing_end_rejects_null_outputs_and_counts_nothing_when_idle():
    L = _lib()
    assert L.attn_timing_begin() == attn.ATTN_OK
    ms, n = ctypes.c_double(-1.0), ctypes.c_int(-1)
    assert L.attn_timing_end(ctypes.byref(ms), ctypes.byref(n)) == attn.ATTN_OK
    assert ms.value == 0.0 and n.value == 0
    assert L.attn_timing_end(None, ctypes.byref(n)) == attn.ATTN_ERR_INVALID


def test_timing_clock_needs_recorded_sums():
    L = _lib()
    mhz = ctypes.c_double(-1.0)
    per = (ctypes.c_double * 8)(*([-1.0] * 8))
    assert L.attn_timing_clock(None, per) == attn.ATTN_ERR_INVALID
    assert L.attn_timing_begin() == attn.ATTN_OK
    assert L.attn_timing_clock(ctypes.byref(mhz), per) == attn.ATTN_ERR_INVALID  # still on
    ms, n = ctypes.c_double(0.0), ctypes.c_int(0)
    assert L.attn_timing_end(ctypes.byref(ms), ctypes.byref(n)) == attn.ATTN_OK
    # no attention kernel ran, so there are no sums: an error, outputs cleared
    assert L.attn_timing_clock(ctypes.byref(mhz), per) == attn.ATTN_ERR_HIP
    assert mhz.value == 0.0 and list(per) == [0.0] * 8


def test_timing_reruns_rejects_null_outputs_and_running_timing():
    L = _lib()
    n, r = ctypes.c_longlong(-1), ctypes.c_longlong(-1)
    assert L.attn_timing_reruns(None, ctypes.byref(r)) == attn.ATTN_ERR_INVALID
    assert L.attn_timing_reruns(ctypes.byref(n), None) == attn.ATTN_ERR_INVALID
    assert L.attn_timing_begin() == attn.ATTN_OK
    assert L.attn_timing_reruns(ctypes.byref(n), ctypes.byref(r)) == attn.ATTN_ERR_INVALID
    assert n.value == 0 and r.value == 0  # cleared on every call
    ms, k = ctypes.c_double(0.0), ctypes.c_int(0)
    assert L.attn_timing_end(ctypes.byref(ms), ctypes.byref(k)) == attn.ATTN_OK


def _kvw(kn=A, vn=A, ks=A, vs=A, pos=A, col=A, srows=None, T=4, Hkv=2, D=64, rows=32, cols=3,
         kns=None, vns=None, kss=None, vss=None, ws=A, ws_bytes=1024):
    L = _lib()
    kns = kns or _s(Hkv * D, D, 1)
    vns = vns or _s(Hkv * D, D, 1)
    kss = kss or _s(cols * Hkv * D, Hkv * D, D, 1)
    vss = vss or _s(cols * Hkv * D, Hkv * D, D, 1)
    return L.attn_kv_write(kn, vn, ks, vs, pos, col, srows, T, Hkv, D, rows, cols, kns, vns,
                           kss, vss, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(ks=None), attn.ATTN_ERR_INVALID),
    (dict(pos=None), attn.ATTN_ERR_INVALID),
    (dict(col=None), attn.ATTN_ERR_INVALID),
    (dict(kn=None), attn.ATTN_ERR_INVALID),
    (dict(T=-1), attn.ATTN_ERR_INVALID),
    (dict(rows=0), attn.ATTN_ERR_INVALID),
    (dict(D=60), attn.ATTN_ERR_UNSUPPORTED),
    (dict(kns=_s(128, 64, 2)), attn.ATTN_ERR_UNSUPPORTED),
    (dict(kss=_s(384, 128, 60, 1)), attn.ATTN_ERR_UNSUPPORTED),
    (dict(ks=A + 8), attn.ATTN_ERR_UNSUPPORTED),
    (dict(pos=A + 4), attn.ATTN_ERR_UNSUPPORTED),
    (dict(ws=None), attn.ATTN_ERR_WORKSPACE),
    (dict(ws_bytes=16), attn.ATTN_ERR_WORKSPACE),
    (dict(ws=A + 16), attn.ATTN_ERR_WORKSPACE),
])
def test_kv_write_validation(kw, code):
    assert _kvw(**kw) == code, attn.lib().attn_last_error()


def test_kv_write_zero_tokens_is_a_no_op_and_reads_no_error():
    """T == 0 enqueues nothing (no GPU needed); its error word reads 0."""
    L = _lib()
    assert _kvw(T=0, kn=None, vn=None, pos=None, col=None) == attn.ATTN_OK
    assert L.attn_kv_write_workspace(0) == 256
    assert L.attn_kv_write_workspace(5) == 256
    assert L.attn_kv_write_workspace(4 * 64 + 1) == 512


def test_kv_write_flags_match_the_oracle_bits():
    assert (attn.KV_COL, attn.KV_POS, attn.KV_ROWS) == (oracle.KVF_COL, oracle.KVF_POS,
                                                         oracle.KVF_ROWS)


def test_prefill_dev_needs_bounds_and_an_error_word():
    L = _lib()
    D, Hq, Hkv, Lq, Lkv = 64, 4, 2, 8, 16
    qs = _s(Hq * Lq * D, Lq * D, D, 1)
    ks = _s(Hkv * Lkv * D, Lkv * D, D, 1)
    args = (A, A, A, A, 1, Hq, Hkv, Lq, Lkv, D, 0.125, qs, ks, ks, qs)
    assert L.attn_causal_prefill_dev(*args, None, 0, A, 4096, None) == attn.ATTN_ERR_INVALID
    assert L.attn_causal_prefill_dev(*args, A, 0, None, 0, None) == attn.ATTN_ERR_WORKSPACE
    assert L.attn_causal_prefill_dev(*args, A, 0, A, 128, None) == attn.ATTN_ERR_WORKSPACE
    assert L.attn_causal_prefill_dev(*args, A + 4, 0, A, 4096, None) == attn.ATTN_ERR_UNSUPPORTED
    # Lq == 0 enqueues nothing
    args0 = (A, A, A, A, 1, Hq, Hkv, 0, Lkv, D, 0.125, qs, ks, ks, qs)
    assert L.attn_causal_prefill_dev(*args0, A, 0, None, 0, None) == attn.ATTN_OK
    assert (attn.BOUND_KV, attn.BOUND_QPOS) == (1, 2)
