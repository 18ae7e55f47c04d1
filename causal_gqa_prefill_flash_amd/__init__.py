"""Causal GQA prefill and varlen SDPA on MI355X (gfx950): the Python binding.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libattn.so`` (built from ``csrc/attn.hip`` by ``build.py``),
called through its C ABI (``include/attn.h``).  PyTorch provides device
memory and the current stream.  There is no fallback: if the library is
missing or the tensors are not on a ROCm device, calls raise.
"""
import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# ATTN_LIB_PATH selects another build of the same library (the host
# sanitizer build, libattn_san.so, for tests/sanitize.py)
LIB_PATH = os.environ.get("ATTN_LIB_PATH") or os.path.join(_HERE, "libattn.so")

ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP = range(5)
SEG_QRANGE, SEG_COL, SEG_KVEND, SEG_ATTR, SEG_OVERLAP, SEG_SPAN = 1, 2, 4, 8, 16, 32
KV_COL, KV_POS, KV_ROWS = 1, 2, 4
BOUND_KV, BOUND_QPOS = 1, 2


class AttnError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("attn status %d: %s" % (status, msg))
        self.status = status


_lib = None


def lib():
    """The loaded libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libattn.so is not built: run causal_gqa_prefill_flash_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    I64A = ctypes.POINTER(ctypes.c_int64)
    L.attn_abi_version.restype = I
    L.attn_abi_version.argtypes = []
    L.attn_last_error.restype = ctypes.c_char_p
    L.attn_last_error.argtypes = []
    L.attn_causal_prefill_workspace.restype = SZ
    L.attn_causal_prefill_workspace.argtypes = [I, I, I, I, I, I]
    L.attn_causal_prefill.restype = I
    L.attn_causal_prefill.argtypes = [P, P, P, P, I, I, I, I, I, I, ctypes.c_float,
                                      I64A, I64A, I64A, I64A, I64, I, P, SZ, P]
    L.attn_causal_prefill_noalloc.restype = I
    L.attn_causal_prefill_noalloc.argtypes = [P, P, P, P, I, I, I, I, I, I, ctypes.c_float,
                                              I64A, I64A, I64A, I64A, I64, I, P]
    L.attn_causal_prefill_dev_workspace.restype = SZ
    L.attn_causal_prefill_dev_workspace.argtypes = [I, I, I, I, I, I]
    L.attn_causal_prefill_dev.restype = I
    L.attn_causal_prefill_dev.argtypes = [P, P, P, P, I, I, I, I, I, I, ctypes.c_float,
                                          I64A, I64A, I64A, I64A, P, I, P, SZ, P]
    L.attn_prefill_read_error.restype = I
    L.attn_prefill_read_error.argtypes = [P, P, ctypes.POINTER(ctypes.c_int32)]
    L.attn_sdpa_varlen_workspace.restype = SZ
    L.attn_sdpa_varlen_workspace.argtypes = [I, I, I, I, I, I, I]
    L.attn_sdpa_varlen.restype = I
    L.attn_sdpa_varlen.argtypes = [P, P, P, P, P, I, P, I, I, I, I, I, I, ctypes.c_float,
                                   I, I, I, I64A, I64A, I64A, I64A, P, SZ, P]
    L.attn_varlen_read_error.restype = I
    L.attn_varlen_read_error.argtypes = [P, I, I, P, ctypes.POINTER(ctypes.c_int32)]
    L.attn_kv_write_workspace.restype = SZ
    L.attn_kv_write_workspace.argtypes = [I]
    L.attn_kv_write.restype = I
    L.attn_kv_write.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I64A, I64A, I64A, I64A,
                                P, SZ, P]
    L.attn_kv_write_read_error.restype = I
    L.attn_kv_write_read_error.argtypes = [P, I, P, ctypes.POINTER(ctypes.c_int32)]
    L.attn_timing_begin.restype = I
    L.attn_timing_begin.argtypes = []
    L.attn_timing_end.restype = I
    L.attn_timing_end.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I)]
    L.attn_timing_clock.restype = I
    L.attn_timing_clock.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    L.attn_timing_reruns.restype = I
    L.attn_timing_reruns.argtypes = [ctypes.POINTER(ctypes.c_longlong), ctypes.POINTER(ctypes.c_longlong)]
    _lib = L
    return L


def last_error():
    return lib().attn_last_error().decode()


def _check(status):
    if status != ATTN_OK:
        raise AttnError(status, last_error())


def _strides(t, n):
    s = t.stride()
    if len(s) != n:
        raise ValueError("expected a %d-d tensor, got shape %s" % (n, tuple(t.shape)))
    return (ctypes.c_int64 * n)(*s)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _gpu(t, name):
    if not t.is_cuda:
        raise ValueError("%s must be a ROCm device tensor" % name)
    if t.dtype != torch.bfloat16:
        raise ValueError("%s must be bfloat16" % name)


def _same_device(named):
    """Every given tensor on the device of the first (the kernels take raw
    pointers, so a tensor elsewhere would be read as device memory)."""
    named = [(t, n) for t, n in named if t is not None]
    d0 = named[0][0].device
    for t, n in named[1:]:
        if t.device != d0:
            raise ValueError("%s is on %s, %s on %s: all tensors must be on one device"
                             % (n, t.device, named[0][1], d0))


def _check_out(out, shape):
    if out is not None and tuple(out.shape) != tuple(shape):
        raise ValueError("out has shape %s, %s expected" % (tuple(out.shape), tuple(shape)))


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return None
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace of %d bytes is too small (%d needed)" %
                             (workspace.numel() * workspace.element_size(), nbytes))
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def prefill_workspace_bytes(B, Hq, Hkv, Lq, Lkv, D):
    return lib().attn_causal_prefill_workspace(B, Hq, Hkv, Lq, Lkv, D)


def causal_prefill(q, k, v, out=None, scale=None, q_pos0=None, window=0, workspace=None):
    """Causal GQA prefill: out[b,h,i] = softmax attention of query row i
    (position q_pos0 + i, default Lkv - Lq) over keys j <= that position
    (and > position - window when window > 0), key/value head h // (Hq/Hkv).

    q [B,Hq,Lq,D], k/v [B,Hkv,Lkv,D] bf16 on the device, any strides with a
    unit innermost stride.  Returns ``out`` ([B,Hq,Lq,D] bf16).
    """
    B, Hq, Lq, D = q.shape
    Bk, Hkv, Lkv, Dk = k.shape
    if Bk != B or Dk != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q/k/v shapes do not agree: %s %s %s" % (q.shape, k.shape, v.shape))
    _check_out(out, (B, Hq, Lq, D))
    _same_device([(q, "q"), (k, "k"), (v, "v"), (out, "out"), (workspace, "workspace")])
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        if t is not None:
            _gpu(t, n)
    if out is None:
        out = torch.empty((B, Hq, Lq, D), dtype=torch.bfloat16, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if q_pos0 is None:
        q_pos0 = Lkv - Lq
    with torch.cuda.device(q.device):
        need = prefill_workspace_bytes(B, Hq, Hkv, Lq, Lkv, D)
        ws = _workspace(need, q.device, workspace)
        st = lib().attn_causal_prefill(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, Lq, Lkv, D, float(scale),
            _strides(q, 4), _strides(k, 4), _strides(v, 4), _strides(out, 4),
            int(q_pos0), int(window), _ptr(ws), need, _stream())
    _check(st)
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20


def causal_prefill_noalloc(q, k, v, out, scale=None, q_pos0=None, window=0):
    """causal_prefill through the entry point that allocates nothing: the
    split partials live in the library's static device buffer
    (NOALLOC_SCRATCH_BYTES per device, shared by every such call on that
    device, so calls that overlap in time race).  ``out`` must be given, so
    that this call allocates nothing either."""
    B, Hq, Lq, D = q.shape
    Bk, Hkv, Lkv, Dk = k.shape
    if Bk != B or Dk != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q/k/v shapes do not agree: %s %s %s" % (q.shape, k.shape, v.shape))
    _check_out(out, (B, Hq, Lq, D))
    _same_device([(q, "q"), (k, "k"), (v, "v"), (out, "out")])
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _gpu(t, n)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if q_pos0 is None:
        q_pos0 = Lkv - Lq
    with torch.cuda.device(q.device):
        st = lib().attn_causal_prefill_noalloc(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, Lq, Lkv, D, float(scale),
            _strides(q, 4), _strides(k, 4), _strides(v, 4), _strides(out, 4),
            int(q_pos0), int(window), _stream())
    _check(st)
    return out


def prefill_dev_workspace_bytes(B, Hq, Hkv, Lq, Lkv, D):
    return lib().attn_causal_prefill_dev_workspace(B, Hq, Hkv, Lq, Lkv, D)


def causal_prefill_dev(q, k, v, bounds, out=None, scale=None, window=0, workspace=None):
    """causal_prefill with a device-resident bound: ``bounds`` is a device
    int64 tensor [2] = (q_pos0, kv_len); k/v [B,Hkv,Lkv,D] hold Lkv >= kv_len
    keys of capacity.  Returns (out, workspace); read the bound flags with
    ``prefill_read_error(workspace)``."""
    B, Hq, Lq, D = q.shape
    Bk, Hkv, Lkv, Dk = k.shape
    if Bk != B or Dk != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q/k/v shapes do not agree: %s %s %s" % (q.shape, k.shape, v.shape))
    _check_out(out, (B, Hq, Lq, D))
    if bounds.dtype != torch.int64 or not bounds.is_contiguous() or bounds.numel() != 2:
        raise ValueError("bounds must be a contiguous int64 device tensor of 2 entries")
    _same_device([(q, "q"), (k, "k"), (v, "v"), (bounds, "bounds"), (out, "out"),
                  (workspace, "workspace")])
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        if t is not None:
            _gpu(t, n)
    if not bounds.is_cuda:
        raise ValueError("bounds must be a contiguous int64 device tensor of 2 entries")
    if out is None:
        out = torch.empty((B, Hq, Lq, D), dtype=torch.bfloat16, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    with torch.cuda.device(q.device):
        need = prefill_dev_workspace_bytes(B, Hq, Hkv, Lq, Lkv, D)
        ws = _workspace(need, q.device, workspace)
        st = lib().attn_causal_prefill_dev(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, Lq, Lkv, D, float(scale),
            _strides(q, 4), _strides(k, 4), _strides(v, 4), _strides(out, 4), _ptr(bounds),
            int(window), _ptr(ws), need, _stream())
    _check(st)
    return out, ws


def prefill_read_error(workspace):
    """The ATTN_BOUND_* flags of the last device-bound prefill on ``workspace``."""
    e = ctypes.c_int32(0)
    _check(lib().attn_prefill_read_error(_ptr(workspace), _stream(), ctypes.byref(e)))
    return e.value


def varlen_workspace_bytes(S, T, Hq, Hkv, D, rows, cols):
    return lib().attn_sdpa_varlen_workspace(S, T, Hq, Hkv, D, rows, cols)


def sdpa_varlen(q, k_store, v_store, seq_info, seg_attr=None, out=None, scale=None, causal=1,
                window=0, ring_rows=0, workspace=None):
    """Varlen SDPA over a [rows, cols, Hkv, D] column store driven by the
    device table seq_info int32 [S,4] = (q_start, q_len, col, kv_end) and the
    optional per-segment seg_attr int32 [S,3] = (causal, window, ring_rows).

    q [T,Hq,D] packed rows; returns ``out`` [T,Hq,D] with every row written
    (rows of no valid segment are zeros).  Pass ``workspace`` (uint8, at
    least ``varlen_workspace_bytes``) to keep the call allocation-free, e.g.
    under graph capture; read its error word with ``varlen_read_error``.
    """
    T, Hq, D = q.shape
    rows, cols, Hkv, Dk = k_store.shape
    if Dk != D or tuple(v_store.shape) != tuple(k_store.shape):
        raise ValueError("store shapes do not agree")
    _check_out(out, (T, Hq, D))
    if seq_info.dtype != torch.int32 or not seq_info.is_contiguous():
        raise ValueError("seq_info must be a contiguous int32 device tensor")
    S = seq_info.shape[0] if seq_info.numel() else 0
    if seq_info.numel() and tuple(seq_info.shape) != (S, 4):
        raise ValueError("seq_info must be [S, 4]")
    if seg_attr is not None:
        if (seg_attr.dtype != torch.int32 or not seg_attr.is_contiguous() or
                tuple(seg_attr.shape) != (S, 3)):
            raise ValueError("seg_attr must be a contiguous int32 device tensor [S, 3]")
    _same_device([(q, "q"), (k_store, "k_store"), (v_store, "v_store"), (seq_info, "seq_info"),
                  (seg_attr, "seg_attr"), (out, "out"), (workspace, "workspace")])
    for t, n in ((q, "q"), (k_store, "k_store"), (v_store, "v_store"), (out, "out")):
        if t is not None:
            _gpu(t, n)
    if not seq_info.is_cuda:
        raise ValueError("seq_info must be a contiguous int32 device tensor")
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    with torch.cuda.device(q.device):
        need = varlen_workspace_bytes(S, T, Hq, Hkv, D, rows, cols)
        ws = _workspace(need, q.device, workspace)
        st = lib().attn_sdpa_varlen(
            _ptr(q), _ptr(k_store), _ptr(v_store), _ptr(out), _ptr(seq_info), S,
            _ptr(seg_attr), T, Hq, Hkv, D, rows, cols, float(scale), int(causal), int(window),
            int(ring_rows), _strides(q, 3), _strides(k_store, 4), _strides(v_store, 4),
            _strides(out, 3), _ptr(ws), need, _stream())
    _check(st)
    return out, ws


def varlen_read_error(workspace, S, T):
    """OR of the ATTN_SEG_* flags of the last varlen call on ``workspace``."""
    e = ctypes.c_int32(0)
    _check(lib().attn_varlen_read_error(_ptr(workspace), S, T, _stream(), ctypes.byref(e)))
    return e.value


def timing_begin():
    """Start recording HIP events around the attention kernel of every call
    made on this thread (a profiling aid)."""
    _check(lib().attn_timing_begin())


def timing_end():
    """Stop recording; returns (summed attention-kernel ms, launches)."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int(0)
    _check(lib().attn_timing_end(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def timing_clock():
    """After ``timing_end``: (average shader clock in MHz over the timed
    attention workgroups, list of 8 per-XCD values, 0 where none ran)."""
    mhz, per = ctypes.c_double(0.0), (ctypes.c_double * 8)()
    _check(lib().attn_timing_clock(ctypes.byref(mhz), per))
    return mhz.value, list(per)


def timing_reruns():
    """After ``timing_end``: (attention workgroups that finished, how many of
    them redid their key range with the exact running maximum)."""
    n, r = ctypes.c_longlong(0), ctypes.c_longlong(0)
    _check(lib().attn_timing_reruns(ctypes.byref(n), ctypes.byref(r)))
    return n.value, r.value


def kv_write_workspace_bytes(T):
    return lib().attn_kv_write_workspace(T)


def kv_write(k_new, v_new, k_store, v_store, positions, seq_cols, slot_rows=None,
             workspace=None):
    """Write a step's new K/V rows [T,Hkv,D] into the [rows,cols,Hkv,D] stores
    at row positions[i] mod R_i of column seq_cols[i] (R_i = slot_rows[i],
    else rows).  positions int64 [T], seq_cols / slot_rows int32 [T], device
    tensors.  Returns the workspace that holds the error word (read it with
    ``kv_write_read_error``)."""
    _same_device([(k_store, "k_store"), (v_store, "v_store"), (k_new, "k_new"),
                  (v_new, "v_new"), (positions, "positions"), (seq_cols, "seq_cols"),
                  (slot_rows, "slot_rows"), (workspace, "workspace")])
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (k_store, "k_store"), (v_store, "v_store")):
        _gpu(t, n)
    T, Hkv, D = k_new.shape
    rows, cols, Hs, Ds = k_store.shape
    if (Hs, Ds) != (Hkv, D) or tuple(v_new.shape) != (T, Hkv, D) or \
            tuple(v_store.shape) != tuple(k_store.shape):
        raise ValueError("new-row and store shapes do not agree")
    for t, n, dt in ((positions, "positions", torch.int64), (seq_cols, "seq_cols", torch.int32),
                     (slot_rows, "slot_rows", torch.int32)):
        if t is None:
            continue
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous() or t.numel() != T:
            raise ValueError("%s must be a contiguous %s device tensor of %d entries" % (n, dt, T))
    with torch.cuda.device(k_store.device):
        need = kv_write_workspace_bytes(T)
        ws = _workspace(need, k_store.device, workspace)
        st = lib().attn_kv_write(
            _ptr(k_new), _ptr(v_new), _ptr(k_store), _ptr(v_store), _ptr(positions),
            _ptr(seq_cols), _ptr(slot_rows), T, Hkv, D, rows, cols, _strides(k_new, 3),
            _strides(v_new, 3), _strides(k_store, 4), _strides(v_store, 4), _ptr(ws), need,
            _stream())
    _check(st)
    return ws


def kv_write_read_error(workspace, T):
    """OR of the ATTN_KV_* flags of the last kv_write call on ``workspace``."""
    e = ctypes.c_int32(0)
    _check(lib().attn_kv_write_read_error(_ptr(workspace), T, _stream(), ctypes.byref(e)))
    return e.value
