"""The reference CPU attention: test infrastructure, not product.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  It loads ``liboracle.so`` (plain C, fp64, built
from ``oracle.c`` by ``oracle/build.py``) and marshals torch CPU tensors into
it.  It never touches a GPU and imports nothing from the HIP library.

What the C code computes, and which passages of the pages it follows, is
stated in the header of ``oracle.c``.  ``kv_write`` (the step's K/V slot
write before the varlen attention) is plain data movement and is written
here directly, a Python loop over the step's tokens.
"""
import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB_PATH selects another build (liboracle_san.so, for tests/sanitize.py)
_LIB_PATH = os.environ.get("ORACLE_LIB_PATH") or os.path.join(_HERE, "liboracle.so")
_lib = None

# Bit meanings of the varlen segment flags (the same as the library's error word).
SEGF_QRANGE = 1
SEGF_COL = 2
SEGF_KVEND = 4
SEGF_ATTR = 8
SEGF_OVERLAP = 16
SEGF_SPAN = 32

# Bit meanings of the slot-write token flags.
KVF_COL = 1
KVF_POS = 2
KVF_ROWS = 4


class OracleInvalid(ValueError):
    """The oracle rejected its arguments (the definition does not apply)."""


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_prefill.restype = I
    lib.oracle_prefill.argtypes = [P, P, P, P, I, I, I, I, I, I, ctypes.c_double,
                                   P, P, P, ctypes.c_int64, I, P, I, P]
    lib.oracle_varlen.restype = I
    lib.oracle_varlen.argtypes = [P, P, P, P, P, I, P, I, I, I, I, I, I,
                                  ctypes.c_double, I, I, I, P, P, P, P]
    lib.oracle_num_threads.restype = I
    lib.oracle_num_threads.argtypes = []
    _lib = lib
    return lib


def num_threads():
    """Threads the oracle's parallel loops use (OpenMP's maximum)."""
    return _load().oracle_num_threads()


def _bits(t):
    """Raw bf16 bits of a CPU bf16 tensor as a uint16 array, plus its strides.

    The array is the tensor's whole underlying storage from its offset on, so
    strided (padded, transposed) views are read through their real strides.
    """
    if t.dtype != torch.bfloat16 or t.device.type != "cpu":
        raise TypeError("oracle inputs are CPU bfloat16 tensors")
    base = t.as_strided((t.untyped_storage().nbytes() // 2 - t.storage_offset(),), (1,))
    arr = base.view(torch.int16).numpy().view(np.uint16)
    return arr, np.asarray(t.stride(), dtype=np.int64)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def prefill(q, k, v, scale, q_pos0=None, window=0, rows=None, return_probs=False):
    """fp64 causal GQA attention (the plain definition).

    q [B,Hq,Lq,D], k/v [B,Hkv,Lkv,D]: CPU bf16 tensors with any strides.
    Query row i sits at position q_pos0 + i (default Lkv - Lq, end-aligned)
    and sees keys j <= that position, within the last ``window`` positions
    when window > 0.  ``rows`` selects query rows (default all).
    Returns float64 [B,Hq,len(rows),D] (and the [.., Lkv] weights on request).
    """
    B, Hq, Lq, D = q.shape
    Bk, Hkv, Lkv, Dk = k.shape
    if Bk != B or Dk != D or tuple(v.shape) != tuple(k.shape):
        raise OracleInvalid("shape mismatch")
    if q_pos0 is None:
        q_pos0 = Lkv - Lq
    qa, qs = _bits(q)
    ka, ks = _bits(k)
    va, vs = _bits(v)
    sel = None
    n_sel = Lq
    if rows is not None:
        sel = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        n_sel = int(sel.size)
    out = np.zeros((B, Hq, n_sel, D), dtype=np.float64)
    probs = np.zeros((B, Hq, n_sel, max(Lkv, 1)), dtype=np.float64) if return_probs else None
    st = _load().oracle_prefill(
        _ptr(qa), _ptr(ka), _ptr(va), _ptr(out), B, Hq, Hkv, Lq, Lkv, D, float(scale),
        _ptr(qs), _ptr(ks), _ptr(vs), int(q_pos0), int(window),
        _ptr(sel) if sel is not None else None, n_sel,
        _ptr(probs) if probs is not None else None)
    if st != 0:
        raise OracleInvalid("oracle_prefill rejected its arguments")
    if return_probs:
        return torch.from_numpy(out), torch.from_numpy(probs[..., :Lkv])
    return torch.from_numpy(out)


def varlen(q, k_store, v_store, seq_info, T=None, seg_attr=None, scale=None,
           causal=1, window=0, ring_rows=0, return_flags=False):
    """fp64 varlen SDPA over a column store (the plain definition).

    q [T,Hq,D] packed rows; k_store/v_store [rows, cols, Hkv, D]; all CPU
    bf16 with any strides.  seq_info int32 [S,4] = (q_start, q_len, col,
    kv_end); seg_attr optional int32 [S,3] = (causal, window, ring_rows).
    Returns float64 [T,Hq,D] (and the OR of segment flags on request).
    """
    Tq, Hq, D = q.shape
    if T is None:
        T = Tq
    rows, cols, Hkv, Dk = k_store.shape
    if Dk != D or tuple(v_store.shape) != tuple(k_store.shape) or Tq < T:
        raise OracleInvalid("shape mismatch")
    if scale is None:
        scale = 1.0 / float(np.sqrt(D))
    si = np.ascontiguousarray(np.asarray(seq_info, dtype=np.int32).reshape(-1, 4))
    S = si.shape[0]
    sa = None
    if seg_attr is not None:
        sa = np.ascontiguousarray(np.asarray(seg_attr, dtype=np.int32).reshape(-1, 3))
        if sa.shape[0] != S:
            raise OracleInvalid("seg_attr rows != seq_info rows")
    qa, qs = _bits(q)
    ka, ks = _bits(k_store)
    va, vs = _bits(v_store)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    err = np.zeros(1, dtype=np.int32)
    st = _load().oracle_varlen(
        _ptr(qa), _ptr(ka), _ptr(va), _ptr(out), _ptr(si), S,
        _ptr(sa) if sa is not None else None, T, Hq, Hkv, D, rows, cols,
        float(scale), int(causal), int(window), int(ring_rows),
        _ptr(qs), _ptr(ks), _ptr(vs), _ptr(err))
    if st != 0:
        raise OracleInvalid("oracle_varlen rejected its arguments (flags %d)" % int(err[0]))
    if return_flags:
        return torch.from_numpy(out), int(err[0])
    return torch.from_numpy(out)


def kv_write(k_store, v_store, k_new, v_new, positions, seq_cols, slot_rows=None):
    """The K/V slot write of one step (the plain definition), functional.

    Follows "[executorch][cuda] Add a length-aware Triton SDPA over
    per-sequence KV columns", the stacked commits on the batched-sequence
    manifest layout (each step token is written to slot (position mod rows)
    x columns + its column, i.e. store row position mod R of that column)
    and on the batched sequence cache (one column per sequence, the last
    column scratch for padded writes; a ring layer's row count is its
    modulus).

    k_store/v_store [rows, cols, Hkv, D] and k_new/v_new [T, Hkv, D]: CPU
    bf16.  positions int64 [T], seq_cols int32 [T]; slot_rows optional int32
    [T], the modulus R of each token (<= 0: rows).  Token i writes
    new[i, h, :] to store[positions[i] mod R_i, seq_cols[i], h, :].  A token
    with a column outside [0, cols), a negative position or R_i > rows is
    skipped and flagged (KVF_COL, KVF_POS, KVF_ROWS).  Tokens are applied in
    order, so when two share a slot the later one stays.
    Returns (k_out, v_out, OR of the flags).
    """
    rows, cols, Hkv, D = k_store.shape
    T = k_new.shape[0]
    if tuple(v_store.shape) != tuple(k_store.shape) or tuple(k_new.shape) != (T, Hkv, D) \
            or tuple(v_new.shape) != (T, Hkv, D):
        raise OracleInvalid("shape mismatch")
    pos = [int(x) for x in positions]
    col = [int(x) for x in seq_cols]
    rr = [int(x) for x in slot_rows] if slot_rows is not None else [0] * T
    if len(pos) != T or len(col) != T or len(rr) != T:
        raise OracleInvalid("per-token arrays must have T entries")
    k_out = k_store.clone()
    v_out = v_store.clone()
    flags = 0
    for i in range(T):
        R = rows if rr[i] <= 0 else rr[i]
        f = 0
        if not 0 <= col[i] < cols:
            f |= KVF_COL
        if pos[i] < 0:
            f |= KVF_POS
        if R > rows:
            f |= KVF_ROWS
        flags |= f
        if f:
            continue
        r = pos[i] % R
        k_out[r, col[i]] = k_new[i]
        v_out[r, col[i]] = v_new[i]
    return k_out, v_out, flags
