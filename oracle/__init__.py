"""CPU oracle for the block-sparse attention forward -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library never imports, links or
calls anything here, and this package shares no code with it.

* ``attn_rows`` / ``attn_full`` / ``probs_row`` wrap ``vsa_oracle.c``, a plain
  fp32 masked SDPA (FastVideo page, ``bench_vsa_blackwell.py``,
  ``ref_masked_sdpa_fp32``); ``bwd_dq_rows`` / ``bwd_dkv_rows`` / ``bwd_full``
  its gradients with respect to Q, K and V.
* ``mask_to_csr`` / ``build_worklist`` / ``expand_valid`` / ``transpose_csr``
  live in ``frontend.py`` (numpy).

Parity of every function here is pinned by ``tests/test_oracle_pins.py`` and
``tests/test_frontend_oracle.py`` against brute force, library routines,
closed forms and invariants.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .frontend import build_worklist, expand_valid, mask_to_csr, transpose_csr  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vsa_oracle.c")
_LIB = os.path.join(_HERE, "libvsa_oracle.so")
_lib = None

_ERRORS = {
    -1: "invalid argument",
    -2: "kv_block_idx entry out of range",
    -3: "duplicate kv_block_idx entry in a row",
    -4: "kv_block_cnt outside [0, ld]",
    -5: "out of memory",
}


def build(force: bool = True) -> str:
    """Compile vsa_oracle.c with plain gcc (no fast-math) into a shared library."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i32 = ctypes.c_int
        i64 = ctypes.c_int64
        lib.vsa_oracle_attn_rows.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32,
                                             ctypes.c_float, p, i64, p, p, i32]
        lib.vsa_oracle_attn_rows.restype = i32
        lib.vsa_oracle_probs_row.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32,
                                             ctypes.c_float, i64, p]
        lib.vsa_oracle_probs_row.restype = i32
        lib.vsa_oracle_bwd_dq_rows.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32,
                                               ctypes.c_float, p, i64, p, i32]
        lib.vsa_oracle_bwd_dq_rows.restype = i32
        lib.vsa_oracle_bwd_dkv_rows.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32,
                                                ctypes.c_float, p, i64, p, p, i32]
        lib.vsa_oracle_bwd_dkv_rows.restype = i32
        lib.vsa_oracle_bwd_full.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32,
                                            ctypes.c_float, p, p, p, i32]
        lib.vsa_oracle_bwd_full.restype = i32
        _lib = lib
    return _lib


def _bits(x) -> np.ndarray:
    """bf16 input as a contiguous uint16 array of raw bits."""
    if isinstance(x, np.ndarray):
        if x.dtype != np.uint16:
            raise TypeError("numpy inputs must hold bf16 bit patterns as uint16")
        return np.ascontiguousarray(x)
    import torch

    if x.dtype != torch.bfloat16:
        raise TypeError("torch inputs must be bfloat16")
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int):
    if rc != 0:
        raise ValueError(f"oracle: {_ERRORS.get(rc, rc)}")


def _valid_arr(kv_valid, S, block_kv):
    if kv_valid is None:
        return None
    a = np.ascontiguousarray(np.asarray(kv_valid), dtype=np.int32)
    if a.shape != (S // block_kv,):
        raise ValueError("kv_valid must hold one count per KV tile: [S/block_kv]")
    return a


def attn_rows(q, k, v, kv_block_idx, kv_block_cnt, block_q, block_kv, scale, rows=None, threads=0, kv_valid=None):
    """O (fp32 [n, D]) and LSE (fp32 [n]) for flat rows (b*H + h)*S + i.

    q, k, v: bf16 [B, S, H, D] (torch tensors or uint16 bit arrays);
    kv_block_idx [B, H, NQ, ld] / kv_block_cnt [B, H, NQ] int32 block CSR.
    ``rows=None`` computes every row in (b, h, i) order. ``kv_valid``
    [S/block_kv]: valid leading key tokens of each KV tile (None: all full).
    """
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    B, S, H, D = qb.shape
    if kb.shape != qb.shape or vb.shape != qb.shape:
        raise ValueError("q, k, v must share the shape [B, S, H, D]")
    idx = np.ascontiguousarray(kv_block_idx, dtype=np.int32)
    cnt = np.ascontiguousarray(kv_block_cnt, dtype=np.int32)
    nq = S // block_q
    if idx.ndim != 4 or idx.shape[:3] != (B, H, nq) or cnt.shape != (B, H, nq):
        raise ValueError("CSR shapes must be idx [B,H,S/block_q,ld], cnt [B,H,S/block_q]")
    ld = idx.shape[3]
    if rows is None:
        n = B * H * S
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows_arr.size
    o = np.empty((n, D), dtype=np.float32)
    lse = np.empty((n,), dtype=np.float32)
    val = _valid_arr(kv_valid, S, block_kv)
    rc = _load().vsa_oracle_attn_rows(
        _ptr(qb), _ptr(kb), _ptr(vb), _ptr(idx), _ptr(cnt), None if val is None else _ptr(val), B, S, H, D, ld,
        block_q, block_kv,
        ctypes.c_float(scale), None if rows_arr is None else _ptr(rows_arr), n, _ptr(o), _ptr(lse),
        int(threads))
    _check(rc)
    return o, lse


def attn_full(q, k, v, kv_block_idx, kv_block_cnt, block_q, block_kv, scale, threads=0, kv_valid=None):
    """O fp32 [B, S, H, D] and LSE fp32 [B, H, S] for every row."""
    qb = _bits(q)
    B, S, H, D = qb.shape
    o, lse = attn_rows(qb, k, v, kv_block_idx, kv_block_cnt, block_q, block_kv, scale, None, threads, kv_valid)
    o = o.reshape(B, H, S, D).transpose(0, 2, 1, 3).copy()
    return o, lse.reshape(B, H, S)


def _bwd_common(q, k, v, dout, kv_block_idx, kv_block_cnt, block_q, block_kv, kv_valid):
    qb, kb, vb, db = _bits(q), _bits(k), _bits(v), _bits(dout)
    B, S, H, D = qb.shape
    for t in (kb, vb, db):
        if t.shape != qb.shape:
            raise ValueError("q, k, v, dout must share the shape [B, S, H, D]")
    idx = np.ascontiguousarray(kv_block_idx, dtype=np.int32)
    cnt = np.ascontiguousarray(kv_block_cnt, dtype=np.int32)
    nq = S // block_q
    if idx.ndim != 4 or idx.shape[:3] != (B, H, nq) or cnt.shape != (B, H, nq):
        raise ValueError("CSR shapes must be idx [B,H,S/block_q,ld], cnt [B,H,S/block_q]")
    val = _valid_arr(kv_valid, S, block_kv)
    return qb, kb, vb, db, idx, cnt, val, (B, S, H, D)


def bwd_dq_rows(q, k, v, dout, kv_block_idx, kv_block_cnt, block_q, block_kv, scale, rows=None, threads=0,
                kv_valid=None):
    """dQ (fp32 [n, D]) for flat query rows (b*H + h)*S + i (None: all rows)."""
    qb, kb, vb, db, idx, cnt, val, (B, S, H, D) = _bwd_common(q, k, v, dout, kv_block_idx, kv_block_cnt,
                                                               block_q, block_kv, kv_valid)
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = B * H * S if rows_arr is None else rows_arr.size
    dq = np.empty((n, D), dtype=np.float32)
    rc = _load().vsa_oracle_bwd_dq_rows(
        _ptr(qb), _ptr(kb), _ptr(vb), _ptr(db), _ptr(idx), _ptr(cnt), None if val is None else _ptr(val), B, S, H,
        D, idx.shape[3], block_q, block_kv, ctypes.c_float(scale), None if rows_arr is None else _ptr(rows_arr), n,
        _ptr(dq), int(threads))
    _check(rc)
    return dq


def bwd_dkv_rows(q, k, v, dout, kv_block_idx, kv_block_cnt, block_q, block_kv, scale, rows=None, threads=0,
                 kv_valid=None):
    """dK, dV (fp32 [n, D] each) for flat key rows (b*H + h)*S + j (None: all rows)."""
    qb, kb, vb, db, idx, cnt, val, (B, S, H, D) = _bwd_common(q, k, v, dout, kv_block_idx, kv_block_cnt,
                                                               block_q, block_kv, kv_valid)
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = B * H * S if rows_arr is None else rows_arr.size
    dk = np.empty((n, D), dtype=np.float32)
    dv = np.empty((n, D), dtype=np.float32)
    rc = _load().vsa_oracle_bwd_dkv_rows(
        _ptr(qb), _ptr(kb), _ptr(vb), _ptr(db), _ptr(idx), _ptr(cnt), None if val is None else _ptr(val), B, S, H,
        D, idx.shape[3], block_q, block_kv, ctypes.c_float(scale), None if rows_arr is None else _ptr(rows_arr), n,
        _ptr(dk), _ptr(dv), int(threads))
    _check(rc)
    return dk, dv


def bwd_full(q, k, v, dout, kv_block_idx, kv_block_cnt, block_q, block_kv, scale, threads=0, kv_valid=None):
    """dQ, dK, dV fp32 [B, S, H, D] for every row (one pass per head)."""
    qb, kb, vb, db, idx, cnt, val, (B, S, H, D) = _bwd_common(q, k, v, dout, kv_block_idx, kv_block_cnt,
                                                               block_q, block_kv, kv_valid)
    dq = np.empty((B, S, H, D), dtype=np.float32)
    dk = np.empty_like(dq)
    dv = np.empty_like(dq)
    rc = _load().vsa_oracle_bwd_full(
        _ptr(qb), _ptr(kb), _ptr(vb), _ptr(db), _ptr(idx), _ptr(cnt), None if val is None else _ptr(val), B, S, H,
        D, idx.shape[3], block_q, block_kv, ctypes.c_float(scale), _ptr(dq), _ptr(dk), _ptr(dv), int(threads))
    _check(rc)
    return dq, dk, dv


def probs_row(q, k, kv_block_idx, kv_block_cnt, block_q, block_kv, scale, flat_row, kv_valid=None):
    """Softmax weights [S] of one query row over all key tokens (0 if masked)."""
    qb, kb = _bits(q), _bits(k)
    B, S, H, D = qb.shape
    idx = np.ascontiguousarray(kv_block_idx, dtype=np.int32)
    cnt = np.ascontiguousarray(kv_block_cnt, dtype=np.int32)
    p = np.empty((S,), dtype=np.float32)
    val = _valid_arr(kv_valid, S, block_kv)
    rc = _load().vsa_oracle_probs_row(_ptr(qb), _ptr(kb), _ptr(idx), _ptr(cnt), None if val is None else _ptr(val),
                                      B, S, H, D,
                                      idx.shape[3], block_q, block_kv, ctypes.c_float(scale),
                                      int(flat_row), _ptr(p))
    _check(rc)
    return p
