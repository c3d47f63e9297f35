"""Block-sparse attention forward for AMD Instinct MI355X (gfx950).

Thin Python binding over ``libvsa_attn.so`` (C ABI in ``include/vsa_attn.h``).
Functions carry the C names and only marshal arguments: they check tensor
placement, dtypes and shapes, allocate outputs when none are given, and pass
raw device pointers plus the current HIP stream. Every step of the forward
pass runs in the library's HIP kernels; there is no fallback path.

Layouts: q, k, v, o ``[B, S, H, D]`` bf16; lse ``[B, H, S]`` fp32;
kv_block_idx ``[B, H, S/block_q, ld]`` int32; kv_block_cnt
``[B, H, S/block_q]`` int32; logical masks ``[B, H, NQ, NKV]`` uint8.
"""

from __future__ import annotations

import ctypes
import functools
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libvsa_attn.so")

VSA_OK = 0
VSA_ERR_INVALID_ARG = -1
VSA_ERR_UNSUPPORTED = -2
VSA_ERR_HIP = -3

# Exported symbols of the C ABI (checked by the test suite against the header).
SYMBOLS = (
    "vsa_abi_version",
    "vsa_status_string",
    "vsa_last_error",
    "vsa_mask_to_csr",
    "vsa_build_worklist",
    "vsa_expand_valid",
    "vsa_csr_transpose",
    "vsa_pair_q_tiles",
    "vsa_attn_fwd",
    "vsa_attn_fwd_strided",
    "vsa_attn_fwd_noalloc",
    "vsa_attn_fwd_paired",
    "vsa_attn_fwd_coalesced",
    "vsa_attn_fwd_worklist",
    "vsa_attn_bwd",
    "vsa_attn_bwd_strided",
    "vsa_release",
    "vsa_set_max_splits",
    "vsa_measure_mfma",
)


class VsaError(RuntimeError):
    """A library call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libvsa_attn.so (built by ``build.py``); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} not found: build it with `python -m block_sparse_attention_flashattention_amd.build`")
    lib = ctypes.CDLL(path)
    p, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    lib.vsa_abi_version.argtypes = []
    lib.vsa_abi_version.restype = i32
    lib.vsa_status_string.argtypes = [i32]
    lib.vsa_status_string.restype = ctypes.c_char_p
    lib.vsa_last_error.argtypes = []
    lib.vsa_last_error.restype = ctypes.c_char_p
    lib.vsa_mask_to_csr.argtypes = [p, i32, i32, i32, i32, i32, i32, i32, i32, p, p, i32, p, p, p]
    lib.vsa_mask_to_csr.restype = i32
    lib.vsa_build_worklist.argtypes = [p, i32, i32, i32, p, p]
    lib.vsa_build_worklist.restype = i32
    lib.vsa_attn_fwd.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32, f32, p, p, p]
    lib.vsa_attn_fwd.restype = i32
    lib.vsa_attn_fwd_strided.argtypes = [p, p, p, ctypes.POINTER(ctypes.c_int64), p, p, p, i32, i32, i32, i32, i32,
                                         i32, i32, f32, p, p, p]
    lib.vsa_attn_fwd_strided.restype = i32
    lib.vsa_attn_fwd_noalloc.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32, f32, p, p, p]
    lib.vsa_attn_fwd_noalloc.restype = i32
    lib.vsa_attn_fwd_worklist.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32, f32, p, i32, p,
                                          p, p]
    lib.vsa_attn_fwd_worklist.restype = i32
    lib.vsa_expand_valid.argtypes = [p, i32, i32, i32, p, p]
    lib.vsa_expand_valid.restype = i32
    lib.vsa_csr_transpose.argtypes = [p, p, i32, i32, i32, i32, i32, p, i32, p, p, p]
    lib.vsa_csr_transpose.restype = i32
    lib.vsa_pair_q_tiles.argtypes = [p, p, i32, i32, i32, i32, p, p, p, p]
    lib.vsa_pair_q_tiles.restype = i32
    lib.vsa_attn_fwd_paired.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, p, p, p]
    lib.vsa_attn_fwd_paired.restype = i32
    lib.vsa_attn_fwd_coalesced.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32, f32, p, p, p]
    lib.vsa_attn_fwd_coalesced.restype = i32
    lib.vsa_attn_bwd.argtypes = [p, p, p, p, p, p, p, p, i32, p, p, i32, p, i32, i32, i32, i32, i32, i32, f32, p, p,
                                 p, p]
    lib.vsa_attn_bwd.restype = i32
    lib.vsa_attn_bwd_strided.argtypes = [p, p, p, p, p, p, ctypes.POINTER(ctypes.c_int64), p, p, i32, p, p, i32, p,
                                         i32, i32, i32, i32, i32, i32, f32, p, p, p, p]
    lib.vsa_attn_bwd_strided.restype = i32
    lib.vsa_release.argtypes = []
    lib.vsa_release.restype = None
    lib.vsa_set_max_splits.argtypes = [i32]
    lib.vsa_set_max_splits.restype = i32
    lib.vsa_measure_mfma.argtypes = [i32, i32, ctypes.POINTER(f32), ctypes.POINTER(f32), p]
    lib.vsa_measure_mfma.restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().vsa_status_string(int(status)).decode()


def _check(rc: int) -> None:
    if rc != VSA_OK:
        raise VsaError(rc, load_library().vsa_last_error().decode())


def _stream_ptr(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int, views: bool = False) -> None:
    """Checks a device tensor argument; ``views``: a strided view whose last
    dimension is contiguous is accepted."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if views:
        if t.stride(-1) != 1:
            raise ValueError(f"{name} must have a contiguous last dimension")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _fwd_args(q, k, v, kv_block_idx, kv_block_cnt, block_q, block_kv, o, lse, views=False):
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, name, torch.bfloat16, 4, views)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share the shape [B, S, H, D]")
    B, S, H, D = q.shape
    _dev(kv_block_idx, "kv_block_idx", torch.int32, 4)
    _dev(kv_block_cnt, "kv_block_cnt", torch.int32, 3)
    if S % block_q or S % block_kv:
        raise ValueError(f"seqlen {S} must be divisible by block_q {block_q} and block_kv {block_kv}")
    nq = S // block_q
    if tuple(kv_block_idx.shape[:3]) != (B, H, nq) or tuple(kv_block_cnt.shape) != (B, H, nq):
        raise ValueError(f"kv_block_idx must be [B,H,{nq},ld] and kv_block_cnt [B,H,{nq}]")
    if o is None:
        o = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=q.device)  # contiguous, whatever q's strides
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    _dev(o, "o", torch.bfloat16, 4)
    _dev(lse, "lse", torch.float32, 3)
    if o.shape != q.shape or tuple(lse.shape) != (B, H, S):
        raise ValueError("o must be [B,S,H,D] and lse [B,H,S]")
    for name, t in (("k", k), ("v", v), ("kv_block_idx", kv_block_idx), ("kv_block_cnt", kv_block_cnt),
                    ("o", o), ("lse", lse)):
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    return B, S, H, D, o, lse


def _valid_ptr(kv_valid, S, block_kv, device):
    if kv_valid is None:
        return None
    _dev(kv_valid, "kv_valid", torch.int32, 1)
    if kv_valid.numel() != S // block_kv or kv_valid.device != device:
        raise ValueError(f"kv_valid must be an int32 [{S // block_kv}] tensor on {device}")
    return kv_valid.data_ptr()


def _on_tensor_device(fn):
    """Run a binding function with the device of its first tensor argument
    current: every library call works on the calling thread's current HIP
    device, whose stream and memory the call's pointers must belong to."""
    @functools.wraps(fn)
    def wrapped(*args, **kwargs):
        for a in (*args, *kwargs.values()):
            if isinstance(a, torch.Tensor):
                if a.is_cuda:
                    with torch.cuda.device(a.device):
                        return fn(*args, **kwargs)
                break
        return fn(*args, **kwargs)
    return wrapped


@_on_tensor_device
def vsa_attn_fwd(q, k, v, kv_block_idx, kv_block_cnt, block_q, block_kv, scale=None, o=None, lse=None,
                 stream=None, kv_valid=None):
    """Block-sparse attention forward; returns (o, lse).

    Builds the count-sorted work list internally, then runs the fused
    kernel. ``scale`` defaults to 1/sqrt(D). ``kv_valid`` (int32
    [S/block_kv], optional): valid leading keys of each KV tile. q, k, v
    that are strided views (last dimension contiguous) go through
    vsa_attn_fwd_strided.
    """
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        return vsa_attn_fwd_strided(q, k, v, kv_block_idx, kv_block_cnt, block_q, block_kv, scale, o, lse, stream,
                                    kv_valid)
    B, S, H, D, o, lse = _fwd_args(q, k, v, kv_block_idx, kv_block_cnt, block_q, block_kv, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rc = load_library().vsa_attn_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), kv_block_idx.data_ptr(), kv_block_cnt.data_ptr(),
        _valid_ptr(kv_valid, S, block_kv, q.device), B, S, H, D,
        kv_block_idx.shape[3], block_q, block_kv, float(scale), o.data_ptr(), lse.data_ptr(),
        _stream_ptr(stream, q.device))
    _check(rc)
    return o, lse


@_on_tensor_device
def vsa_attn_fwd_strided(q, k, v, kv_block_idx, kv_block_cnt, block_q, block_kv, scale=None, o=None, lse=None,
                         stream=None, kv_valid=None):
    """vsa_attn_fwd reading q, k, v in place through their strides (each a
    [B, S, H, D] view with a contiguous last dimension, e.g. slices of a
    packed QKV projection); returns (o, lse)."""
    B, S, H, D, o, lse = _fwd_args(q, k, v, kv_block_idx, kv_block_cnt, block_q, block_kv, o, lse, views=True)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    strides = (ctypes.c_int64 * 9)(*[t.stride(i) for t in (q, k, v) for i in range(3)])
    rc = load_library().vsa_attn_fwd_strided(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), strides, kv_block_idx.data_ptr(), kv_block_cnt.data_ptr(),
        _valid_ptr(kv_valid, S, block_kv, q.device), B, S, H, D,
        kv_block_idx.shape[3], block_q, block_kv, float(scale), o.data_ptr(), lse.data_ptr(),
        _stream_ptr(stream, q.device))
    _check(rc)
    return o, lse


@_on_tensor_device
def vsa_attn_fwd_noalloc(q, k, v, kv_block_idx, kv_block_cnt, block_q, block_kv, scale=None, o=None, lse=None,
                         stream=None, kv_valid=None):
    """vsa_attn_fwd without device allocation in the library: the work list
    and split workspace live in the library's fixed per-GPU array (calls that
    overlap in time on one GPU race). Pass ``o`` and ``lse`` to keep the
    call itself free of allocation; returns (o, lse)."""
    B, S, H, D, o, lse = _fwd_args(q, k, v, kv_block_idx, kv_block_cnt, block_q, block_kv, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rc = load_library().vsa_attn_fwd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), kv_block_idx.data_ptr(), kv_block_cnt.data_ptr(),
        _valid_ptr(kv_valid, S, block_kv, q.device), B, S, H, D,
        kv_block_idx.shape[3], block_q, block_kv, float(scale), o.data_ptr(), lse.data_ptr(),
        _stream_ptr(stream, q.device))
    _check(rc)
    return o, lse


@_on_tensor_device
def vsa_attn_fwd_paired(q, k, v, kv_block_idx, kv_block_cnt, block_kv, scale=None, o=None, lse=None, stream=None,
                        kv_valid=None):
    """Forward over a 64-row query tile CSR that runs adjacent tiles as one
    128-row tile when every pair has identical lists (decided on the device);
    returns (o, lse), the same as vsa_attn_fwd with block_q=64 up to rounding order."""
    B, S, H, D, o, lse = _fwd_args(q, k, v, kv_block_idx, kv_block_cnt, 64, block_kv, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rc = load_library().vsa_attn_fwd_paired(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), kv_block_idx.data_ptr(), kv_block_cnt.data_ptr(),
        _valid_ptr(kv_valid, S, block_kv, q.device), B, S, H, D,
        kv_block_idx.shape[3], block_kv, float(scale), o.data_ptr(), lse.data_ptr(), _stream_ptr(stream, q.device))
    _check(rc)
    return o, lse


@_on_tensor_device
def vsa_attn_fwd_coalesced(q, k, v, kv_block_idx, kv_block_cnt, block_q, block_kv, scale=None, o=None, lse=None,
                           stream=None, kv_valid=None):
    """Forward over a 64- or 128-row query tile CSR that runs adjacent tiles
    with identical lists as one tile, level by level up to 256 rows (decided
    on the device); returns (o, lse), those of vsa_attn_fwd up to rounding order."""
    B, S, H, D, o, lse = _fwd_args(q, k, v, kv_block_idx, kv_block_cnt, block_q, block_kv, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rc = load_library().vsa_attn_fwd_coalesced(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), kv_block_idx.data_ptr(), kv_block_cnt.data_ptr(),
        _valid_ptr(kv_valid, S, block_kv, q.device), B, S, H, D,
        kv_block_idx.shape[3], block_q, block_kv, float(scale), o.data_ptr(), lse.data_ptr(),
        _stream_ptr(stream, q.device))
    _check(rc)
    return o, lse


@_on_tensor_device
def vsa_pair_q_tiles(kv_block_idx, kv_block_cnt, paired_idx=None, paired_cnt=None, unpaired=None, stream=None):
    """Pair query tiles (2p, 2p+1): returns (paired_idx [B,H,NQ/2,ld],
    paired_cnt [B,H,NQ/2], unpaired [1]) as GPU tensors; no host sync."""
    _dev(kv_block_idx, "kv_block_idx", torch.int32, 4)
    _dev(kv_block_cnt, "kv_block_cnt", torch.int32, 3)
    B, H, NQ, LD = kv_block_idx.shape
    if tuple(kv_block_cnt.shape) != (B, H, NQ):
        raise ValueError("kv_block_cnt must be [B, H, NQ]")
    dev = kv_block_idx.device
    if paired_idx is None:
        paired_idx = torch.full((B, H, NQ // 2, LD), -1, dtype=torch.int32, device=dev)
    if paired_cnt is None:
        paired_cnt = torch.empty((B, H, NQ // 2), dtype=torch.int32, device=dev)
    if unpaired is None:
        unpaired = torch.empty((1,), dtype=torch.int32, device=dev)
    _dev(paired_idx, "paired_idx", torch.int32, 4)
    _dev(paired_cnt, "paired_cnt", torch.int32, 3)
    _dev(unpaired, "unpaired", torch.int32, 1)
    if tuple(paired_idx.shape) != (B, H, NQ // 2, LD) or tuple(paired_cnt.shape) != (B, H, NQ // 2):
        raise ValueError("paired_idx / paired_cnt must be [B, H, NQ/2, ld] / [B, H, NQ/2]")
    rc = load_library().vsa_pair_q_tiles(kv_block_idx.data_ptr(), kv_block_cnt.data_ptr(), B, H, NQ, LD,
                                         paired_idx.data_ptr(), paired_cnt.data_ptr(), unpaired.data_ptr(),
                                         _stream_ptr(stream, dev))
    _check(rc)
    return paired_idx, paired_cnt, unpaired


@_on_tensor_device
def vsa_attn_fwd_worklist(q, k, v, kv_block_idx, kv_block_cnt, block_q, block_kv, work_list, scale=None, o=None,
                          lse=None, stream=None, kv_valid=None):
    """The fused kernel alone over a caller-built work list; returns (o, lse)."""
    B, S, H, D, o, lse = _fwd_args(q, k, v, kv_block_idx, kv_block_cnt, block_q, block_kv, o, lse)
    _dev(work_list, "work_list", torch.int32, 1)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rc = load_library().vsa_attn_fwd_worklist(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), kv_block_idx.data_ptr(), kv_block_cnt.data_ptr(),
        _valid_ptr(kv_valid, S, block_kv, q.device), B, S, H, D,
        kv_block_idx.shape[3], block_q, block_kv, float(scale), work_list.data_ptr(), work_list.numel(),
        o.data_ptr(), lse.data_ptr(), _stream_ptr(stream, q.device))
    _check(rc)
    return o, lse


@_on_tensor_device
def vsa_mask_to_csr(mask, logical_block, block, idx_ld, kv_block_idx=None, kv_block_cnt=None, overflow=None,
                    stream=None, kv_valid=None):
    """Exact expansion of a logical mask to ``block`` tiles + block CSR.

    Returns (kv_block_idx, kv_block_cnt). Slots past a row's count are left
    as allocated (zero when allocated here). ``overflow`` (optional int32
    [1] GPU tensor) is set to 1 if some row holds more than ``idx_ld`` tiles.
    ``kv_valid`` (optional int32 [S/block_kv]): valid keys per physical KV
    tile; tiles without a valid key are left out of the lists.
    """
    _dev(mask, "mask", torch.uint8, 4)
    B, H, NQL, NKVL = mask.shape
    lq, lkv = logical_block
    pq, pkv = block
    if lq % pq or lkv % pkv:
        raise ValueError("physical tile sizes must divide the logical block sizes")
    nqp = NQL * (lq // pq)
    if kv_block_idx is None:
        kv_block_idx = torch.zeros((B, H, nqp, idx_ld), dtype=torch.int32, device=mask.device)
    if kv_block_cnt is None:
        kv_block_cnt = torch.empty((B, H, nqp), dtype=torch.int32, device=mask.device)
    _dev(kv_block_idx, "kv_block_idx", torch.int32, 4)
    _dev(kv_block_cnt, "kv_block_cnt", torch.int32, 3)
    if tuple(kv_block_idx.shape) != (B, H, nqp, idx_ld) or tuple(kv_block_cnt.shape) != (B, H, nqp):
        raise ValueError("output CSR shapes do not match the mask and tile shape")
    ovf_ptr = None
    if overflow is not None:
        _dev(overflow, "overflow", torch.int32, 1)
        ovf_ptr = overflow.data_ptr()
    rc = load_library().vsa_mask_to_csr(mask.data_ptr(), B, H, NQL, NKVL, lq, lkv, pq, pkv,
                                        _valid_ptr(kv_valid, NQL * lq, pkv, mask.device),
                                        kv_block_idx.data_ptr(), idx_ld, kv_block_cnt.data_ptr(), ovf_ptr,
                                        _stream_ptr(stream, mask.device))
    _check(rc)
    return kv_block_idx, kv_block_cnt


@_on_tensor_device
def vsa_build_worklist(kv_block_cnt, max_cnt, work_list=None, segment=None, stream=None):
    """Count-sorted work list as int32 [n]: largest count first (stable)
    within each segment of ``segment`` consecutive items. The default
    segment is the last dimension of ``kv_block_cnt`` (one segment per batch
    and head); ``segment = numel`` sorts the whole list."""
    if not kv_block_cnt.is_cuda or kv_block_cnt.dtype != torch.int32 or not kv_block_cnt.is_contiguous():
        raise ValueError("kv_block_cnt must be a contiguous int32 GPU tensor")
    n = kv_block_cnt.numel()
    if segment is None:
        segment = kv_block_cnt.shape[-1] if kv_block_cnt.dim() > 0 else n
    if n and (segment < 1 or n % segment):
        raise ValueError("segment must divide the number of items")
    if work_list is None:
        work_list = torch.empty((n,), dtype=torch.int32, device=kv_block_cnt.device)
    _dev(work_list, "work_list", torch.int32, 1)
    if work_list.numel() != n:
        raise ValueError("work_list must hold one entry per count")
    rc = load_library().vsa_build_worklist(kv_block_cnt.data_ptr(), n, int(max(segment, 1)), int(max_cnt),
                                           work_list.data_ptr(), _stream_ptr(stream, kv_block_cnt.device))
    _check(rc)
    return work_list


@_on_tensor_device
def vsa_expand_valid(vbs, logical_block_kv, block_kv, kv_valid=None, stream=None):
    """Valid keys per physical KV tile (int32 [nkv_logical * LKV/PKV]) from the
    valid tokens per logical KV block ``vbs`` (int32 [nkv_logical] GPU tensor)."""
    _dev(vbs, "vbs", torch.int32, 1)
    if logical_block_kv % block_kv:
        raise ValueError("block_kv must divide logical_block_kv")
    n = vbs.numel() * (logical_block_kv // block_kv)
    if kv_valid is None:
        kv_valid = torch.empty((n,), dtype=torch.int32, device=vbs.device)
    _dev(kv_valid, "kv_valid", torch.int32, 1)
    if kv_valid.numel() != n:
        raise ValueError(f"kv_valid must hold {n} entries")
    rc = load_library().vsa_expand_valid(vbs.data_ptr(), vbs.numel(), logical_block_kv, block_kv,
                                         kv_valid.data_ptr(), _stream_ptr(stream, vbs.device))
    _check(rc)
    return kv_valid


@_on_tensor_device
def vsa_csr_transpose(kv_block_idx, kv_block_cnt, nkv, q_ld, q_block_idx=None, q_block_cnt=None, overflow=None,
                      stream=None):
    """Q-direction block CSR for the backward pass: (q_block_idx [B,H,nkv,q_ld],
    q_block_cnt [B,H,nkv]), rows listing ascending query tiles."""
    _dev(kv_block_idx, "kv_block_idx", torch.int32, 4)
    _dev(kv_block_cnt, "kv_block_cnt", torch.int32, 3)
    B, H, NQ, LD = kv_block_idx.shape
    if tuple(kv_block_cnt.shape) != (B, H, NQ):
        raise ValueError("kv_block_cnt must be [B, H, NQ] matching kv_block_idx")
    dev = kv_block_idx.device
    if q_block_idx is None:
        q_block_idx = torch.full((B, H, nkv, q_ld), -1, dtype=torch.int32, device=dev)
    if q_block_cnt is None:
        q_block_cnt = torch.empty((B, H, nkv), dtype=torch.int32, device=dev)
    _dev(q_block_idx, "q_block_idx", torch.int32, 4)
    _dev(q_block_cnt, "q_block_cnt", torch.int32, 3)
    if tuple(q_block_idx.shape) != (B, H, nkv, q_ld) or tuple(q_block_cnt.shape) != (B, H, nkv):
        raise ValueError("output shapes must be [B,H,nkv,q_ld] and [B,H,nkv]")
    ovf_ptr = None
    if overflow is not None:
        _dev(overflow, "overflow", torch.int32, 1)
        ovf_ptr = overflow.data_ptr()
    rc = load_library().vsa_csr_transpose(kv_block_idx.data_ptr(), kv_block_cnt.data_ptr(), B, H, NQ, nkv, LD,
                                          q_block_idx.data_ptr(), q_ld, q_block_cnt.data_ptr(), ovf_ptr,
                                          _stream_ptr(stream, dev))
    _check(rc)
    return q_block_idx, q_block_cnt


@_on_tensor_device
def vsa_attn_bwd(q, k, v, o, lse, dout, kv_block_idx, kv_block_cnt, q_block_idx, q_block_cnt, block_q, block_kv,
                 scale=None, dq=None, dk=None, dv=None, stream=None, kv_valid=None):
    """Backward pass of vsa_attn_fwd; returns (dq, dk, dv), bf16 [B, S, H, D].

    ``o`` and ``lse`` are the forward's outputs; ``q_block_idx`` /
    ``q_block_cnt`` the transposed CSR from ``vsa_csr_transpose``. q, k, v
    and dout that are strided views (last dimension contiguous) go through
    vsa_attn_bwd_strided."""
    if not all(t.is_contiguous() for t in (q, k, v, dout)):
        return vsa_attn_bwd_strided(q, k, v, o, lse, dout, kv_block_idx, kv_block_cnt, q_block_idx, q_block_cnt,
                                    block_q, block_kv, scale, dq, dk, dv, stream, kv_valid)
    return _bwd(q, k, v, o, lse, dout, kv_block_idx, kv_block_cnt, q_block_idx, q_block_cnt, block_q, block_kv, scale,
                dq, dk, dv, stream, kv_valid, views=False)


@_on_tensor_device
def vsa_attn_bwd_strided(q, k, v, o, lse, dout, kv_block_idx, kv_block_cnt, q_block_idx, q_block_cnt, block_q,
                         block_kv, scale=None, dq=None, dk=None, dv=None, stream=None, kv_valid=None):
    """vsa_attn_bwd reading q, k, v and dout in place through their strides
    (each a [B, S, H, D] view with a contiguous last dimension); o, lse and
    the gradients are contiguous. Returns (dq, dk, dv)."""
    return _bwd(q, k, v, o, lse, dout, kv_block_idx, kv_block_cnt, q_block_idx, q_block_cnt, block_q, block_kv, scale,
                dq, dk, dv, stream, kv_valid, views=True)


def _bwd(q, k, v, o, lse, dout, kv_block_idx, kv_block_cnt, q_block_idx, q_block_cnt, block_q, block_kv, scale, dq,
         dk, dv, stream, kv_valid, views):
    B, S, H, D, o, lse = _fwd_args(q, k, v, kv_block_idx, kv_block_cnt, block_q, block_kv, o, lse, views=views)
    _dev(dout, "dout", torch.bfloat16, 4, views=views)
    if dout.shape != q.shape:
        raise ValueError("dout must match q")
    nkv = S // block_kv
    _dev(q_block_idx, "q_block_idx", torch.int32, 4)
    _dev(q_block_cnt, "q_block_cnt", torch.int32, 3)
    if tuple(q_block_idx.shape[:3]) != (B, H, nkv) or tuple(q_block_cnt.shape) != (B, H, nkv):
        raise ValueError(f"q_block_idx must be [B,H,{nkv},q_ld] and q_block_cnt [B,H,{nkv}]")
    grads = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            t = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
        _dev(t, name, torch.bfloat16, 4)
        if t.shape != q.shape:
            raise ValueError(f"{name} must match q")
        grads.append(t)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    lib = load_library()
    tail = (kv_block_idx.data_ptr(), kv_block_cnt.data_ptr(), kv_block_idx.shape[3], q_block_idx.data_ptr(),
            q_block_cnt.data_ptr(), q_block_idx.shape[3], _valid_ptr(kv_valid, S, block_kv, q.device), B, S, H, D,
            block_q, block_kv, float(scale), grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(),
            _stream_ptr(stream, q.device))
    head = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr())
    if views:
        strides = (ctypes.c_int64 * 12)(*[t.stride(i) for t in (q, k, v, dout) for i in range(3)])
        rc = lib.vsa_attn_bwd_strided(*head, strides, *tail)
    else:
        rc = lib.vsa_attn_bwd(*head, *tail)
    _check(rc)
    return tuple(grads)


def vsa_release() -> None:
    load_library().vsa_release()


def vsa_set_max_splits(max_splits: int) -> int:
    """Most parts (1, 2 or 4) a work item's list may be split into when a
    launch has too few items; returns the previous value."""
    return int(load_library().vsa_set_max_splits(int(max_splits)))


MFMA_MODES = {"random": 0, "zero": 1, "pingpong_softmax": 2}


def vsa_measure_mfma(mode: str = "random", iters: int = 200000, stream=None, device=None) -> dict:
    """What the matrix cores sustain on v_mfma_f32_32x32x16_bf16 with the
    given operands ("random": bf16 N(0,1), "zero", or "pingpong_softmax":
    random operands beside softmax-shaped vector work on the other wave of
    each SIMD): {"tflops": ..., "clock_mhz": ...}. Synchronises."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    t, c = ctypes.c_float(0.0), ctypes.c_float(0.0)
    with torch.cuda.device(dev):  # the library measures on the current device
        _check(load_library().vsa_measure_mfma(MFMA_MODES[mode], int(iters), ctypes.byref(t), ctypes.byref(c),
                                               _stream_ptr(stream, dev)))
    return {"tflops": float(t.value), "clock_mhz": float(c.value)}
