"""Host-side checks of libvsa_attn.so (no GPU needed).

The library must load, export every function ``include/vsa_attn.h``
declares, and reject invalid arguments during host validation, before any
HIP call is made.
"""

import ctypes
import os
import re

import pytest

import block_sparse_attention_flashattention_amd as vsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vsa_attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(vsa_[a-z0-9_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return vsa.load_library()


def test_header_declares_the_binding_symbols():
    assert _declared_functions() == sorted(vsa.SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.vsa_abi_version() == 12


def test_set_max_splits_rounds_and_returns_previous(lib):
    prev = lib.vsa_set_max_splits(3)
    try:
        assert prev in (1, 2, 4)
        assert lib.vsa_set_max_splits(0) == 2  # 3 was rounded down to 2
        assert lib.vsa_set_max_splits(100) == 1
        assert lib.vsa_set_max_splits(-5) == 4
        assert lib.vsa_set_max_splits(2) == 1
    finally:
        lib.vsa_set_max_splits(prev)


def test_status_strings(lib):
    assert lib.vsa_status_string(0) == b"VSA_OK"
    assert lib.vsa_status_string(-1) == b"VSA_ERR_INVALID_ARG"
    assert lib.vsa_status_string(-2) == b"VSA_ERR_UNSUPPORTED"
    assert lib.vsa_status_string(-3) == b"VSA_ERR_HIP"


# Fake device addresses: validation must reject each call before any launch,
# so these are never dereferenced.
A = 0x10000


def _fwd(lib, **kw):
    args = dict(q=A, k=A, v=A, idx=A, cnt=A, valid=None, B=1, S=1024, H=2, D=128, ld=16, bq=128, bkv=64, scale=0.1,
                o=A, lse=A)
    args.update(kw)
    return lib.vsa_attn_fwd(args["q"], args["k"], args["v"], args["idx"], args["cnt"], args["valid"], args["B"],
                            args["S"], args["H"], args["D"], args["ld"], args["bq"], args["bkv"], args["scale"],
                            args["o"], args["lse"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), -1, "null"),
    (dict(lse=None), -1, "null"),
    (dict(B=0), -1, ">= 1"),
    (dict(S=1000), -1, "divisible"),
    (dict(ld=0), -1, "idx_ld"),
    (dict(scale=0.0), -1, "scale"),
    (dict(scale=float("nan")), -1, "scale"),
    (dict(scale=-1.0), -1, "scale"),
    (dict(D=96), -2, "head_dim"),
    (dict(bq=32), -2, "block_q"),
    (dict(bkv=256), -2, "block_kv"),
    (dict(q=A + 2), -1, "aligned"),
    (dict(lse=A + 2), -1, "aligned"),
    (dict(ld=9000), -2, "maximum"),
    (dict(valid=A + 2), -1, "kv_valid"),
    (dict(S=1 << 28, bq=256, H=1), -2, "KV tiles"),
])
def test_attn_fwd_rejects_invalid_arguments(lib, kw, status, needle):
    assert _fwd(lib, **kw) == status
    assert needle in lib.vsa_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), -1, "null"),
    (dict(S=1000), -1, "divisible"),
    (dict(D=96), -2, "head_dim"),
    (dict(ld=9000), -2, "maximum"),
    # 64 * 64 * 65536/64 = 4,194,304 work items: above what the fixed array holds
    (dict(B=64, H=64, S=65536, bq=64, bkv=64), -2, "scratch"),
])
def test_attn_fwd_noalloc_rejects_before_touching_the_device(lib, kw, status, needle):
    args = dict(q=A, k=A, v=A, idx=A, cnt=A, valid=None, B=1, S=1024, H=2, D=128, ld=16, bq=128, bkv=64, scale=0.1,
                o=A, lse=A)
    args.update(kw)
    rc = lib.vsa_attn_fwd_noalloc(args["q"], args["k"], args["v"], args["idx"], args["cnt"], args["valid"],
                                  args["B"], args["S"], args["H"], args["D"], args["ld"], args["bq"], args["bkv"],
                                  args["scale"], args["o"], args["lse"], None)
    assert rc == status
    assert needle in lib.vsa_last_error().decode()


def _packed(B=1, S=1024, H=2, D=128):
    """Strides (elements) of q, k, v sliced from a packed [B, S, 3, H, D] projection."""
    one = [S * 3 * H * D, 3 * H * D, D]
    return one * 3


@pytest.mark.parametrize("edit,status,needle", [
    ({1: 3 * 2 * 128 + 4}, -1, "multiples of 8"),       # q token stride not a 16-byte multiple
    ({5: 36}, -1, "multiples of 8"),                      # k head stride not a 16-byte multiple
    ({0: -1024}, -1, ">= 0"),                             # q batch stride negative
    ({4: -8}, -1, ">= 0"),
    ({4: (1 << 24) + 8}, -2, "2^24"),
])
def test_attn_fwd_strided_rejects_bad_strides(lib, edit, status, needle):
    strides = _packed()
    for i, x in edit.items():
        strides[i] = x
    arr = (ctypes.c_int64 * 9)(*strides)
    B = 2 if 0 in edit else 1
    rc = lib.vsa_attn_fwd_strided(A, A, A, arr, A, A, None, B, 1024, 2, 128, 16, 128, 64, 0.1, A, A, None)
    assert rc == status
    assert needle in lib.vsa_last_error().decode()


def test_attn_fwd_strided_checks_the_common_arguments_first(lib):
    arr = (ctypes.c_int64 * 9)(*_packed())
    rc = lib.vsa_attn_fwd_strided(A, A, A, arr, A, A, None, 1, 1000, 2, 128, 16, 128, 64, 0.1, A, A, None)
    assert rc == -1 and "divisible" in lib.vsa_last_error().decode()
    rc = lib.vsa_attn_fwd_strided(A + 8, A, A, arr, A, A, None, 1, 1024, 2, 128, 16, 128, 64, 0.1, A, A, None)
    assert rc == -1 and "aligned" in lib.vsa_last_error().decode()


def test_attn_fwd_worklist_rejects_bad_work_list(lib):
    rc = lib.vsa_attn_fwd_worklist(A, A, A, A, A, None, 1, 1024, 2, 128, 16, 128, 64, 0.1, None, 5, A, A, None)
    assert rc == -1 and "work_list" in lib.vsa_last_error().decode()
    rc = lib.vsa_attn_fwd_worklist(A, A, A, A, A, None, 1, 1024, 2, 128, 16, 128, 64, 0.1, A, -1, A, A, None)
    assert rc == -1
    rc = lib.vsa_attn_fwd_worklist(A, A, A, A, A, A + 1, 1, 1024, 2, 128, 16, 128, 64, 0.1, A, 4, A, A, None)
    assert rc == -1 and "kv_valid" in lib.vsa_last_error().decode()
    # n_work == 0 is a no-op that succeeds without touching the device
    assert lib.vsa_attn_fwd_worklist(A, A, A, A, A, None, 1, 1024, 2, 128, 16, 128, 64, 0.1, None, 0, A, A,
                                     None) == 0


def test_mask_to_csr_rejects_invalid_arguments(lib):
    f = lib.vsa_mask_to_csr
    # mask, B, H, NQl, NKVl, LQ, LKV, PQ, PKV, kv_valid, idx, ld, cnt, overflow, stream
    assert f(None, 1, 1, 4, 4, 256, 256, 128, 64, None, A, 8, A, None, None) == -1
    # physical tile must divide the logical block
    assert f(A, 1, 1, 4, 4, 256, 256, 96, 64, None, A, 8, A, None, None) == -1
    assert "divide" in lib.vsa_last_error().decode()
    # query and key lengths must agree
    assert f(A, 1, 1, 4, 8, 256, 256, 128, 64, None, A, 8, A, None, None) == -1
    assert f(A, 1, 1, 4, 4, 256, 256, 128, 64, None, A, 0, A, None, None) == -1
    assert f(A, 1, 1, 4, 4, 256, 256, 128, 64, A + 2, A, 8, A, None, None) == -1  # misaligned kv_valid
    assert "kv_valid" in lib.vsa_last_error().decode()


def test_build_worklist_validation(lib):
    assert lib.vsa_build_worklist(A, -1, 1, 10, A, None) == -1
    assert lib.vsa_build_worklist(A, 10, 10, -1, A, None) == -1
    assert lib.vsa_build_worklist(A, 10, 10, 9000, A, None) == -1
    assert lib.vsa_build_worklist(None, 10, 10, 10, A, None) == -1
    assert lib.vsa_build_worklist(A, 10, 3, 10, A, None) == -1  # segment must divide n_items
    assert "segment" in lib.vsa_last_error().decode()
    assert lib.vsa_build_worklist(A, 10, 0, 10, A, None) == -1
    assert lib.vsa_build_worklist(None, 0, 1, 10, None, None) == 0  # empty list: nothing to do


def test_expand_valid_validation(lib):
    f = lib.vsa_expand_valid
    assert f(A, 4, 256, 96, A, None) == -1  # block_kv must divide the logical block
    assert "divide" in lib.vsa_last_error().decode()
    assert f(None, 4, 256, 64, A, None) == -1
    assert f(A, 4, 256, 64, None, None) == -1
    assert f(A + 2, 4, 256, 64, A, None) == -1
    assert f(A, -1, 256, 64, A, None) == -1
    assert f(None, 0, 256, 64, None, None) == 0  # nothing to do


def test_binding_refuses_cpu_tensors():
    import torch

    q = torch.zeros(1, 128, 1, 64, dtype=torch.bfloat16)
    idx = torch.zeros(1, 1, 2, 2, dtype=torch.int32)
    cnt = torch.zeros(1, 1, 2, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        vsa.vsa_attn_fwd(q, q, q, idx, cnt, 64, 64)


def test_csr_transpose_validation(lib):
    f = lib.vsa_csr_transpose
    # kv_block_idx, kv_block_cnt, B, H, nq, nkv, idx_ld, q_block_idx, q_ld, q_block_cnt, overflow, stream
    assert f(None, A, 1, 1, 4, 4, 4, A, 4, A, None, None) == -1
    assert f(A, A, 0, 1, 4, 4, 4, A, 4, A, None, None) == -1
    assert f(A, A, 1, 1, 4, 4, 0, A, 4, A, None, None) == -1
    assert f(A, A, 1, 1, 4, 4, 4, A, 0, A, None, None) == -1
    assert f(A, A, 1, 1, 1 << 20, 4, 4, A, 4, A, None, None) == -2  # nq above the bitmap limit
    assert f(A, A, 1, 1, 4, 4, 4, A + 2, 4, A, None, None) == -1


def _bwd(lib, **kw):
    a = dict(q=A, k=A, v=A, o=A, lse=A, do=A, idx=A, cnt=A, ld=16, qidx=A, qcnt=A, qld=16, valid=None, B=1, S=1024,
             H=2, D=128, bq=128, bkv=64, scale=0.1, dq=A, dk=A, dv=A)
    a.update(kw)
    return lib.vsa_attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["idx"], a["cnt"], a["ld"], a["qidx"],
                            a["qcnt"], a["qld"], a["valid"], a["B"], a["S"], a["H"], a["D"], a["bq"], a["bkv"],
                            a["scale"], a["dq"], a["dk"], a["dv"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(do=None), -1, "null"),
    (dict(dq=None), -1, "null"),
    (dict(qidx=None), -1, "null"),
    (dict(o=None), -1, "null"),
    (dict(dk=A + 4), -1, "aligned"),
    (dict(qld=0), -2, "q_ld"),
    (dict(qld=9000), -2, "q_ld"),
    (dict(S=1000), -1, "divisible"),
    (dict(D=96), -2, "head_dim"),
    (dict(valid=A + 2), -1, "kv_valid"),
])
def test_attn_bwd_rejects_invalid_arguments(lib, kw, status, needle):
    assert _bwd(lib, **kw) == status
    assert needle in lib.vsa_last_error().decode()


def test_pair_q_tiles_validation(lib):
    f = lib.vsa_pair_q_tiles
    # kv_block_idx, kv_block_cnt, B, H, nq, idx_ld, paired_idx, paired_cnt, unpaired, stream
    assert f(None, A, 1, 1, 4, 4, A, A, A, None) == -1
    assert f(A, A, 1, 1, 4, 4, A, A, None, None) == -1
    assert f(A, A, 1, 1, 5, 4, A, A, A, None) == -1  # odd tile count
    assert "even" in lib.vsa_last_error().decode()
    assert f(A, A, 1, 1, 0, 4, A, A, A, None) == -1
    assert f(A, A, 1, 1, 4, 0, A, A, A, None) == -1
    assert f(A, A, 1, 1, 4, 4, A, A, A + 2, None) == -1


def test_attn_fwd_paired_validation(lib):
    f = lib.vsa_attn_fwd_paired
    # q, k, v, idx, cnt, kv_valid, B, S, H, D, ld, block_kv, scale, o, lse, stream
    assert f(A, A, A, A, A, None, 1, 1024, 2, 128, 16, 64, 0.1, None, A, None) == -1
    assert f(A, A, A, A, A, None, 1, 1000, 2, 128, 16, 64, 0.1, A, A, None) == -1  # not a multiple of 64
    assert f(A, A, A, A, A, None, 1, 1024, 2, 96, 16, 64, 0.1, A, A, None) == -2
    assert f(A, A, A, A, A, None, 1, 1024, 2, 128, 16, 256, 0.1, A, A, None) == -2
    assert f(A, A, A, A, A, None, 1, 1024, 2, 128, 9000, 64, 0.1, A, A, None) in (-1, -2)


def test_attn_fwd_coalesced_validation(lib):
    f = lib.vsa_attn_fwd_coalesced
    # q, k, v, idx, cnt, kv_valid, B, S, H, D, ld, block_q, block_kv, scale, o, lse, stream
    assert f(A, A, A, A, A, None, 1, 1024, 2, 128, 16, 256, 64, 0.1, A, A, None) == -2  # 256-row input: unsupported
    assert "block_q 64 or 128" in lib.vsa_last_error().decode()
    assert f(A, A, A, A, A, None, 1, 1024, 2, 128, 16, 32, 64, 0.1, A, A, None) == -2
    assert f(A, A, A, A, A, None, 1, 1024, 2, 128, 16, 64, 64, 0.1, None, A, None) == -1  # null o
    assert f(A, A, A, A, A, None, 1, 1000, 2, 128, 16, 64, 64, 0.1, A, A, None) == -1  # not a multiple of 64
    assert f(A, A, A, A, A, None, 1, 1024, 2, 96, 16, 128, 64, 0.1, A, A, None) == -2  # head_dim
    assert f(A, A, A, A, A, None, 1, 1024, 2, 128, 9000, 128, 64, 0.1, A, A, None) in (-1, -2)  # ld too large
    assert f(A, A, A, A, A, None, 1, 1024, 2, 128, 16, 128, 64, 0.0, A, A, None) == -1  # scale


def test_measure_mfma_rejects_invalid_arguments(lib):
    t, c = ctypes.c_float(0.0), ctypes.c_float(0.0)
    assert lib.vsa_measure_mfma(3, 100, ctypes.byref(t), ctypes.byref(c), None) == -1
    assert "mode" in lib.vsa_last_error().decode()
    assert lib.vsa_measure_mfma(0, 0, ctypes.byref(t), ctypes.byref(c), None) == -1
    assert "iters" in lib.vsa_last_error().decode()
    assert lib.vsa_measure_mfma(0, 2000001, ctypes.byref(t), ctypes.byref(c), None) == -1
    assert lib.vsa_measure_mfma(0, 100, None, ctypes.byref(c), None) == -1
    assert "null" in lib.vsa_last_error().decode()


@pytest.mark.parametrize("edit,status,needle", [
    ({10: 3 * 2 * 128 + 4}, -1, "multiples of 8"),      # dout token stride not a 16-byte multiple
    ({9: -1024}, -1, ">= 0"),                            # dout batch stride negative
    ({4: (1 << 24) + 8}, -2, "2^24"),                    # k token stride too large
])
def test_attn_bwd_strided_rejects_bad_strides(lib, edit, status, needle):
    strides = _packed() + [1024 * 2 * 128, 2 * 128, 128]  # q, k, v from a packed projection, dout contiguous
    for i, x in edit.items():
        strides[i] = x
    arr = (ctypes.c_int64 * 12)(*strides)
    rc = lib.vsa_attn_bwd_strided(A, A, A, A, A, A, arr, A, A, 16, A, A, 16, None, 1, 1024, 2, 128, 128, 64, 0.1,
                                  A, A, A, None)
    assert rc == status
    assert needle in lib.vsa_last_error().decode()
