"""Property test of the C ABI's host validation (no GPU needed): a call with
at least one invalid argument is rejected with VSA_ERR_INVALID_ARG or
VSA_ERR_UNSUPPORTED and a message, whatever the other arguments are (sizes
up to the int32 limits included), so it never reaches the device.

Every case starts from a valid argument set drawn at random (tile shapes,
head dims, sizes from tiny to far beyond what a GPU holds) and breaks one
to three fields with values that are invalid on their own: a null or
misaligned pointer, a sequence length no tile divides, an unsupported head
dim or tile shape, a list stride out of range, a non-positive or non-finite
scale, a non-positive batch or head count. The pointers are fake addresses:
a rejected call never dereferences them.
"""

import math

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import block_sparse_attention_flashattention_amd as vsa

# The fake addresses below would reach a kernel if validation ever let a call
# through; where a GPU is visible, such a call could fault it, so the property
# is checked on hosts without one only.
pytestmark = pytest.mark.skipif(__import__("torch").cuda.device_count() > 0,
                                reason="fake device addresses: runs only where no GPU is visible")

A = 0x10000  # fake, 256-byte aligned "device" address
MAX_LD = 8192

TENSORS_FWD = ("q", "k", "v", "idx", "cnt", "o", "lse")
TENSORS_BWD = ("q", "k", "v", "o", "lse", "do", "idx", "cnt", "qidx", "qcnt", "dq", "dk", "dv")
ALIGN = {"q": 16, "k": 16, "v": 16, "o": 16, "do": 16, "dq": 16, "dk": 16, "dv": 16, "lse": 4, "idx": 4, "cnt": 4,
         "qidx": 4, "qcnt": 4}


@pytest.fixture(scope="module")
def lib():
    return vsa.load_library()


@st.composite
def valid_base(draw, tensors):
    bq = draw(st.sampled_from([64, 128, 256]))
    bkv = draw(st.sampled_from([64, 128]))
    unit = max(bq, bkv)
    S = unit * draw(st.one_of(st.integers(1, 64), st.integers(1, (1 << 31) // unit - 1)))
    args = {t: A for t in tensors}
    args.update(B=draw(st.one_of(st.integers(1, 4), st.integers(1, (1 << 31) - 1))),
                H=draw(st.one_of(st.integers(1, 48), st.integers(1, (1 << 31) - 1))),
                S=S, D=draw(st.sampled_from([64, 128])), bq=bq, bkv=bkv,
                ld=draw(st.integers(1, MAX_LD)), qld=draw(st.integers(1, MAX_LD)),
                scale=draw(st.floats(1e-3, 4.0)), valid=None)
    return args


def corruption(tensors):
    """One invalid field, as a function that edits an argument dict."""
    def null(t):
        return lambda a: a.update({t: None})

    def misalign(t):
        return lambda a: a.update({t: A + ALIGN[t] // 2})

    edits = [st.sampled_from(tensors).map(null),
             st.sampled_from(tensors).map(misalign),
             st.just(lambda a: a.update(S=a["S"] + 32)),           # no tile shape divides it
             st.sampled_from([0, 32, 96, 192, 256]).map(lambda d: lambda a: a.update(D=d)),
             st.sampled_from([0, 32, 96, 512]).map(lambda b: lambda a: a.update(bq=b)),
             st.sampled_from([0, 32, 96, 256]).map(lambda b: lambda a: a.update(bkv=b)),
             st.sampled_from([0, -1, MAX_LD + 1, (1 << 31) - 1]).map(lambda x: lambda a: a.update(ld=x)),
             st.sampled_from([0.0, -0.5, math.nan, math.inf, -math.inf]).map(lambda x: lambda a: a.update(scale=x)),
             st.sampled_from([0, -1, -(1 << 31)]).map(lambda x: lambda a: a.update(B=x)),
             st.sampled_from([0, -1, -(1 << 31)]).map(lambda x: lambda a: a.update(H=x)),
             st.just(lambda a: a.update(valid=A + 2))]
    return st.one_of(*edits)


def _fwd(lib, a):
    return lib.vsa_attn_fwd(a["q"], a["k"], a["v"], a["idx"], a["cnt"], a["valid"], a["B"], a["S"], a["H"], a["D"],
                            a["ld"], a["bq"], a["bkv"], a["scale"], a["o"], a["lse"], None)


def _bwd(lib, a):
    return lib.vsa_attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["idx"], a["cnt"], a["ld"], a["qidx"],
                            a["qcnt"], a["qld"], a["valid"], a["B"], a["S"], a["H"], a["D"], a["bq"], a["bkv"],
                            a["scale"], a["dq"], a["dk"], a["dv"], None)


FUZZ = settings(max_examples=400, deadline=None, derandomize=True, database=None,
                suppress_health_check=[HealthCheck.too_slow])


@FUZZ
@given(base=valid_base(TENSORS_FWD), edits=st.lists(corruption(TENSORS_FWD), min_size=1, max_size=3))
def test_forward_rejects_any_invalid_field_on_the_host(lib, base, edits):
    for e in edits:
        e(base)
    rc = _fwd(lib, base)
    assert rc in (-1, -2), (rc, base)
    assert lib.vsa_last_error().decode()


@FUZZ
@given(base=valid_base(TENSORS_BWD),
       edits=st.lists(st.one_of(corruption(TENSORS_BWD),
                                st.sampled_from([0, -1, MAX_LD + 1]).map(lambda x: lambda a: a.update(qld=x))),
                      min_size=1, max_size=3))
def test_backward_rejects_any_invalid_field_on_the_host(lib, base, edits):
    for e in edits:
        e(base)
    rc = _bwd(lib, base)
    assert rc in (-1, -2), (rc, base)
    assert lib.vsa_last_error().decode()
