"""C-ABI checks that need no GPU: the library loads, exports what the header
declares, and rejects every invalid argument before touching HIP."""

import ctypes
import os
import re

import numpy as np
import pytest

import attention_causal_gqa_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def lib():
    return A.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_api():
    names = declared_functions()
    for n in ("attn_prefill", "attn_prefill_paged", "attn_prefill_paged_append", "attn_decode_paged_append",
              "attn_prefill_varlen",
              "attn_validate_varlen_metadata",
              "attn_kv_append", "attn_decode_paged_fp8", "attn_decode_paged", "attn_decode_workspace_bytes",
              "attn_decode_num_splits", "attn_validate_paged_metadata", "attn_validate_chunk_metadata",
              "attn_status_string", "attn_last_error_message"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        # exported with C linkage (unmangled)
        ctypes.CDLL(A.LIB_PATH)[name]


def test_status_strings(lib):
    for st in (A.ATTN_OK, A.ATTN_ERR_INVALID_ARG, A.ATTN_ERR_UNSUPPORTED, A.ATTN_ERR_WORKSPACE, A.ATTN_ERR_HIP, 7):
        assert A.attn_status_string(st)


FAKE = 1 << 20  # a 16-byte aligned non-null address; never dereferenced by rejected calls


def prefill(lib, q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, B=1, Hq=4, Hkv=2, T=16, d=128, scale=0.1, dtype=1):
    return lib.attn_prefill(q, k, v, out, lse, B, Hq, Hkv, T, d, scale, dtype, None)


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(q=None), A.ATTN_ERR_INVALID_ARG),
        (dict(out=None), A.ATTN_ERR_INVALID_ARG),
        (dict(q=FAKE + 8), A.ATTN_ERR_INVALID_ARG),
        (dict(lse=FAKE + 2), A.ATTN_ERR_INVALID_ARG),
        (dict(Hq=3, Hkv=2), A.ATTN_ERR_INVALID_ARG),
        (dict(Hkv=0), A.ATTN_ERR_INVALID_ARG),
        (dict(B=-1), A.ATTN_ERR_INVALID_ARG),
        (dict(T=-5), A.ATTN_ERR_INVALID_ARG),
        (dict(d=0), A.ATTN_ERR_INVALID_ARG),
        (dict(scale=float("nan")), A.ATTN_ERR_INVALID_ARG),
        (dict(scale=float("inf")), A.ATTN_ERR_INVALID_ARG),
        (dict(dtype=7), A.ATTN_ERR_INVALID_ARG),
        (dict(d=96), A.ATTN_ERR_UNSUPPORTED),
        (dict(d=256, dtype=0), A.ATTN_ERR_UNSUPPORTED),
        (dict(Hq=256, Hkv=1), A.ATTN_ERR_UNSUPPORTED),
    ],
)
def test_prefill_rejects(lib, kw, status):
    assert prefill(lib, **kw) == status
    assert A.attn_last_error_message() != ""


def test_prefill_empty_is_a_no_op(lib):
    assert prefill(lib, q=None, k=None, v=None, out=None, B=0) == A.ATTN_OK
    assert prefill(lib, q=None, k=None, v=None, out=None, T=0) == A.ATTN_OK


def decode(lib, q=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, sl=FAKE, out=FAKE, lse=None, B=2, Hq=4, Hkv=2, d=128, ps=16,
           P=10, W=8, scale=0.1, dtype=1, ns=0, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = lib.attn_decode_workspace_bytes(max(B, 0), Hq, Hkv, d, ps, W, ns) if B >= 0 else 0
    return lib.attn_decode_paged(q, kp, vp, bt, sl, out, lse, B, Hq, Hkv, d, ps, P, W, scale, dtype, ns, ws, wsb,
                                 None)


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(q=None), A.ATTN_ERR_INVALID_ARG),
        (dict(bt=None), A.ATTN_ERR_INVALID_ARG),
        (dict(sl=None), A.ATTN_ERR_INVALID_ARG),
        (dict(kp=FAKE + 4), A.ATTN_ERR_INVALID_ARG),
        (dict(bt=FAKE + 2), A.ATTN_ERR_INVALID_ARG),
        (dict(Hq=5, Hkv=2), A.ATTN_ERR_INVALID_ARG),
        (dict(B=-1), A.ATTN_ERR_INVALID_ARG),
        (dict(W=0), A.ATTN_ERR_INVALID_ARG),
        (dict(P=-1), A.ATTN_ERR_INVALID_ARG),
        (dict(ns=-2), A.ATTN_ERR_INVALID_ARG),
        (dict(scale=float("nan")), A.ATTN_ERR_INVALID_ARG),
        (dict(ws=FAKE + 4), A.ATTN_ERR_INVALID_ARG),
        (dict(dtype=0), A.ATTN_ERR_UNSUPPORTED),
        (dict(d=80), A.ATTN_ERR_UNSUPPORTED),
        (dict(ps=32), A.ATTN_ERR_UNSUPPORTED),
        (dict(Hq=34, Hkv=2), A.ATTN_ERR_UNSUPPORTED),
        (dict(ws=None), A.ATTN_ERR_WORKSPACE),
        (dict(wsb=16), A.ATTN_ERR_WORKSPACE),
    ],
)
def test_decode_rejects(lib, kw, status):
    assert decode(lib, **kw) == status


def decode_append(lib, q=FAKE, kn=FAKE, vn=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, sl=FAKE, out=FAKE, lse=None, B=2, Hq=4,
                  Hkv=2, d=128, ps=16, P=10, W=8, scale=0.1, dtype=1, ns=0, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = lib.attn_decode_workspace_bytes(max(B, 0), Hq, Hkv, d, ps, W, ns) if B >= 0 else 0
    return lib.attn_decode_paged_append(q, kn, vn, kp, vp, bt, sl, out, lse, B, Hq, Hkv, d, ps, P, W, scale, dtype,
                                        ns, ws, wsb, None)


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(q=None), A.ATTN_ERR_INVALID_ARG),
        (dict(kn=None), A.ATTN_ERR_INVALID_ARG),
        (dict(vn=None), A.ATTN_ERR_INVALID_ARG),
        (dict(vp=None), A.ATTN_ERR_INVALID_ARG),
        (dict(sl=None), A.ATTN_ERR_INVALID_ARG),
        (dict(kn=FAKE + 8), A.ATTN_ERR_INVALID_ARG),
        (dict(vn=FAKE + 2), A.ATTN_ERR_INVALID_ARG),
        (dict(bt=FAKE + 2), A.ATTN_ERR_INVALID_ARG),
        (dict(Hq=5, Hkv=2), A.ATTN_ERR_INVALID_ARG),
        (dict(B=-1), A.ATTN_ERR_INVALID_ARG),
        (dict(W=0), A.ATTN_ERR_INVALID_ARG),
        (dict(ns=-2), A.ATTN_ERR_INVALID_ARG),
        (dict(scale=float("inf")), A.ATTN_ERR_INVALID_ARG),
        (dict(dtype=0), A.ATTN_ERR_UNSUPPORTED),
        (dict(d=80), A.ATTN_ERR_UNSUPPORTED),
        (dict(ps=32), A.ATTN_ERR_UNSUPPORTED),
        (dict(ws=None), A.ATTN_ERR_WORKSPACE),
        (dict(wsb=16), A.ATTN_ERR_WORKSPACE),
    ],
)
def test_decode_append_rejects(lib, kw, status):
    assert decode_append(lib, **kw) == status
    assert A.attn_last_error_message() != ""


def test_decode_append_empty_batch_is_a_no_op(lib):
    assert decode_append(lib, q=None, kn=None, vn=None, kp=None, vp=None, bt=None, sl=None, out=None, B=0, ws=None,
                         wsb=0) == A.ATTN_OK


def decode_noalloc(lib, q=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, sl=FAKE, out=FAKE, lse=None, B=2, Hq=4, Hkv=2, d=128,
                   ps=16, P=10, W=8, scale=0.1, dtype=1, ns=0):
    return lib.attn_decode_paged_noalloc(q, kp, vp, bt, sl, out, lse, B, Hq, Hkv, d, ps, P, W, scale, dtype, ns, None)


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(q=None), A.ATTN_ERR_INVALID_ARG),
        (dict(out=None), A.ATTN_ERR_INVALID_ARG),
        (dict(bt=FAKE + 2), A.ATTN_ERR_INVALID_ARG),
        (dict(Hq=5, Hkv=2), A.ATTN_ERR_INVALID_ARG),
        (dict(scale=float("inf")), A.ATTN_ERR_INVALID_ARG),
        (dict(dtype=0), A.ATTN_ERR_UNSUPPORTED),
        (dict(d=80), A.ATTN_ERR_UNSUPPORTED),
        # 4000 sequences x 32 heads x (128 + 1) fp32 values, plus 4096 slots of 4 heads: past the 64 MiB scratch
        (dict(B=4000, Hq=32, Hkv=8), A.ATTN_ERR_WORKSPACE),
    ],
)
def test_decode_noalloc_rejects(lib, kw, status):
    """The no-allocation decode checks every argument, and the workspace its shape needs against the 64 MiB
    static scratch, before any HIP call."""
    assert decode_noalloc(lib, **kw) == status
    if status == A.ATTN_ERR_WORKSPACE:
        msg = A.attn_last_error_message()
        assert "67108864" in msg and str(lib.attn_decode_workspace_bytes(4000, 32, 8, 128, 16, 8, 0)) in msg


def test_decode_noalloc_limit_is_the_workspace_size(lib):
    # the largest batch of 32 heads (Hkv 8, d 128) that fits the scratch, and the next one
    fits = [B for B in (3524, 3525) if lib.attn_decode_workspace_bytes(B, 32, 8, 128, 16, 8, 0) <= 64 << 20]
    assert fits == [3524]
    assert decode_noalloc(lib, B=3525, Hq=32, Hkv=8) == A.ATTN_ERR_WORKSPACE
    assert decode_noalloc(lib, q=None, B=0) == A.ATTN_OK  # B = 0: nothing to do, nothing checked past the sizes


def decode_fp8(lib, q=FAKE, kp=FAKE, vp=FAKE, ks=1.0, vs=1.0, bt=FAKE, sl=FAKE, out=FAKE, B=2, Hq=4, Hkv=2, d=128,
               ps=16, P=10, W=8, scale=0.1, ns=0, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = lib.attn_decode_workspace_bytes(max(B, 0), Hq, Hkv, d, ps, W, ns) if B >= 0 else 0
    return lib.attn_decode_paged_fp8(q, kp, vp, ks, vs, bt, sl, out, None, B, Hq, Hkv, d, ps, P, W, scale, ns, ws,
                                     wsb, None)


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(kp=None), A.ATTN_ERR_INVALID_ARG),
        (dict(vp=FAKE + 8), A.ATTN_ERR_INVALID_ARG),
        (dict(ks=float("nan")), A.ATTN_ERR_INVALID_ARG),
        (dict(vs=float("inf")), A.ATTN_ERR_INVALID_ARG),
        (dict(Hq=6, Hkv=4), A.ATTN_ERR_INVALID_ARG),
        (dict(W=0), A.ATTN_ERR_INVALID_ARG),
        (dict(d=80), A.ATTN_ERR_UNSUPPORTED),
        (dict(Hq=34, Hkv=2), A.ATTN_ERR_UNSUPPORTED),
        (dict(ws=None), A.ATTN_ERR_WORKSPACE),
    ],
)
def test_decode_fp8_rejects(lib, kw, status):
    assert decode_fp8(lib, **kw) == status


def test_decode_empty_batch_is_a_no_op(lib):
    assert decode(lib, q=None, kp=None, vp=None, bt=None, sl=None, out=None, B=0, ws=None, wsb=0) == A.ATTN_OK


def prefill_paged(lib, q=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, sl=FAKE, out=FAKE, lse=None, B=2, Hq=4, Hkv=2, Tq=40,
                  d=128, ps=16, P=10, W=8, scale=0.1, dtype=1):
    return lib.attn_prefill_paged(q, kp, vp, bt, sl, out, lse, B, Hq, Hkv, Tq, d, ps, P, W, scale, dtype, None)


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(q=None), A.ATTN_ERR_INVALID_ARG),
        (dict(bt=None), A.ATTN_ERR_INVALID_ARG),
        (dict(sl=None), A.ATTN_ERR_INVALID_ARG),
        (dict(out=None), A.ATTN_ERR_INVALID_ARG),
        (dict(kp=FAKE + 4), A.ATTN_ERR_INVALID_ARG),
        (dict(bt=FAKE + 2), A.ATTN_ERR_INVALID_ARG),
        (dict(lse=FAKE + 1), A.ATTN_ERR_INVALID_ARG),
        (dict(Hq=5, Hkv=2), A.ATTN_ERR_INVALID_ARG),
        (dict(B=-1), A.ATTN_ERR_INVALID_ARG),
        (dict(Tq=-1), A.ATTN_ERR_INVALID_ARG),
        (dict(Tq=8 * 16 + 1), A.ATTN_ERR_INVALID_ARG),  # longer than the cache can hold
        (dict(W=0), A.ATTN_ERR_INVALID_ARG),
        (dict(P=-1), A.ATTN_ERR_INVALID_ARG),
        (dict(scale=float("inf")), A.ATTN_ERR_INVALID_ARG),
        (dict(dtype=5), A.ATTN_ERR_INVALID_ARG),
        (dict(dtype=0), A.ATTN_ERR_UNSUPPORTED),
        (dict(d=96), A.ATTN_ERR_UNSUPPORTED),
        (dict(ps=32, Tq=40), A.ATTN_ERR_UNSUPPORTED),
        (dict(Hq=256, Hkv=1), A.ATTN_ERR_UNSUPPORTED),
        (dict(W=8193), A.ATTN_ERR_UNSUPPORTED),
    ],
)
def test_prefill_paged_rejects(lib, kw, status):
    assert prefill_paged(lib, **kw) == status
    assert A.attn_last_error_message() != ""


def test_prefill_paged_empty_is_a_no_op(lib):
    assert prefill_paged(lib, q=None, kp=None, vp=None, bt=None, sl=None, out=None, B=0) == A.ATTN_OK
    assert prefill_paged(lib, q=None, kp=None, vp=None, bt=None, sl=None, out=None, Tq=0) == A.ATTN_OK


def prefill_paged_append(lib, q=FAKE, kn=FAKE, vn=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, sl=FAKE, out=FAKE, lse=None, B=2,
                         Hq=4, Hkv=2, Tq=40, d=128, ps=16, P=10, W=8, scale=0.1, dtype=1):
    return lib.attn_prefill_paged_append(q, kn, vn, kp, vp, bt, sl, out, lse, B, Hq, Hkv, Tq, d, ps, P, W, scale, dtype,
                                         None)


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(q=None), A.ATTN_ERR_INVALID_ARG),
        (dict(kn=None), A.ATTN_ERR_INVALID_ARG),
        (dict(vn=None), A.ATTN_ERR_INVALID_ARG),
        (dict(kp=None), A.ATTN_ERR_INVALID_ARG),
        (dict(vp=None), A.ATTN_ERR_INVALID_ARG),
        (dict(bt=None), A.ATTN_ERR_INVALID_ARG),
        (dict(sl=None), A.ATTN_ERR_INVALID_ARG),
        (dict(out=None), A.ATTN_ERR_INVALID_ARG),
        (dict(vn=FAKE + 8), A.ATTN_ERR_INVALID_ARG),
        (dict(vp=FAKE + 4), A.ATTN_ERR_INVALID_ARG),
        (dict(bt=FAKE + 2), A.ATTN_ERR_INVALID_ARG),
        (dict(lse=FAKE + 1), A.ATTN_ERR_INVALID_ARG),
        (dict(Hq=5, Hkv=2), A.ATTN_ERR_INVALID_ARG),
        (dict(B=-1), A.ATTN_ERR_INVALID_ARG),
        (dict(Tq=-1), A.ATTN_ERR_INVALID_ARG),
        (dict(Tq=8 * 16 + 1), A.ATTN_ERR_INVALID_ARG),
        (dict(W=0), A.ATTN_ERR_INVALID_ARG),
        (dict(P=-1), A.ATTN_ERR_INVALID_ARG),
        (dict(scale=float("nan")), A.ATTN_ERR_INVALID_ARG),
        (dict(dtype=5), A.ATTN_ERR_INVALID_ARG),
        (dict(dtype=0), A.ATTN_ERR_UNSUPPORTED),
        (dict(d=96), A.ATTN_ERR_UNSUPPORTED),
        (dict(ps=32, Tq=40), A.ATTN_ERR_UNSUPPORTED),
        (dict(Hq=256, Hkv=1), A.ATTN_ERR_UNSUPPORTED),
        (dict(W=8193), A.ATTN_ERR_UNSUPPORTED),
    ],
)
def test_prefill_paged_append_rejects(lib, kw, status):
    assert prefill_paged_append(lib, **kw) == status
    assert A.attn_last_error_message() != ""


def test_prefill_paged_append_empty_is_a_no_op(lib):
    none = dict(q=None, kn=None, vn=None, kp=None, vp=None, bt=None, sl=None, out=None)
    assert prefill_paged_append(lib, B=0, **none) == A.ATTN_OK
    assert prefill_paged_append(lib, Tq=0, **none) == A.ATTN_OK


def kv_append(lib, kn=FAKE, vn=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, sl=FAKE, B=2, Hkv=2, Tn=40, d=128, ps=16, P=10, W=8,
              dtype=1):
    return lib.attn_kv_append(kn, vn, kp, vp, bt, sl, B, Hkv, Tn, d, ps, P, W, dtype, None)


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(kn=None), A.ATTN_ERR_INVALID_ARG),
        (dict(vp=None), A.ATTN_ERR_INVALID_ARG),
        (dict(bt=None), A.ATTN_ERR_INVALID_ARG),
        (dict(kn=FAKE + 8), A.ATTN_ERR_INVALID_ARG),
        (dict(sl=FAKE + 1), A.ATTN_ERR_INVALID_ARG),
        (dict(B=-1), A.ATTN_ERR_INVALID_ARG),
        (dict(Tn=-1), A.ATTN_ERR_INVALID_ARG),
        (dict(Tn=8 * 16 + 1), A.ATTN_ERR_INVALID_ARG),
        (dict(Hkv=0), A.ATTN_ERR_INVALID_ARG),
        (dict(W=0), A.ATTN_ERR_INVALID_ARG),
        (dict(dtype=9), A.ATTN_ERR_INVALID_ARG),
        (dict(dtype=0), A.ATTN_ERR_UNSUPPORTED),
        (dict(d=32), A.ATTN_ERR_UNSUPPORTED),
        (dict(ps=8, Tn=4), A.ATTN_ERR_UNSUPPORTED),
    ],
)
def test_kv_append_rejects(lib, kw, status):
    assert kv_append(lib, **kw) == status
    assert A.attn_last_error_message() != ""


def test_kv_append_empty_is_a_no_op(lib):
    assert kv_append(lib, kn=None, vn=None, kp=None, vp=None, bt=None, sl=None, B=0) == A.ATTN_OK
    assert kv_append(lib, kn=None, vn=None, kp=None, vp=None, bt=None, sl=None, Tn=0) == A.ATTN_OK


def prefill_varlen(lib, q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, cu=FAKE, S=3, N=100, Tmax=60, Hq=4, Hkv=2,
                   d=128, scale=0.1, dtype=1):
    return lib.attn_prefill_varlen(q, k, v, out, lse, cu, S, N, Tmax, Hq, Hkv, d, scale, dtype, None)


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(q=None), A.ATTN_ERR_INVALID_ARG),
        (dict(cu=None), A.ATTN_ERR_INVALID_ARG),
        (dict(v=FAKE + 8), A.ATTN_ERR_INVALID_ARG),
        (dict(cu=FAKE + 2), A.ATTN_ERR_INVALID_ARG),
        (dict(S=-1), A.ATTN_ERR_INVALID_ARG),
        (dict(N=-1), A.ATTN_ERR_INVALID_ARG),
        (dict(Hq=6, Hkv=4), A.ATTN_ERR_INVALID_ARG),
        (dict(scale=float("nan")), A.ATTN_ERR_INVALID_ARG),
        (dict(dtype=3), A.ATTN_ERR_INVALID_ARG),
        (dict(dtype=0), A.ATTN_ERR_UNSUPPORTED),
        (dict(d=256), A.ATTN_ERR_UNSUPPORTED),
        (dict(Hq=256, Hkv=1), A.ATTN_ERR_UNSUPPORTED),
    ],
)
def test_prefill_varlen_rejects(lib, kw, status):
    assert prefill_varlen(lib, **kw) == status
    assert A.attn_last_error_message() != ""


def test_prefill_varlen_empty_is_a_no_op(lib):
    for kw in (dict(S=0), dict(N=0, Tmax=0), dict(Tmax=0)):
        assert prefill_varlen(lib, q=None, k=None, v=None, out=None, cu=None, **kw) == A.ATTN_OK


def test_validate_varlen_metadata():
    A.attn_validate_varlen_metadata(np.array([0, 3, 3, 10], dtype=np.int32), 10, 7)
    for cu, N, T in (([1, 3, 10], 10, 7), ([0, 5, 3], 3, 7), ([0, 3, 10], 11, 7), ([0, 3, 11], 11, 7)):
        with pytest.raises(A.AttnError):
            A.attn_validate_varlen_metadata(np.array(cu, dtype=np.int32), N, T)


def test_validate_chunk_metadata():
    bt = np.array([[3, 1, -1], [0, 2, -1]], dtype=np.int32)
    A.attn_validate_chunk_metadata(bt, np.array([20, 32], dtype=np.int32), 16, 4, 20)
    with pytest.raises(A.AttnError):
        A.attn_validate_chunk_metadata(bt, np.array([19, 32], dtype=np.int32), 16, 4, 20)  # shorter than the chunk
    with pytest.raises(A.AttnError):
        A.attn_validate_chunk_metadata(bt, np.array([33, 32], dtype=np.int32), 16, 4, 20)  # reads entry -1


def test_split_plan_and_workspace(lib):
    # Explicit split counts: ceil(W / ceil(W / S)), clamped to W.
    assert A.attn_decode_num_splits(4, 8, 4, 128, 16, 128, 1) == 1
    assert A.attn_decode_num_splits(4, 8, 4, 128, 16, 128, 8) == 8
    assert A.attn_decode_num_splits(4, 8, 4, 128, 16, 128, 3) == 3
    assert A.attn_decode_num_splits(4, 8, 4, 128, 16, 5, 100) == 5
    # Automatic plans for the two paged workloads of the benchmark.
    s4 = A.attn_decode_num_splits(32, 16, 8, 128, 16, 128, 0)
    s5 = A.attn_decode_num_splits(64, 32, 8, 128, 16, 512, 0)
    assert 32 * 8 * s4 >= 4096 and 64 * 8 * s5 >= 4096
    # Workspace: P = B * Hkv + 4096 piece slots of G = Hq / Hkv partial rows (d + 1 fp32 each, in two
    # 256-byte aligned regions) plus a 16-byte record per (sequence, kv head); independent of W and the split.
    def r256(x):
        return (x + 255) // 256 * 256

    for (B, Hq, Hkv, W, ns) in ((32, 16, 8, 128, 0), (64, 32, 8, 512, 0), (3, 6, 2, 9, 2), (4096, 32, 8, 8, 0)):
        need = A.attn_decode_workspace_bytes(B, Hq, Hkv, 128, 16, W, ns)
        rows = (B * Hkv + 4096) * (Hq // Hkv)
        assert need == r256(rows * 128 * 4) + r256(rows * 4) + r256(B * Hkv * 16)
        assert need == A.attn_decode_workspace_bytes(B, Hq, Hkv, 128, 16, 3 * W, 1)
    assert A.attn_decode_workspace_bytes(64, 32, 8, 128, 16, 512, 0) < 10 * 2**20  # workload 5: under 10 MiB
    assert A.attn_decode_workspace_bytes(1, 3, 2, 128, 16, 4, 0) == 0  # invalid -> 0
    # The flattened page stream is indexed with 32-bit offsets.
    assert A.attn_decode_workspace_bytes(2**16, 8, 8, 128, 16, 2**12, 0) == 0
    with pytest.raises(A.AttnError) as ei:
        A.attn_decode_num_splits(2**16, 8, 8, 128, 16, 2**12, 0)
    assert ei.value.status == A.ATTN_ERR_UNSUPPORTED
    with pytest.raises(A.AttnError):
        A.attn_decode_num_splits(1, 4, 2, 96, 16, 4, 0)


def test_validate_paged_metadata():
    bt = np.array([[3, 1, -1], [0, -1, -1]], dtype=np.int32)
    A.attn_validate_paged_metadata(bt, np.array([20, 16], dtype=np.int32), 16, 4)
    A.attn_validate_paged_metadata(bt, np.array([0, 0], dtype=np.int32), 16, 4)
    with pytest.raises(A.AttnError):
        A.attn_validate_paged_metadata(bt, np.array([33, 1], dtype=np.int32), 16, 4)  # reads entry -1
    with pytest.raises(A.AttnError):
        A.attn_validate_paged_metadata(bt, np.array([49, 1], dtype=np.int32), 16, 4)  # past W * page_size
    with pytest.raises(A.AttnError):
        A.attn_validate_paged_metadata(bt, np.array([20, 1], dtype=np.int32), 16, 3)  # page 3 outside pool
    with pytest.raises(A.AttnError):
        A.attn_validate_paged_metadata(bt, np.array([-1, 1], dtype=np.int32), 16, 4)


def test_product_path_has_no_cpu_fallback():
    """The package never imports the oracle and has no compute of its own."""
    pkg = os.path.join(ROOT, "attention_causal_gqa_amd")
    for name in os.listdir(pkg):
        if name.endswith(".py"):
            src = open(os.path.join(pkg, name)).read()
            assert not re.search(r"^\s*(import|from)\s+(\.\.)?oracle\b", src, flags=re.M), name
            assert "import_module" not in src and "__import__" not in src, name


def test_asm_load_guard_flags_early_use():
    """The build-time ISA check: a register of an inline-asm load may be touched
    only after the vmcnt wait that retires that load."""
    from attention_causal_gqa_amd.asm_guard import hazards as _asm_load_hazards
    head = "k:\n;;#ASMSTART\n\tglobal_load_dwordx4 v[50:53], v[34:35], off\n;;#ASMEND\n"
    assert _asm_load_hazards(head + "\tv_mov_b32_e32 v34, v50\n\ts_waitcnt vmcnt(0)\n")
    # loads retire in issue order: vmcnt(1) retires the older plain load, not the asm one
    young = "k:\n\tglobal_load_dword v9, v[2:3], off\n;;#ASMSTART\n\tglobal_load_dwordx4 v[50:53], v[34:35], off\n;;#ASMEND\n"
    assert _asm_load_hazards(young + "\ts_waitcnt vmcnt(1)\n\tv_add_f32_e32 v1, v52, v1\n")
    assert not _asm_load_hazards(young + "\ts_waitcnt vmcnt(0)\n\tv_add_f32_e32 v1, v52, v1\n")
    assert not _asm_load_hazards(head + "\tglobal_load_dword v9, v[2:3], off\n\ts_waitcnt vmcnt(1)\n"
                                        "\tv_add_f32_e32 v1, v1, v2\n\ts_waitcnt vmcnt(0)\n\tv_mov_b32_e32 v1, v9\n")
    assert not _asm_load_hazards(head + "\ts_waitcnt vmcnt(0)\n\tv_mov_b32_e32 v34, v50\n")


def test_read_probe_library_loads_and_rejects_bad_arguments():
    """The benchmark's read-bandwidth probe (a library of its own, outside the C ABI) is built beside
    libattn.so; its argument checks run before any HIP call."""
    import ctypes
    import os
    probe = ctypes.CDLL(os.path.join(os.path.dirname(A.__file__), "libattn_probe.so"))
    f = probe.probe_read_slices
    vp = ctypes.c_void_p
    f.argtypes = [vp, vp, ctypes.c_longlong, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, vp]
    f.restype = ctypes.c_int
    good = dict(base=FAKE, offs=None, n=4, slice_bytes=4096, sink=FAKE, blocks=8, nt=1)
    for bad in (dict(base=None), dict(sink=None), dict(n=-1), dict(slice_bytes=8), dict(slice_bytes=4100),
                dict(slice_bytes=8192), dict(blocks=0), dict(nt=2), dict(nt=-1)):
        a = {**good, **bad}
        assert f(a["base"], a["offs"], a["n"], a["slice_bytes"], a["sink"], a["blocks"], a["nt"], None) != 0, bad
    assert f(FAKE, None, 0, 4096, FAKE, 8, 0, None) == 0  # nothing to read: no launch
    assert f(FAKE, None, 0, 4096, FAKE, 8, 1, None) == 0
