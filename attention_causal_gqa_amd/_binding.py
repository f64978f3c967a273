"""ctypes binding of libattn.so: same names as the C ABI, argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI;
this module turns torch tensors into pointers and sizes, picks the current
HIP stream, allocates outputs or workspace with torch when the caller gives
none, and raises ``AttnError`` on a non-zero status.  If the library is not
built, every call raises: there is no other path.
"""

import contextlib
import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# ATTN_LIBRARY names another build of the same library (for instance the
# host-sanitized one that the CPU tests run the ABI checks against).
LIB_PATH = os.environ.get("ATTN_LIBRARY") or os.path.join(PKG, "libattn.so")

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = -1
ATTN_ERR_UNSUPPORTED = -2
ATTN_ERR_WORKSPACE = -3
ATTN_ERR_HIP = -4

ATTN_F32 = 0
ATTN_BF16 = 1

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


def load_library():
    """The ctypes handle of libattn.so, with argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise AttnError(ATTN_ERR_HIP, f"{LIB_PATH} is not built; run `python -m attention_causal_gqa_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_prefill.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.attn_prefill.restype = i32
    lib.attn_decode_num_splits.argtypes = [i32] * 7
    lib.attn_decode_num_splits.restype = i32
    lib.attn_decode_workspace_bytes.argtypes = [i32] * 7
    lib.attn_decode_workspace_bytes.restype = sz
    lib.attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32, i32,
                                      vp, sz, vp]
    lib.attn_decode_paged.restype = i32
    lib.attn_decode_paged_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                             f32, i32, i32, vp, sz, vp]
    lib.attn_decode_paged_append.restype = i32
    lib.attn_decode_paged_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32,
                                              i32, i32, vp]
    lib.attn_decode_paged_noalloc.restype = i32
    lib.attn_prefill_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32,
                                       vp]
    lib.attn_prefill_paged.restype = i32
    lib.attn_prefill_paged_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                              i32, f32, i32, vp]
    lib.attn_prefill_paged_append.restype = i32
    lib.attn_prefill_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.attn_prefill_varlen.restype = i32
    lib.attn_validate_varlen_metadata.argtypes = [vp, i32, i32, i32]
    lib.attn_validate_varlen_metadata.restype = i32
    lib.attn_kv_append.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.attn_kv_append.restype = i32
    lib.attn_validate_chunk_metadata.argtypes = [vp, vp, i32, i32, i32, i32, i32]
    lib.attn_validate_chunk_metadata.restype = i32
    lib.attn_decode_paged_fp8.argtypes = [vp, vp, vp, f32, f32, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                          f32, i32, vp, sz, vp]
    lib.attn_decode_paged_fp8.restype = i32
    lib.attn_validate_paged_metadata.argtypes = [vp, vp, i32, i32, i32, i32]
    lib.attn_validate_paged_metadata.restype = i32
    lib.attn_status_string.argtypes = [i32]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_last_error_message.argtypes = []
    lib.attn_last_error_message.restype = ctypes.c_char_p
    _lib = lib
    return lib


def attn_status_string(status):
    return load_library().attn_status_string(status).decode()


def attn_last_error_message():
    return load_library().attn_last_error_message().decode()


def _check(status):
    if status != ATTN_OK:
        raise AttnError(status, f"{attn_status_string(status)}: {attn_last_error_message()}")


def _torch():
    import torch

    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise AttnError(ATTN_ERR_UNSUPPORTED, f"dtype {t.dtype} is not supported")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    return _torch().cuda.current_stream().cuda_stream


def _alloc_stream(stream):
    """Context in which torch allocates on the stream the kernels run on.

    Outputs and workspaces allocated here belong to that stream in torch's
    caching allocator, so a block released after the call is reused only by
    later work on the same stream, which runs after these kernels."""
    if stream is None:
        return contextlib.nullcontext()
    torch = _torch()
    s = torch.cuda.ExternalStream(stream) if isinstance(stream, int) else stream
    return torch.cuda.stream(s)


def _require(cond, msg):
    if not cond:
        raise AttnError(ATTN_ERR_INVALID_ARG, msg)


def _dense_on_gpu(name, t):
    _require(t.is_cuda, f"{name} must be a GPU tensor")
    _require(t.is_contiguous(), f"{name} must be contiguous")


def attn_prefill(q, k, v, out=None, lse=None, scale=None, stream=None):
    """Causal prefill.  q [B,Hq,T,d], k/v [B,Hkv,T,d] (bf16 or fp32) -> (out, lse fp32 [B,Hq,T])."""
    torch = _torch()
    _require(q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "q, k, v must be [B, H, T, d]")
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    _require(k.shape == v.shape and k.shape[0] == B and k.shape[2] == T and k.shape[3] == d, "k/v shape mismatch")
    _require(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dense_on_gpu(n, t)
    with _alloc_stream(stream):
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _dense_on_gpu("out", out)
    _require(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    if lse is not False:
        _dense_on_gpu("lse", lse)
        _require(lse.shape == (B, Hq, T) and lse.dtype == torch.float32, "lse must be float32 [B, Hq, T]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lib = load_library()
    _check(lib.attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), None if lse is False else _ptr(lse),
                            B, Hq, Hkv, T, d, float(scale), _dtype_code(q), _stream(stream)))
    return out, (None if lse is False else lse)


def attn_prefill_paged(q, k_pages, v_pages, block_table, seq_lens, out=None, lse=None, scale=None, stream=None):
    """Chunked causal prefill over a paged cache.  q [B,Hq,Tq,d] (the last Tq tokens of each sequence);
    pools [P,Hkv,page,d]; block_table [B,W] int32; seq_lens [B] int32 (>= Tq) -> (out, lse fp32 [B,Hq,Tq])."""
    torch = _torch()
    _require(q.dim() == 4 and k_pages.dim() == 4 and k_pages.shape == v_pages.shape, "bad q / page pool shapes")
    B, Hq, Tq, d = q.shape
    P, Hkv, page_size, dk = k_pages.shape
    _require(dk == d, "page pools and q disagree on d")
    _require(block_table.dim() == 2 and block_table.shape[0] == B and block_table.dtype == torch.int32,
             "block_table must be int32 [B, W]")
    _require(seq_lens.shape == (B,) and seq_lens.dtype == torch.int32, "seq_lens must be int32 [B]")
    for n, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages), ("block_table", block_table),
                 ("seq_lens", seq_lens)):
        _dense_on_gpu(n, t)
    _require(q.dtype == k_pages.dtype == v_pages.dtype, "q and the page pools must share a dtype")
    W = block_table.shape[1]
    with _alloc_stream(stream):
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device)
    _dense_on_gpu("out", out)
    _require(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    if lse is not False:
        _dense_on_gpu("lse", lse)
        _require(lse.shape == (B, Hq, Tq) and lse.dtype == torch.float32, "lse must be float32 [B, Hq, Tq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(load_library().attn_prefill_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                                             _ptr(seq_lens), _ptr(out), None if lse is False else _ptr(lse), B, Hq,
                                             Hkv, Tq, d, page_size, P, W, float(scale), _dtype_code(q),
                                             _stream(stream)))
    return out, (None if lse is False else lse)


def attn_prefill_paged_append(q, k_new, v_new, k_pages, v_pages, block_table, seq_lens, out=None, lse=None,
                              scale=None, stream=None):
    """KV append + chunked prefill in one launch.  q [B,Hq,Tq,d]; k_new/v_new [B,Hkv,Tq,d] (the chunk's keys and
    values, written into the pools in place); pools [P,Hkv,page,d]; block_table [B,W] int32; seq_lens [B] int32 =
    lengths after the append (>= Tq) -> (out, lse fp32 [B,Hq,Tq])."""
    torch = _torch()
    _require(q.dim() == 4 and k_new.dim() == 4 and k_new.shape == v_new.shape, "bad q / k_new / v_new shapes")
    _require(k_pages.dim() == 4 and k_pages.shape == v_pages.shape, "bad page pool shapes")
    B, Hq, Tq, d = q.shape
    P, Hkv, page_size, dk = k_pages.shape
    _require(dk == d, "page pools and q disagree on d")
    _require(k_new.shape == (B, Hkv, Tq, d), "k_new and v_new must be [B, Hkv, Tq, d]")
    _require(block_table.dim() == 2 and block_table.shape[0] == B and block_table.dtype == torch.int32,
             "block_table must be int32 [B, W]")
    _require(seq_lens.shape == (B,) and seq_lens.dtype == torch.int32, "seq_lens must be int32 [B]")
    for n, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_pages", k_pages), ("v_pages", v_pages),
                 ("block_table", block_table), ("seq_lens", seq_lens)):
        _dense_on_gpu(n, t)
    _require(q.dtype == k_new.dtype == v_new.dtype == k_pages.dtype == v_pages.dtype,
             "q, k_new, v_new and the page pools must share a dtype")
    W = block_table.shape[1]
    with _alloc_stream(stream):
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device)
    _dense_on_gpu("out", out)
    _require(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    if lse is not False:
        _dense_on_gpu("lse", lse)
        _require(lse.shape == (B, Hq, Tq) and lse.dtype == torch.float32, "lse must be float32 [B, Hq, Tq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(load_library().attn_prefill_paged_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pages),
                                                    _ptr(v_pages), _ptr(block_table), _ptr(seq_lens), _ptr(out),
                                                    None if lse is False else _ptr(lse), B, Hq, Hkv, Tq, d,
                                                    page_size, P, W, float(scale), _dtype_code(q), _stream(stream)))
    return out, (None if lse is False else lse)


def attn_prefill_varlen(q, k, v, cu_seqlens, max_seqlen, out=None, lse=None, scale=None, stream=None):
    """Causal prefill of a ragged batch packed along tokens.  q [N,Hq,d], k/v [N,Hkv,d], cu_seqlens [S+1] int32
    (device), max_seqlen (host int) -> (out [N,Hq,d], lse fp32 [N,Hq])."""
    torch = _torch()
    _require(q.dim() == 3 and k.dim() == 3 and k.shape == v.shape, "q must be [N, Hq, d] and k, v [N, Hkv, d]")
    N, Hq, d = q.shape
    Hkv = k.shape[1]
    _require(k.shape[0] == N and k.shape[2] == d, "k/v shape mismatch")
    _require(cu_seqlens.dim() == 1 and cu_seqlens.numel() >= 1 and cu_seqlens.dtype == torch.int32,
             "cu_seqlens must be int32 [num_seqs + 1]")
    for n, t in (("q", q), ("k", k), ("v", v), ("cu_seqlens", cu_seqlens)):
        _dense_on_gpu(n, t)
    _require(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    with _alloc_stream(stream):
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((N, Hq), dtype=torch.float32, device=q.device)
    _dense_on_gpu("out", out)
    _require(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    if lse is not False:
        _dense_on_gpu("lse", lse)
        _require(lse.shape == (N, Hq) and lse.dtype == torch.float32, "lse must be float32 [N, Hq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(load_library().attn_prefill_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), None if lse is False else _ptr(lse),
                                              _ptr(cu_seqlens), cu_seqlens.numel() - 1, N, int(max_seqlen), Hq, Hkv,
                                              d, float(scale), _dtype_code(q), _stream(stream)))
    return out, (None if lse is False else lse)


def attn_kv_append(k_new, v_new, k_pages, v_pages, block_table, seq_lens, stream=None):
    """Write the last Tn tokens of each sequence into the paged cache, in place.  k_new/v_new [B,Hkv,Tn,d];
    pools [P,Hkv,page,d]; block_table [B,W] int32; seq_lens [B] int32 = lengths after the append (>= Tn)."""
    torch = _torch()
    _require(k_new.dim() == 4 and k_new.shape == v_new.shape, "k_new and v_new must be [B, Hkv, Tn, d]")
    _require(k_pages.dim() == 4 and k_pages.shape == v_pages.shape, "bad page pool shapes")
    B, Hkv, Tn, d = k_new.shape
    P, Hkv_p, page_size, dk = k_pages.shape
    _require(Hkv_p == Hkv and dk == d, "page pools and k_new disagree on Hkv or d")
    _require(block_table.dim() == 2 and block_table.shape[0] == B and block_table.dtype == torch.int32,
             "block_table must be int32 [B, W]")
    _require(seq_lens.shape == (B,) and seq_lens.dtype == torch.int32, "seq_lens must be int32 [B]")
    for n, t in (("k_new", k_new), ("v_new", v_new), ("k_pages", k_pages), ("v_pages", v_pages),
                 ("block_table", block_table), ("seq_lens", seq_lens)):
        _dense_on_gpu(n, t)
    _require(k_new.dtype == v_new.dtype == k_pages.dtype == v_pages.dtype, "k_new, v_new and the pools must share a dtype")
    _check(load_library().attn_kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                                         _ptr(seq_lens), B, Hkv, Tn, d, page_size, P, block_table.shape[1],
                                         _dtype_code(k_new), _stream(stream)))
    return k_pages, v_pages


def attn_decode_num_splits(B, Hq, Hkv, d, page_size, max_pages_per_seq, num_splits=0):
    s = load_library().attn_decode_num_splits(B, Hq, Hkv, d, page_size, max_pages_per_seq, num_splits)
    _check(min(s, 0))
    return s


def attn_decode_workspace_bytes(B, Hq, Hkv, d, page_size, max_pages_per_seq, num_splits=0):
    return load_library().attn_decode_workspace_bytes(B, Hq, Hkv, d, page_size, max_pages_per_seq, num_splits)


def attn_decode_paged(q, k_pages, v_pages, block_table, seq_lens, out=None, lse=None, scale=None, num_splits=0,
                      workspace=None, stream=None):
    """Paged single-token decode.  q [B,Hq,d]; pools [P,Hkv,page,d]; block_table [B,W] int32; seq_lens [B] int32."""
    torch = _torch()
    _require(q.dim() == 3 and k_pages.dim() == 4 and k_pages.shape == v_pages.shape, "bad q / page pool shapes")
    B, Hq, d = q.shape
    P, Hkv, page_size, dk = k_pages.shape
    _require(dk == d, "page pools and q disagree on d")
    _require(block_table.dim() == 2 and block_table.shape[0] == B and block_table.dtype == torch.int32,
             "block_table must be int32 [B, W]")
    _require(seq_lens.shape == (B,) and seq_lens.dtype == torch.int32, "seq_lens must be int32 [B]")
    for n, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages), ("block_table", block_table),
                 ("seq_lens", seq_lens)):
        _dense_on_gpu(n, t)
    _require(q.dtype == k_pages.dtype == v_pages.dtype, "q and the page pools must share a dtype")
    W = block_table.shape[1]
    with _alloc_stream(stream):
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _dense_on_gpu("out", out)
    _require(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    if lse is not False:
        _dense_on_gpu("lse", lse)
        _require(lse.shape == (B, Hq) and lse.dtype == torch.float32, "lse must be float32 [B, Hq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lib = load_library()
    need = lib.attn_decode_workspace_bytes(B, Hq, Hkv, d, page_size, W, num_splits)
    if workspace is None:
        with _alloc_stream(stream):
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dense_on_gpu("workspace", workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.attn_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seq_lens), _ptr(out),
                                 None if lse is False else _ptr(lse), B, Hq, Hkv, d, page_size, P, W, float(scale),
                                 _dtype_code(q), num_splits, _ptr(workspace), ws_bytes, _stream(stream)))
    return out, (None if lse is False else lse)


def attn_decode_paged_append(q, k_new, v_new, k_pages, v_pages, block_table, seq_lens, out=None, lse=None,
                             scale=None, num_splits=0, workspace=None, stream=None):
    """Paged single-token decode with the newest token's KV append fused.  q [B,Hq,d]; k_new/v_new [B,Hkv,d] or
    [B,Hkv,1,d] (written into the pools in place at position seq_lens[b] - 1); pools [P,Hkv,page,d]; block_table
    [B,W] int32; seq_lens [B] int32 = lengths after the append."""
    torch = _torch()
    _require(q.dim() == 3 and k_pages.dim() == 4 and k_pages.shape == v_pages.shape, "bad q / page pool shapes")
    B, Hq, d = q.shape
    P, Hkv, page_size, dk = k_pages.shape
    _require(dk == d, "page pools and q disagree on d")
    _require(k_new.shape == v_new.shape and tuple(k_new.shape) in ((B, Hkv, d), (B, Hkv, 1, d)),
             "k_new and v_new must be [B, Hkv, d] or [B, Hkv, 1, d]")
    _require(block_table.dim() == 2 and block_table.shape[0] == B and block_table.dtype == torch.int32,
             "block_table must be int32 [B, W]")
    _require(seq_lens.shape == (B,) and seq_lens.dtype == torch.int32, "seq_lens must be int32 [B]")
    for n, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_pages", k_pages), ("v_pages", v_pages),
                 ("block_table", block_table), ("seq_lens", seq_lens)):
        _dense_on_gpu(n, t)
    _require(q.dtype == k_new.dtype == v_new.dtype == k_pages.dtype == v_pages.dtype,
             "q, k_new, v_new and the page pools must share a dtype")
    W = block_table.shape[1]
    with _alloc_stream(stream):
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _dense_on_gpu("out", out)
    _require(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    if lse is not False:
        _dense_on_gpu("lse", lse)
        _require(lse.shape == (B, Hq) and lse.dtype == torch.float32, "lse must be float32 [B, Hq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lib = load_library()
    need = lib.attn_decode_workspace_bytes(B, Hq, Hkv, d, page_size, W, num_splits)
    if workspace is None:
        with _alloc_stream(stream):
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dense_on_gpu("workspace", workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.attn_decode_paged_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pages), _ptr(v_pages),
                                        _ptr(block_table), _ptr(seq_lens), _ptr(out),
                                        None if lse is False else _ptr(lse), B, Hq, Hkv, d, page_size, P, W,
                                        float(scale), _dtype_code(q), num_splits, _ptr(workspace), ws_bytes,
                                        _stream(stream)))
    return out, (None if lse is False else lse)


def attn_decode_paged_noalloc(q, k_pages, v_pages, block_table, seq_lens, out, lse=None, scale=None, num_splits=0,
                              stream=None):
    """attn_decode_paged without a workspace: the library's static per-GPU scratch serves instead, and nothing
    is allocated (the caller passes out, and lse or None to skip it).  Calls overlapping on one GPU race."""
    torch = _torch()
    _require(q.dim() == 3 and k_pages.dim() == 4 and k_pages.shape == v_pages.shape, "bad q / page pool shapes")
    B, Hq, d = q.shape
    P, Hkv, page_size, dk = k_pages.shape
    _require(dk == d, "page pools and q disagree on d")
    _require(block_table.dim() == 2 and block_table.shape[0] == B and block_table.dtype == torch.int32,
             "block_table must be int32 [B, W]")
    _require(seq_lens.shape == (B,) and seq_lens.dtype == torch.int32, "seq_lens must be int32 [B]")
    for n, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages), ("block_table", block_table),
                 ("seq_lens", seq_lens), ("out", out)):
        _dense_on_gpu(n, t)
    _require(q.dtype == k_pages.dtype == v_pages.dtype, "q and the page pools must share a dtype")
    _require(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    if lse is not None:
        _dense_on_gpu("lse", lse)
        _require(lse.shape == (B, Hq) and lse.dtype == torch.float32, "lse must be float32 [B, Hq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(load_library().attn_decode_paged_noalloc(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                                                    _ptr(seq_lens), _ptr(out), _ptr(lse), B, Hq, Hkv, d, page_size,
                                                    P, block_table.shape[1], float(scale), _dtype_code(q),
                                                    num_splits, _stream(stream)))
    return out, lse


def attn_decode_paged_fp8(q, k_pages, v_pages, k_scale, v_scale, block_table, seq_lens, out=None, lse=None,
                          scale=None, num_splits=0, workspace=None, stream=None):
    """Paged single-token decode over an FP8 E4M3 cache.  q [B,Hq,d] bf16; pools [P,Hkv,page,d] uint8 codes
    (or torch.float8_e4m3fn); key = code value * k_scale, value = code value * v_scale."""
    torch = _torch()
    _require(q.dim() == 3 and k_pages.dim() == 4 and k_pages.shape == v_pages.shape, "bad q / page pool shapes")
    B, Hq, d = q.shape
    P, Hkv, page_size, dk = k_pages.shape
    _require(dk == d, "page pools and q disagree on d")
    fp8 = getattr(torch, "float8_e4m3fn", None)
    _require(k_pages.dtype in (torch.uint8, fp8) and v_pages.dtype in (torch.uint8, fp8),
             "FP8 pools must be uint8 codes or float8_e4m3fn")
    _require(q.dtype == torch.bfloat16, "q must be bfloat16")
    _require(block_table.dim() == 2 and block_table.shape[0] == B and block_table.dtype == torch.int32,
             "block_table must be int32 [B, W]")
    _require(seq_lens.shape == (B,) and seq_lens.dtype == torch.int32, "seq_lens must be int32 [B]")
    for n, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages), ("block_table", block_table),
                 ("seq_lens", seq_lens)):
        _dense_on_gpu(n, t)
    W = block_table.shape[1]
    with _alloc_stream(stream):
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _dense_on_gpu("out", out)
    _require(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    if lse is not False:
        _dense_on_gpu("lse", lse)
        _require(lse.shape == (B, Hq) and lse.dtype == torch.float32, "lse must be float32 [B, Hq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lib = load_library()
    need = lib.attn_decode_workspace_bytes(B, Hq, Hkv, d, page_size, W, num_splits)
    if workspace is None:
        with _alloc_stream(stream):
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dense_on_gpu("workspace", workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.attn_decode_paged_fp8(_ptr(q), _ptr(k_pages), _ptr(v_pages), float(k_scale), float(v_scale),
                                     _ptr(block_table), _ptr(seq_lens), _ptr(out), None if lse is False else _ptr(lse),
                                     B, Hq, Hkv, d, page_size, P, W, float(scale), num_splits, _ptr(workspace),
                                     ws_bytes, _stream(stream)))
    return out, (None if lse is False else lse)


def attn_validate_paged_metadata(block_table, seq_lens, page_size, num_pages):
    """Host check of paged metadata (CPU int32 tensors or arrays); raises AttnError if out of contract."""
    import numpy as np

    bt = np.ascontiguousarray(np.asarray(block_table.cpu() if hasattr(block_table, "cpu") else block_table,
                                         dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(seq_lens.cpu() if hasattr(seq_lens, "cpu") else seq_lens, dtype=np.int32))
    B, W = bt.shape
    _check(load_library().attn_validate_paged_metadata(bt.ctypes.data, sl.ctypes.data, B, W, page_size, num_pages))


def attn_validate_chunk_metadata(block_table, seq_lens, page_size, num_pages, chunk_len):
    """attn_validate_paged_metadata plus seq_lens >= chunk_len (host copies); raises AttnError if out of contract."""
    import numpy as np

    bt = np.ascontiguousarray(np.asarray(block_table.cpu() if hasattr(block_table, "cpu") else block_table,
                                         dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(seq_lens.cpu() if hasattr(seq_lens, "cpu") else seq_lens, dtype=np.int32))
    B, W = bt.shape
    _check(load_library().attn_validate_chunk_metadata(bt.ctypes.data, sl.ctypes.data, B, W, page_size, num_pages,
                                                       chunk_len))


def attn_validate_varlen_metadata(cu_seqlens, total_tokens, max_seqlen):
    """Host check of cu_seqlens (CPU int32 tensor or array) for attn_prefill_varlen; raises AttnError."""
    import numpy as np

    cu = np.ascontiguousarray(np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
                                         dtype=np.int32))
    _check(load_library().attn_validate_varlen_metadata(cu.ctypes.data, cu.size - 1, total_tokens, max_seqlen))
