"""fp64 reference attention: causal prefill and paged single-token decode.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Definition followed (the pages name the operation but print no formula, so
the plainest reading of "causal multi-head / grouped-query scaled-dot-product
attention" is written out; every reading is listed with its reason in the
design notes of the repository):

  for query head h of batch b, with kv head  kv = floor(h / g),  g = Hq / Hkv
  (GQA as in the microLLM-rocm README, "Why this project exists": decoder-only
  MHA/GQA causal attention; consecutive query heads share one kv head),

      s_ij   = scale * <q_i, k_j>          for every visible key j
      m_i    = max_j s_ij
      p_ij   = exp(s_ij - m_i)             (max subtracted: same value, no overflow)
      l_i    = sum_j p_ij
      out_i  = sum_j (p_ij / l_i) v_j
      lse_i  = m_i + ln l_i                (natural log, scale included)

  Prefill: T queries against the same T keys; query i sees keys 0..i
  inclusive (the causal mask).  The score matrix is materialised in full and
  the masked entries set to -inf before the row softmax: the "naive" backend
  of the RoseLLM README ("Systems highlights", "Inference and serving") and
  the Softmax / ScaledDotProductAttention primitives of the llm-from-scratch
  "Project Overview" page ("Core Stack: llm/").

  Chunked prefill over a paged cache: the last Tq tokens of each sequence
  (a chunk of a long prompt processed after its prefix) attend over the
  sequence's L = seq_lens[b] cached tokens, their own K/V already appended.
  Query i of the chunk stands at position L - Tq + i and sees keys
  0..L - Tq + i: the causal mask aligned to the bottom-right corner of the
  Tq x L score block (RoseLLM README, "Systems highlights", "Inference and
  serving": chunked prefill and prefix reuse over the paged cache).  Decode
  is the case Tq = 1; a chunk that is the whole sequence (L = Tq) is the
  dense prefill above.

  Ragged (varlen) batched prefill: several sequences of different lengths
  packed token after token in one tensor, sequence s holding tokens
  cu_seqlens[s] .. cu_seqlens[s+1]-1; each is an independent causal prefill
  (no token sees another sequence) (ragged / varlen prefill of the
  RoseLLM README, "Systems highlights", "Inference and serving").

  Paged decode: one query per sequence, standing at position L-1 of a
  sequence of L = seq_lens[b] cached tokens, so it sees keys 0..L-1 (its own
  K/V already appended).  Token j lives in physical page
  block_table[b][j // page_size], slot j % page_size: the paged KV cache of
  the RoseLLM README ("What is inside"; "Systems highlights", "Inference and
  serving") and the mapped KV store of the microLLM-rocm README ("Why this
  project exists").  Slots at or past L are never read.  L == 0 has no
  visible key: the sum is empty, so lse = ln 0 = -inf, and out is defined
  as 0.

  Fused KV append (RoseLLM README, "Systems highlights", "Inference and
  serving"): the append of a chunk's keys and values (or of each sequence's
  newest token) composed with the chunked prefill (or the decode) that
  follows it, the two steps in that order: prefill_paged_append,
  decode_paged_append.

Arithmetic is NumPy float64 throughout.  Inputs may be any real dtype; bf16
tensors must be converted by the caller (exactly, via float32) before they
arrive here.
"""

import numpy as np


def kv_head_of(h, Hq, Hkv):
    """kv head read by query head ``h``: consecutive groups of g = Hq/Hkv."""
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    return h // (Hq // Hkv)


def _attend(qrows, keys, vals, scale, visible):
    """Softmax attention of R query rows over N keys, scores materialised.

    qrows [R, d], keys [N, d], vals [N, dv]; visible: bool [R, N], every row
    with at least one True.  Returns (out [R, dv], lse [R]).
    """
    s = scale * (qrows @ keys.T)
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    out = (e @ vals) / l
    lse = m[:, 0] + np.log(l[:, 0])
    return out, lse


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def _check_prefill(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, T, d]")
    B, Hq, T, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != T or k.shape[3] != d:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    kv_head_of(0, Hq, k.shape[1])
    return B, Hq, k.shape[1], T, d


def prefill(q, k, v, scale):
    """Causal prefill.  q [B,Hq,T,d], k/v [B,Hkv,T,d] -> (out [B,Hq,T,d], lse [B,Hq,T])."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, Hq, Hkv, T, d = _check_prefill(q, k, v)
    scale = float(scale)
    visible = np.tril(np.ones((T, T), dtype=bool), k=0)
    out = np.zeros((B, Hq, T, d))
    lse = np.zeros((B, Hq, T))
    if T == 0:
        return out, lse
    for b in range(B):
        for h in range(Hq):
            kv = kv_head_of(h, Hq, Hkv)
            out[b, h], lse[b, h] = _attend(q[b, h], k[b, kv], v[b, kv], scale, visible)
    return out, lse


def prefill_rows(q, k, v, scale, b, h, rows):
    """Selected causal-prefill rows of one (b, h), each row computed on its own.

    Row i attends over keys 0..i only, so only the keys a row can see are
    touched; used to check outputs sampled from shapes too large for
    ``prefill``.  Returns (out [len(rows), d], lse [len(rows)]).
    """
    Hq, Hkv = q.shape[1], k.shape[1]
    kv = kv_head_of(h, Hq, Hkv)
    outs, lses = [], []
    for i in rows:
        i = int(i)
        qi = _as64(q[b, h, i : i + 1])
        ks = _as64(k[b, kv, : i + 1])
        vs = _as64(v[b, kv, : i + 1])
        o, s = _attend(qi, ks, vs, float(scale), np.ones((1, i + 1), dtype=bool))
        outs.append(o[0])
        lses.append(s[0])
    d = q.shape[3]
    return np.array(outs).reshape(len(outs), d), np.array(lses)


def gather_pages(pages, table_row, L, page_size, kvh):
    """Tokens 0..L-1 of one sequence and kv head, read through its block table.

    pages [num_pages, Hkv, page_size, d]; table_row [max_pages_per_seq].
    """
    j = np.arange(L)
    page_ids = np.asarray(table_row)[j // page_size]
    slots = j % page_size
    if np.any(page_ids < 0) or np.any(page_ids >= pages.shape[0]):
        raise ValueError("block table names a page outside the pool")
    return _as64(pages[page_ids, kvh, slots])


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale, page_size):
    """Single-token decode over a paged KV cache.

    q [B,Hq,d]; k_pages/v_pages [num_pages,Hkv,page_size,d];
    block_table [B, W] int; seq_lens [B] int.  Returns (out [B,Hq,d], lse [B,Hq]).
    """
    q = _as64(q)
    B, Hq, d = q.shape
    Hkv = k_pages.shape[1]
    if k_pages.shape != v_pages.shape or k_pages.shape[2] != page_size or k_pages.shape[3] != d:
        raise ValueError("page pools must be [num_pages, Hkv, page_size, d]")
    bt = np.asarray(block_table)
    sl = np.asarray(seq_lens)
    if bt.shape[0] != B or sl.shape != (B,):
        raise ValueError("block_table must be [B, W] and seq_lens [B]")
    kv_head_of(0, Hq, Hkv)
    out = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        L = int(sl[b])
        if L < 0 or L > bt.shape[1] * page_size:
            raise ValueError(f"seq_lens[{b}]={L} outside [0, W*page_size]")
        if L == 0:
            continue
        for h in range(Hq):
            kv = kv_head_of(h, Hq, Hkv)
            keys = gather_pages(k_pages, bt[b], L, page_size, kv)
            vals = gather_pages(v_pages, bt[b], L, page_size, kv)
            o, s = _attend(q[b, h][None, :], keys, vals, float(scale), np.ones((1, L), dtype=bool))
            out[b, h], lse[b, h] = o[0], s[0]
    return out, lse


def prefill_paged(q, k_pages, v_pages, block_table, seq_lens, scale, page_size, rows=None):
    """Chunked causal prefill over a paged KV cache (bottom-right aligned mask).

    q [B,Hq,Tq,d]; k_pages/v_pages [num_pages,Hkv,page_size,d]; block_table
    [B, W] int; seq_lens [B] int with Tq <= seq_lens[b] <= W * page_size.
    Query i of sequence b sees keys 0..seq_lens[b] - Tq + i.  ``rows``, if
    given, lists the chunk rows to compute (the others are left 0 / -inf).
    Returns (out [B,Hq,Tq,d], lse [B,Hq,Tq]).
    """
    q = _as64(q)
    if q.ndim != 4:
        raise ValueError("q must be [B, Hq, Tq, d]")
    B, Hq, Tq, d = q.shape
    Hkv = k_pages.shape[1]
    if k_pages.shape != v_pages.shape or k_pages.shape[2] != page_size or k_pages.shape[3] != d:
        raise ValueError("page pools must be [num_pages, Hkv, page_size, d]")
    bt = np.asarray(block_table)
    sl = np.asarray(seq_lens)
    if bt.shape[0] != B or sl.shape != (B,):
        raise ValueError("block_table must be [B, W] and seq_lens [B]")
    kv_head_of(0, Hq, Hkv)
    rows = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((B, Hq, Tq, d))
    lse = np.full((B, Hq, Tq), -np.inf)
    if Tq == 0 or rows.size == 0:
        return out, lse
    for b in range(B):
        ctx = int(sl[b])
        if ctx < Tq or ctx > bt.shape[1] * page_size:
            raise ValueError(f"seq_lens[{b}]={ctx} outside [Tq={Tq}, W*page_size]")
        pos = ctx - Tq + rows                     # position of each computed query
        visible = np.arange(ctx)[None, :] <= pos[:, None]
        for h in range(Hq):
            kvh = kv_head_of(h, Hq, Hkv)
            keys = gather_pages(k_pages, bt[b], ctx, page_size, kvh)
            vals = gather_pages(v_pages, bt[b], ctx, page_size, kvh)
            o, s = _attend(q[b, h, rows], keys, vals, float(scale), visible)
            out[b, h, rows], lse[b, h, rows] = o, s
    return out, lse


def kv_append(k_pages, v_pages, k_new, v_new, block_table, seq_lens, page_size):
    """Write the newest tokens' keys and values into their paged-cache slots.

    The cache write that precedes attention over a paged cache (the KV-cache
    writer of the RoseLLM README, "Systems highlights", "Inference and
    serving").  k_new/v_new [B, Hkv, Tn, d] are the last Tn tokens of each
    sequence, whose length after the append is seq_lens[b] (>= Tn): token t
    goes to position seq_lens[b] - Tn + t, i.e. slot position % page_size of
    page block_table[b][position // page_size], for every kv head.  Returns
    new pools (copies); every other slot keeps its value.  Values are copied
    unchanged (no arithmetic).
    """
    k_out = np.array(k_pages, copy=True)
    v_out = np.array(v_pages, copy=True)
    B, Hkv, Tn, d = np.shape(k_new)
    bt = np.asarray(block_table)
    sl = np.asarray(seq_lens)
    if np.shape(v_new) != (B, Hkv, Tn, d) or k_out.shape[1:] != (Hkv, page_size, d):
        raise ValueError("k_new/v_new must be [B, Hkv, Tn, d] and the pools [P, Hkv, page_size, d]")
    for b in range(B):
        total = int(sl[b])
        if total < Tn or total > bt.shape[1] * page_size:
            raise ValueError(f"seq_lens[{b}]={total} outside [Tn={Tn}, W*page_size]")
        for t in range(Tn):
            position = total - Tn + t
            page = int(bt[b, position // page_size])
            if page < 0 or page >= k_out.shape[0]:
                raise ValueError("block table names a page outside the pool")
            k_out[page, :, position % page_size] = np.asarray(k_new)[b, :, t]
            v_out[page, :, position % page_size] = np.asarray(v_new)[b, :, t]
    return k_out, v_out


def prefill_paged_append(q, k_new, v_new, k_pages, v_pages, block_table, seq_lens, scale, page_size, rows=None):
    """KV append of a chunk followed by the chunked prefill of its queries.

    The step of a chunked prefill in a paged-cache server (RoseLLM README,
    "Systems highlights", "Inference and serving": the KV-cache writer, then
    chunked prefill over the paged cache): the chunk's keys and values
    k_new / v_new [B, Hkv, Tq, d] are written into their slots (kv_append),
    then the chunk's queries q [B, Hq, Tq, d] attend over the updated cache
    (prefill_paged).  Returns (out, lse, k_pages after, v_pages after).
    """
    k_after, v_after = kv_append(k_pages, v_pages, k_new, v_new, block_table, seq_lens, page_size)
    out, lse = prefill_paged(q, k_after, v_after, block_table, seq_lens, scale, page_size, rows=rows)
    return out, lse, k_after, v_after


def decode_paged_append(q, k_new, v_new, k_pages, v_pages, block_table, seq_lens, scale, page_size):
    """KV append of each sequence's newest token followed by the paged decode.

    The decode step of a paged-cache server (RoseLLM README, "Systems
    highlights", "Inference and serving": the KV-cache writer, then decode
    over the paged cache): k_new / v_new [B, Hkv, d] (or [B, Hkv, 1, d]) are
    written at position seq_lens[b] - 1 (kv_append with one token), then the
    query of each sequence attends over its seq_lens[b] cached tokens
    (decode_paged).  A sequence with seq_lens[b] = 0 appends nothing.
    Returns (out, lse, k_pages after, v_pages after).
    """
    B = np.shape(q)[0]
    kn = np.asarray(k_new).reshape(B, -1, 1, np.shape(k_new)[-1])
    vn = np.asarray(v_new).reshape(B, -1, 1, np.shape(v_new)[-1])
    sl = np.asarray(seq_lens)
    some = np.nonzero(sl > 0)[0]
    k_after, v_after = kv_append(k_pages, v_pages, kn[some], vn[some], np.asarray(block_table)[some], sl[some],
                                 page_size)
    out, lse = decode_paged(q, k_after, v_after, block_table, seq_lens, scale, page_size)
    return out, lse, k_after, v_after


def prefill_varlen(q, k, v, cu_seqlens, scale):
    """Causal prefill of a ragged batch packed along the token axis.

    q [N, Hq, d], k/v [N, Hkv, d] with N = cu_seqlens[-1]; cu_seqlens [S+1]
    non-decreasing from 0.  Token i of sequence s (packed index
    cu_seqlens[s] + i) sees keys cu_seqlens[s] .. cu_seqlens[s] + i.
    Returns (out [N, Hq, d], lse [N, Hq]).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if q.ndim != 3 or k.ndim != 3 or k.shape != v.shape or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]:
        raise ValueError("q must be [N, Hq, d] and k, v [N, Hkv, d]")
    N, Hq, d = q.shape
    Hkv = k.shape[1]
    kv_head_of(0, Hq, Hkv)
    if cu.ndim != 1 or cu.size < 1 or cu[0] != 0 or cu[-1] != N or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must rise from 0 to N")
    out = np.zeros((N, Hq, d))
    lse = np.zeros((N, Hq))
    for s in range(cu.size - 1):
        first, last = int(cu[s]), int(cu[s + 1])
        n = last - first
        if n == 0:
            continue
        seen = np.tril(np.ones((n, n), dtype=bool))
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            o, l = _attend(q[first:last, h], k[first:last, g], v[first:last, g], float(scale), seen)
            out[first:last, h], lse[first:last, h] = o, l
    return out, lse


def fp8_e4m3_value(codes):
    """Real value of FP8 E4M3 codes (the OCP 8-bit float, finite-only form).

    Bit 7 is the sign, bits 6..3 the exponent (bias 7), bits 2..0 the
    mantissa.  Exponent 0 holds subnormals m/8 * 2^-6; codes with all
    exponent and mantissa bits set (0x7F, 0xFF) are NaN; there is no
    infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


def decode_paged_fp8(q, k_codes, v_codes, k_scale, v_scale, block_table, seq_lens, scale, page_size):
    """Single-token decode over a paged cache whose keys and values are FP8 E4M3.

    The cache stores codes [num_pages, Hkv, page_size, d] with one scale per
    tensor: key = fp8_e4m3_value(code) * k_scale, likewise for values (the
    FP8 KV cache of the microLLM-rocm README, "Why this project exists", on
    MI300X; gfx950's FP8 formats).  The result is decode_paged over those
    real values.
    """
    keys = fp8_e4m3_value(k_codes) * float(k_scale)
    vals = fp8_e4m3_value(v_codes) * float(v_scale)
    return decode_paged(q, keys, vals, block_table, seq_lens, scale, page_size)
