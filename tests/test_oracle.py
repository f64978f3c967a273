"""Pins for the fp64 oracle, checked against facts that do not come from the oracle.

Each pin rests on something the oracle does not compute itself: a closed form
derived by hand (``tests/golden``), an invariant of softmax attention, an
independent library routine (torch's scaled_dot_product_attention in float64
on the CPU) or a 50-digit brute force with mpmath.  The pin table:

  p1  q = 0 (or scale = 0): out_i is the causal prefix mean of V of the head's
      kv head, lse_i = ln(i + 1)                          -> mask, normalisation,
                                                             head mapping, LSE base
  p2  T = 1: out = v_0, lse = scale * q_0 . k_0           -> scale placement
  p3  decode with L = t + 1 cached tokens == prefill row t -> decode alignment, gather
  p4  a different physical page order leaves decode bit-identical -> indirection
  p5  torch SDPA (float64, CPU, is_causal, enable_gqa) on Tq = Tk  -> whole prefill
  p6  GQA == MHA with K, V repeated per group             -> head mapping
  p7  K + 1u^T: same out, lse + scale q.u;  V + 1c^T: out + c;  out linear in V
  p8  changing K/V past position i leaves rows <= i bit-identical -> causality
  p9  mpmath brute force at 50 digits on tiny inputs      -> the oracle's own rounding
  golden: hand-derived closed forms (log keys, GQA prefix mean, paged read-back)
"""

import math
import os
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


def gqa_case(seed, B=2, Hq=4, Hkv=2, T=9, d=5):
    r = rng(seed)
    q = r.standard_normal((B, Hq, T, d))
    k = r.standard_normal((B, Hkv, T, d))
    v = r.standard_normal((B, Hkv, T, d))
    return q, k, v


def paged_copy(k, v, L, page_size, seed, extra_pages=0):
    """Scatter dense K/V [Hkv, T, d] tokens 0..L-1 into a shuffled NaN-filled pool."""
    Hkv, T, d = k.shape
    n = -(-L // page_size)
    P = n + extra_pages
    r = rng(seed)
    perm = r.permutation(P)
    W = -(-T // page_size)
    table = np.full(W, -1, dtype=np.int64)
    table[:n] = perm[:n]
    kp = np.full((P, Hkv, page_size, d), np.nan)
    vp = np.full((P, Hkv, page_size, d), np.nan)
    for j in range(L):
        kp[table[j // page_size], :, j % page_size] = k[:, j]
        vp[table[j // page_size], :, j % page_size] = v[:, j]
    return kp, vp, table


# ---------------------------------------------------------------- p1: q = 0
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (8, 2), (6, 1)])
def test_p1_zero_query_is_prefix_mean(Hq, Hkv):
    _, k, v = gqa_case(1, Hq=Hq, Hkv=Hkv)
    q = np.zeros((2, Hq, 9, 5))
    out, lse = oracle.prefill(q, k, v, scale=0.7)
    g = Hq // Hkv
    for b in range(2):
        for h in range(Hq):
            c = h // g
            for i in range(9):
                np.testing.assert_allclose(out[b, h, i], v[b, c, : i + 1].mean(axis=0), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(np.arange(1, 10)), lse.shape), rtol=0, atol=1e-14)


def test_p1_zero_scale_is_prefix_mean():
    q, k, v = gqa_case(2)
    out, lse = oracle.prefill(q, k, v, scale=0.0)
    csum = np.cumsum(v, axis=2) / np.arange(1, 10)[None, None, :, None]
    np.testing.assert_allclose(out, np.repeat(csum, 2, axis=1), atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, 10)), atol=1e-14)


def test_p1_zero_query_decode():
    _, k, v = gqa_case(3, B=1, T=40)
    for L in (1, 17, 40):
        kp, vp, table = paged_copy(k[0], v[0], L, 16, seed=L)
        out, lse = oracle.decode_paged(np.zeros((1, 4, 5)), kp, vp, table[None], np.array([L]), 1.3, 16)
        for h in range(4):
            np.testing.assert_allclose(out[0, h], v[0, h // 2, :L].mean(axis=0), atol=1e-14)
        np.testing.assert_allclose(lse[0], math.log(L), atol=1e-14)


# ---------------------------------------------------------------- p2: T = 1
def test_p2_single_token():
    q, k, v = gqa_case(4, T=1, d=7)
    out, lse = oracle.prefill(q, k, v, scale=0.37)
    for b in range(2):
        for h in range(4):
            np.testing.assert_array_equal(out[b, h, 0], v[b, h // 2, 0])
            dot = math.fsum(float(x) * float(y) for x, y in zip(q[b, h, 0], k[b, h // 2, 0]))
            assert abs(lse[b, h, 0] - 0.37 * dot) < 1e-14


# ---------------------------------------------------------------- p3: decode == prefill row
@pytest.mark.parametrize("page_size", [1, 4, 16])
def test_p3_decode_equals_prefill_row(page_size):
    q, k, v = gqa_case(5, B=2, Hq=8, Hkv=2, T=37, d=6)
    out_p, lse_p = oracle.prefill(q, k, v, 0.41)
    for b in range(2):
        for t in (0, 1, 15, 16, 17, 36):
            L = t + 1
            kp, vp, table = paged_copy(k[b], v[b], L, page_size, seed=100 + t, extra_pages=3)
            out_d, lse_d = oracle.decode_paged(q[b : b + 1, :, t], kp, vp, table[None], np.array([L]), 0.41, page_size)
            np.testing.assert_allclose(out_d[0], out_p[b, :, t], rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse_d[0], lse_p[b, :, t], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- p4: page permutation
def test_p4_page_permutation_is_bit_identical():
    r = rng(6)
    B, Hq, Hkv, d, ps = 3, 4, 2, 8, 16
    L = np.array([5, 33, 64])
    W = 4
    P = int(sum(-(-x // ps) for x in L)) + 2
    kp = r.standard_normal((P, Hkv, ps, d))
    vp = r.standard_normal((P, Hkv, ps, d))
    perm = r.permutation(P)
    table = np.full((B, W), -1)
    off = 0
    for b in range(B):
        n = -(-L[b] // ps)
        table[b, :n] = perm[off : off + n]
        off += n
    q = r.standard_normal((B, Hq, d))
    out1, lse1 = oracle.decode_paged(q, kp, vp, table, L, 0.3, ps)
    new = r.permutation(P)  # old page i moves to new[i]
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[new] = kp
    vp2[new] = vp
    table2 = np.where(table >= 0, new[np.maximum(table, 0)], -1)
    out2, lse2 = oracle.decode_paged(q, kp2, vp2, table2, L, 0.3, ps)
    np.testing.assert_array_equal(out1, out2)
    np.testing.assert_array_equal(lse1, lse2)
    assert not np.array_equal(table, table2)


# ---------------------------------------------------------------- p5: library routine
@pytest.mark.parametrize("B,Hq,Hkv,T,d", [(1, 1, 1, 1, 3), (2, 4, 4, 7, 5), (1, 8, 2, 33, 16), (2, 6, 3, 64, 8)])
def test_p5_matches_torch_sdpa_float64(B, Hq, Hkv, T, d):
    q, k, v = gqa_case(7 + T, B=B, Hq=Hq, Hkv=Hkv, T=T, d=d)
    scale = 0.29
    out, _ = oracle.prefill(q, k, v, scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=True, scale=scale, enable_gqa=True,
    ).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)


def test_p5_prefill_rows_matches_prefill():
    q, k, v = gqa_case(8, T=20)
    out, lse = oracle.prefill(q, k, v, 0.5)
    rows = [0, 3, 19]
    o, s = oracle.prefill_rows(q, k, v, 0.5, 1, 3, rows)
    np.testing.assert_allclose(o, out[1, 3, rows], atol=1e-14)
    np.testing.assert_allclose(s, lse[1, 3, rows], atol=1e-14)


# ---------------------------------------------------------------- p6: GQA == MHA with repeats
def test_p6_gqa_equals_repeated_mha():
    q, k, v = gqa_case(9, Hq=8, Hkv=2)
    out, lse = oracle.prefill(q, k, v, 0.6)
    out2, lse2 = oracle.prefill(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.6)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_p6_head_groups_are_consecutive():
    # Distinct V per kv head: head h must read kv head h // g, not h % Hkv.
    q, k, v = gqa_case(10, Hq=4, Hkv=2)
    v[:, 1] += 1000.0
    out, _ = oracle.prefill(q, k, v, 0.6)
    assert np.all(out[:, :2] < 100) and np.all(out[:, 2:] > 900)


# ---------------------------------------------------------------- p7: shift invariance, linearity
def test_p7_shift_and_linearity():
    q, k, v = gqa_case(11, T=12)
    scale = 0.45
    out, lse = oracle.prefill(q, k, v, scale)
    u = rng(12).standard_normal(5)
    out_k, lse_k = oracle.prefill(q, k + u, v, scale)
    np.testing.assert_allclose(out_k, out, atol=1e-12)
    shift = scale * np.einsum("bhtd,d->bht", q, u)
    np.testing.assert_allclose(lse_k, lse + shift, atol=1e-12)
    c = rng(13).standard_normal(5)
    out_v, lse_v = oracle.prefill(q, k, v + c, scale)
    np.testing.assert_allclose(out_v, out + c, atol=1e-12)
    np.testing.assert_array_equal(lse_v, lse)
    v2 = rng(14).standard_normal(v.shape)
    out_2, _ = oracle.prefill(q, k, v2, scale)
    out_lin, _ = oracle.prefill(q, k, 2.0 * v - 3.0 * v2, scale)
    np.testing.assert_allclose(out_lin, 2.0 * out - 3.0 * out_2, atol=1e-12)


# ---------------------------------------------------------------- p8: causality
def test_p8_future_keys_do_not_leak():
    q, k, v = gqa_case(15, T=16)
    out, lse = oracle.prefill(q, k, v, 0.5)
    for i in (0, 7, 14):
        k2, v2 = k.copy(), v.copy()
        # Finite changes: prefill inputs are real tokens, never NaN (NaN
        # poisoning applies to the unused slots of a paged cache, which the
        # decode path never reads; see test_decode_* and the golden pages).
        k2[:, :, i + 1 :] = 1e3
        v2[:, :, i + 1 :] = -7e5
        out2, lse2 = oracle.prefill(q, k2, v2, 0.5)
        np.testing.assert_array_equal(out2[:, :, : i + 1], out[:, :, : i + 1])
        np.testing.assert_array_equal(lse2[:, :, : i + 1], lse[:, :, : i + 1])


# ---------------------------------------------------------------- p9: 50-digit brute force
def _mp_attention_row(qi, keys, vals, scale):
    mpmath.mp.dps = 50
    s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(b) for a, b in zip(qi, kj)) for kj in keys]
    w = [mpmath.exp(x) for x in s]
    tot = mpmath.fsum(w)
    out = [mpmath.fsum(wj * mpmath.mpf(vj[c]) for wj, vj in zip(w, vals)) / tot for c in range(len(vals[0]))]
    return [float(o) for o in out], float(mpmath.log(tot))


@pytest.mark.parametrize("seed", [16, 17, 18])
def test_p9_prefill_brute_force(seed):
    r = rng(seed)
    T, d = int(r.integers(1, 7)), int(r.integers(1, 5))
    q, k, v = gqa_case(seed, B=1, Hq=2, Hkv=1, T=T, d=d)
    q *= 3.0  # sharper softmax
    scale = float(np.float32(1.0 / math.sqrt(d)))
    out, lse = oracle.prefill(q, k, v, scale)
    for h in range(2):
        for i in range(T):
            o, s = _mp_attention_row(q[0, h, i], k[0, 0, : i + 1], v[0, 0, : i + 1], scale)
            np.testing.assert_allclose(out[0, h, i], o, rtol=0, atol=1e-14)
            assert abs(lse[0, h, i] - s) < 1e-13


def test_p9_decode_brute_force():
    r = rng(19)
    Hq, Hkv, d, ps = 4, 2, 3, 2
    L = np.array([1, 4, 7])
    P = int(sum(-(-x // ps) for x in L))
    kp = r.standard_normal((P, Hkv, ps, d))
    vp = r.standard_normal((P, Hkv, ps, d))
    perm = r.permutation(P)
    table = np.full((3, 4), -1)
    off = 0
    for b in range(3):
        n = -(-L[b] // ps)
        table[b, :n] = perm[off : off + n]
        off += n
    q = 2.0 * r.standard_normal((3, Hq, d))
    out, lse = oracle.decode_paged(q, kp, vp, table, L, 0.8, ps)
    for b in range(3):
        for h in range(Hq):
            keys = [kp[table[b, j // ps], h // 2, j % ps] for j in range(L[b])]
            vals = [vp[table[b, j // ps], h // 2, j % ps] for j in range(L[b])]
            o, s = _mp_attention_row(q[b, h], keys, vals, 0.8)
            np.testing.assert_allclose(out[b, h], o, rtol=0, atol=1e-14)
            assert abs(lse[b, h] - s) < 1e-13


# ---------------------------------------------------------------- chunked prefill over pages
def chunk_case(seed, Ls, Tq, Hq=4, Hkv=2, d=3, ps=4):
    """Dense K/V of len max(Ls) per sequence, scattered into one shuffled NaN pool; q for the chunk."""
    r = rng(seed)
    B, T = len(Ls), max(Ls)
    k = r.standard_normal((B, Hkv, T, d))
    v = r.standard_normal((B, Hkv, T, d))
    W = -(-T // ps)
    P = sum(-(-L // ps) for L in Ls)
    perm = r.permutation(P)
    table = np.full((B, W), -1)
    kp = np.full((P, Hkv, ps, d), np.nan)
    vp = np.full((P, Hkv, ps, d), np.nan)
    off = 0
    for b, L in enumerate(Ls):
        n = -(-L // ps)
        table[b, :n] = perm[off : off + n]
        off += n
        for j in range(L):
            kp[table[b, j // ps], :, j % ps] = k[b, :, j]
            vp[table[b, j // ps], :, j % ps] = v[b, :, j]
    q = 2.0 * r.standard_normal((B, Hq, Tq, d))
    return q, k, v, kp, vp, table, np.array(Ls), ps


def test_chunk_is_the_tail_of_a_dense_prefill():
    """Rows L-Tq..L-1 of a dense causal prefill over the whole sequence are the chunk's rows."""
    Ls, Tq = [7, 11, 5], 5
    q, k, v, kp, vp, table, L, ps = chunk_case(30, Ls, Tq)
    out, lse = oracle.prefill_paged(q, kp, vp, table, L, 0.7, ps)
    for b, Lb in enumerate(Ls):
        qd = np.zeros((1, q.shape[1], Lb, q.shape[3]))
        qd[0, :, Lb - Tq :] = q[b]
        od, ld = oracle.prefill(qd, k[b : b + 1, :, :Lb], v[b : b + 1, :, :Lb], 0.7)
        np.testing.assert_allclose(out[b], od[0, :, Lb - Tq :], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[b], ld[0, :, Lb - Tq :], rtol=0, atol=1e-13)


def test_chunk_of_one_token_is_decode():
    Ls = [1, 6, 9]
    q, k, v, kp, vp, table, L, ps = chunk_case(31, Ls, 1)
    out, lse = oracle.prefill_paged(q, kp, vp, table, L, 0.9, ps)
    od, ld = oracle.decode_paged(q[:, :, 0], kp, vp, table, L, 0.9, ps)
    np.testing.assert_allclose(out[:, :, 0], od, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[:, :, 0], ld, rtol=0, atol=1e-13)


def test_chunk_zero_query_is_prefix_mean():
    """q = 0: query i of sequence b averages v over keys 0..L_b-Tq+i; lse = ln(L_b-Tq+i+1)."""
    Ls, Tq = [6, 13], 4
    q, k, v, kp, vp, table, L, ps = chunk_case(32, Ls, Tq, Hq=4, Hkv=2)
    v[:, 1] += 5.0  # distinct values per kv head
    for b, Lb in enumerate(Ls):
        for j in range(Lb):
            vp[table[b, j // ps], :, j % ps] = v[b, :, j]
    out, lse = oracle.prefill_paged(np.zeros_like(q), kp, vp, table, L, 0.5, ps)
    for b, Lb in enumerate(Ls):
        for h in range(4):
            for i in range(Tq):
                p = Lb - Tq + i
                np.testing.assert_allclose(out[b, h, i], v[b, h // 2, : p + 1].mean(axis=0), rtol=0, atol=1e-13)
                assert abs(lse[b, h, i] - math.log(p + 1)) < 1e-13


def test_chunk_page_permutation_and_rows():
    Ls, Tq = [9, 14], 6
    q, k, v, kp, vp, table, L, ps = chunk_case(33, Ls, Tq)
    out, lse = oracle.prefill_paged(q, kp, vp, table, L, 0.6, ps)
    r = rng(34)
    perm = r.permutation(kp.shape[0])
    inv = np.argsort(perm)
    t2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1)
    out2, lse2 = oracle.prefill_paged(q, kp[inv], vp[inv], t2, L, 0.6, ps)
    np.testing.assert_array_equal(out2, out)
    np.testing.assert_array_equal(lse2, lse)
    rows = [0, 3, 5]
    out3, lse3 = oracle.prefill_paged(q, kp, vp, table, L, 0.6, ps, rows=rows)
    np.testing.assert_allclose(out3[:, :, rows], out[:, :, rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse3[:, :, rows], lse[:, :, rows], rtol=0, atol=1e-14)


def test_chunk_brute_force():
    Ls, Tq = [3, 5], 3
    q, k, v, kp, vp, table, L, ps = chunk_case(35, Ls, Tq, Hq=2, Hkv=1, d=2, ps=2)
    out, lse = oracle.prefill_paged(q, kp, vp, table, L, 0.8, ps)
    for b, Lb in enumerate(Ls):
        for h in range(2):
            for i in range(Tq):
                p = Lb - Tq + i
                o, s = _mp_attention_row(q[b, h, i], k[b, 0, : p + 1], v[b, 0, : p + 1], 0.8)
                np.testing.assert_allclose(out[b, h, i], o, rtol=0, atol=1e-14)
                assert abs(lse[b, h, i] - s) < 1e-13


# ---------------------------------------------------------------- KV append into the paged cache
def test_append_then_gather_returns_the_new_tokens():
    """Positions L-Tn..L-1 read back through the table are k_new / v_new; every other slot is untouched."""
    r = rng(40)
    ps, Hkv, d, Tn = 4, 3, 5, 6
    Ls = [6, 9, 17]
    W = 5
    P = sum(-(-L // ps) for L in Ls) + 2
    perm = r.permutation(P)
    table = np.full((3, W), -1)
    off = 0
    for b, L in enumerate(Ls):
        n = -(-L // ps)
        table[b, :n] = perm[off : off + n]
        off += n
    kp, vp = r.standard_normal((P, Hkv, ps, d)), r.standard_normal((P, Hkv, ps, d))
    kn, vn = r.standard_normal((3, Hkv, Tn, d)), r.standard_normal((3, Hkv, Tn, d))
    k2, v2 = oracle.kv_append(kp, vp, kn, vn, table, np.array(Ls), ps)
    written = np.zeros((P, ps), dtype=bool)
    for b, L in enumerate(Ls):
        for kvh in range(Hkv):
            np.testing.assert_array_equal(oracle.gather_pages(k2, table[b], L, ps, kvh)[L - Tn :], kn[b, kvh])
            np.testing.assert_array_equal(oracle.gather_pages(v2, table[b], L, ps, kvh)[L - Tn :], vn[b, kvh])
        for j in range(L - Tn, L):
            written[table[b, j // ps], j % ps] = True
    slots = lambda x: x.transpose(0, 2, 1, 3)  # [page, slot, kv head, d]
    np.testing.assert_array_equal(slots(k2)[~written], slots(kp)[~written])
    np.testing.assert_array_equal(slots(v2)[~written], slots(vp)[~written])


def test_append_then_decode_equals_dense_history():
    """Cache the first L-1 tokens densely, append the last one, decode: same as the prefill's last row."""
    q, k, v = gqa_case(41, B=1, Hq=4, Hkv=2, T=11, d=4)
    L, ps = 11, 4
    kp, vp, table = paged_copy(k[0], v[0], L - 1, ps, seed=42, extra_pages=1)
    if -(-L // ps) > -(-(L - 1) // ps):  # the new token opens a page: give it the spare one
        table[(L - 1) // ps] = kp.shape[0] - 1
    k2, v2 = oracle.kv_append(kp, vp, k[:, :, L - 1 : L], v[:, :, L - 1 : L], table[None], np.array([L]), ps)
    od, ld = oracle.decode_paged(q[:, :, L - 1], k2, v2, table[None], np.array([L]), 0.6, ps)
    op, lp = oracle.prefill(q, k, v, 0.6)
    np.testing.assert_allclose(od, op[:, :, L - 1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(ld, lp[:, :, L - 1], rtol=0, atol=1e-13)


def test_fused_chunks_rebuild_a_dense_prefill():
    """Start from an empty (NaN) cache and feed two sequences chunk by chunk through the fused append +
    chunked prefill: each chunk's rows are the matching rows of a dense causal prefill over the whole
    sequence, and the final cache holds every token's K/V."""
    r = rng(43)
    B, Hq, Hkv, d, ps, L = 2, 4, 2, 3, 4, 11
    q = 2.0 * r.standard_normal((B, Hq, L, d))
    k = r.standard_normal((B, Hkv, L, d))
    v = r.standard_normal((B, Hkv, L, d))
    W = -(-L // ps)
    P = B * W
    table = r.permutation(P).reshape(B, W)
    kp = np.full((P, Hkv, ps, d), np.nan)
    vp = np.full((P, Hkv, ps, d), np.nan)
    od, ld = oracle.prefill(q, k, v, 0.7)
    start = 0
    for Tq in (3, 4, 4):
        end = start + Tq
        out, lse, kp, vp = oracle.prefill_paged_append(q[:, :, start:end], k[:, :, start:end], v[:, :, start:end],
                                                       kp, vp, table, np.array([end] * B), 0.7, ps)
        np.testing.assert_allclose(out, od[:, :, start:end], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, ld[:, :, start:end], rtol=0, atol=1e-13)
        start = end
    for b in range(B):
        for kvh in range(Hkv):
            np.testing.assert_array_equal(oracle.gather_pages(kp, table[b], L, ps, kvh), k[b, kvh])
            np.testing.assert_array_equal(oracle.gather_pages(vp, table[b], L, ps, kvh), v[b, kvh])


def test_fused_decode_steps_rebuild_a_dense_prefill():
    """Decode two sequences token by token through the fused append + decode, from an empty (NaN) cache,
    the second starting three steps later (seq_lens 0 meanwhile: nothing appended, out 0, lse -inf): every
    step's output is the matching row of a dense causal prefill, and the final cache holds every token."""
    r = rng(44)
    B, Hq, Hkv, d, ps, T, lag = 2, 4, 2, 3, 4, 9, 3
    q = 2.0 * r.standard_normal((B, Hq, T, d))
    k = r.standard_normal((B, Hkv, T, d))
    v = r.standard_normal((B, Hkv, T, d))
    W = -(-T // ps)
    table = r.permutation(B * W).reshape(B, W)
    kp = np.full((B * W, Hkv, ps, d), np.nan)
    vp = np.full((B * W, Hkv, ps, d), np.nan)
    od, ld = oracle.prefill(q, k, v, 0.8)
    for t in range(T):
        L = np.array([t + 1, max(0, t + 1 - lag)])
        pos = np.maximum(L - 1, 0)
        qs = np.stack([q[b, :, pos[b]] for b in range(B)])
        kn = np.stack([k[b, :, pos[b]] if L[b] else np.full((Hkv, d), np.nan) for b in range(B)])
        vn = np.stack([v[b, :, pos[b]] if L[b] else np.full((Hkv, d), np.nan) for b in range(B)])
        out, lse, kp, vp = oracle.decode_paged_append(qs, kn, vn, kp, vp, table, L, 0.8, ps)
        for b in range(B):
            if L[b]:
                np.testing.assert_allclose(out[b], od[b, :, pos[b]], rtol=0, atol=1e-13)
                np.testing.assert_allclose(lse[b], ld[b, :, pos[b]], rtol=0, atol=1e-13)
            else:
                assert np.all(out[b] == 0) and np.all(lse[b] == -np.inf)
    for b, Lb in enumerate((T, T - lag)):
        for kvh in range(Hkv):
            np.testing.assert_array_equal(oracle.gather_pages(kp, table[b], Lb, ps, kvh), k[b, kvh, :Lb])
            np.testing.assert_array_equal(oracle.gather_pages(vp, table[b], Lb, ps, kvh), v[b, kvh, :Lb])


# ---------------------------------------------------------------- ragged (varlen) prefill
def varlen_case(seed, lens, Hq=4, Hkv=2, d=3):
    r = rng(seed)
    N = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    return r.standard_normal((N, Hq, d)) * 2.0, r.standard_normal((N, Hkv, d)), r.standard_normal((N, Hkv, d)), cu


def test_varlen_single_sequence_is_sdpa():
    """One packed sequence against torch's float64 SDPA (an independent library routine)."""
    q, k, v, cu = varlen_case(50, [9], Hq=4, Hkv=2, d=5)
    out, lse = oracle.prefill_varlen(q, k, v, cu, 0.45)
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=0.45, enable_gqa=True)
    np.testing.assert_allclose(out, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-13)


def test_varlen_sequences_do_not_see_each_other():
    """Changing one sequence's keys and values leaves every other sequence bitwise unchanged;
    the packed result equals each sequence computed alone (empty sequences included)."""
    lens = [5, 0, 8, 1, 6]
    q, k, v, cu = varlen_case(51, lens)
    out, lse = oracle.prefill_varlen(q, k, v, cu, 0.7)
    k2, v2 = k.copy(), v.copy()
    k2[cu[2] : cu[3]] += 3.0
    v2[cu[2] : cu[3]] -= 1.0
    out2, lse2 = oracle.prefill_varlen(q, k2, v2, cu, 0.7)
    other = np.ones(q.shape[0], dtype=bool)
    other[cu[2] : cu[3]] = False
    np.testing.assert_array_equal(out2[other], out[other])
    np.testing.assert_array_equal(lse2[other], lse[other])
    assert not np.allclose(out2[~other], out[~other])
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        o1, l1 = oracle.prefill_varlen(q[a:b], k[a:b], v[a:b], np.array([0, b - a]), 0.7)
        np.testing.assert_allclose(out[a:b], o1, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[a:b], l1, rtol=0, atol=1e-13)


def test_varlen_zero_query_is_prefix_mean():
    lens = [3, 7]
    q, k, v, cu = varlen_case(52, lens, Hq=4, Hkv=2)
    v[:, 1] += 4.0
    out, lse = oracle.prefill_varlen(np.zeros_like(q), k, v, cu, 0.9)
    for s in range(2):
        for i in range(lens[s]):
            t = cu[s] + i
            for h in range(4):
                np.testing.assert_allclose(out[t, h], v[cu[s] : t + 1, h // 2].mean(axis=0), rtol=0, atol=1e-13)
                assert abs(lse[t, h] - math.log(i + 1)) < 1e-13


def test_varlen_brute_force():
    lens = [2, 4]
    q, k, v, cu = varlen_case(53, lens, Hq=2, Hkv=1, d=2)
    out, lse = oracle.prefill_varlen(q, k, v, cu, 0.8)
    for s in range(2):
        for i in range(lens[s]):
            t = cu[s] + i
            for h in range(2):
                o, l = _mp_attention_row(q[t, h], k[cu[s] : t + 1, 0], v[cu[s] : t + 1, 0], 0.8)
                np.testing.assert_allclose(out[t, h], o, rtol=0, atol=1e-14)
                assert abs(lse[t, h] - l) < 1e-13


# ---------------------------------------------------------------- FP8 E4M3 KV cache
def test_fp8_codes_match_torch():
    """All 256 codes against torch's float8_e4m3fn (an independent implementation of the format)."""
    want = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = oracle.fp8_e4m3_value(np.arange(256))
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    np.testing.assert_array_equal(got[~np.isnan(got)], want[~np.isnan(want)])


def test_fp8_known_codes():
    cases = {0x38: 1.0, 0xB8: -1.0, 0x7E: 448.0, 0x01: 2.0 ** -9, 0x08: 2.0 ** -6, 0x07: 7 * 2.0 ** -9, 0x40: 2.0,
             0x00: 0.0, 0x5C: 24.0}
    for code, val in cases.items():
        assert oracle.fp8_e4m3_value(code) == val, hex(code)
    assert np.isnan(oracle.fp8_e4m3_value(0x7F)) and np.isnan(oracle.fp8_e4m3_value(0xFF))


def test_fp8_decode_equals_decode_of_exact_values():
    """K/V values that FP8 holds exactly (n/4, |n| <= 7): the FP8 decode with scales equals the
    plain decode of the scaled values; distinct scales tell K from V."""
    r = rng(60)
    Hq, Hkv, d, ps = 4, 2, 6, 4
    L = np.array([5, 12])
    P = 5
    table = np.array([[3, 0, -1], [1, 4, 2]])
    kn = r.integers(-7, 8, size=(P, Hkv, ps, d)) / 4.0
    vn = r.integers(-7, 8, size=(P, Hkv, ps, d)) / 4.0
    to_code = lambda x: torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    q = r.standard_normal((2, Hq, d))
    out, lse = oracle.decode_paged_fp8(q, to_code(kn), to_code(vn), 0.75, 3.0, table, L, 0.6, ps)
    ref_o, ref_l = oracle.decode_paged(q, kn * 0.75, vn * 3.0, table, L, 0.6, ps)
    np.testing.assert_allclose(out, ref_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- golden closed forms
def _read_fixture(name):
    header, rows, cols = {}, [], None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            if cols is None and len(parts) >= 2 and not parts[1].lstrip("-").replace("/", "").isdigit():
                cols = parts
            elif cols is None:
                header[parts[0]] = [int(x) for x in parts[1:]]
            else:
                rows.append(dict(zip(cols, parts)))
    return header, rows


def _frac(s):
    return float(Fraction(s))


def test_golden_log_keys_prefill():
    header, rows = _read_fixture("log_keys_prefill.txt")
    T = header["T"][0]
    q = np.ones((1, 1, T, 1))
    k = np.log(np.arange(1, T + 1, dtype=np.float64)).reshape(1, 1, T, 1)
    v = np.arange(T, dtype=np.float64).reshape(1, 1, T, 1)
    out, lse = oracle.prefill(q, k, v, 1.0)
    assert len(rows) == T
    for r_ in rows:
        i = int(r_["i"])
        assert abs(out[0, 0, i, 0] - _frac(r_["out"])) < 1e-12
        assert abs(lse[0, 0, i] - math.log(int(r_["lse_arg"]))) < 1e-12


def test_golden_log_keys_decode():
    header, rows = _read_fixture("log_keys_decode.txt")
    ps, P = header["page_size"][0], header["num_pages"][0]
    tables = [np.array(header["table0"]), np.array(header["table1"])]
    for r_ in rows:
        s, L = int(r_["seq"]), int(r_["L"])
        kp = np.full((P, 1, ps, 1), np.nan)
        vp = np.full((P, 1, ps, 1), np.nan)
        for j in range(L):
            kp[tables[s][j // ps], 0, j % ps, 0] = math.log(j + 1)
            vp[tables[s][j // ps], 0, j % ps, 0] = j
        out, lse = oracle.decode_paged(np.ones((1, 1, 1)), kp, vp, tables[s][None], np.array([L]), 1.0, ps)
        assert abs(out[0, 0, 0] - _frac(r_["out"])) < 1e-12
        assert abs(lse[0, 0] - math.log(int(r_["lse_arg"]))) < 1e-12


def test_golden_gqa_prefix_mean():
    header, rows = _read_fixture("gqa_prefix_mean.txt")
    Hq, Hkv, T = header["Hq"][0], header["Hkv"][0], header["T"][0]
    q = np.zeros((1, Hq, T, 2))
    k = rng(20).standard_normal((1, Hkv, T, 2))
    v = np.zeros((1, Hkv, T, 2))
    for c in range(Hkv):
        for j in range(T):
            v[0, c, j] = (100 * c + j, -(100 * c + 2 * j))
    out, lse = oracle.prefill(q, k, v, 0.9)
    for r_ in rows:
        h, i = int(r_["h"]), int(r_["i"])
        assert abs(out[0, h, i, 0] - _frac(r_["out0"])) < 1e-12
        assert abs(out[0, h, i, 1] - _frac(r_["out1"])) < 1e-12
        assert abs(lse[0, h, i] - math.log(int(r_["lse_arg"]))) < 1e-12


# ---------------------------------------------------------------- edge cases and errors
def test_decode_empty_sequence():
    kp = np.full((2, 1, 16, 4), np.nan)
    out, lse = oracle.decode_paged(np.ones((2, 2, 4)), kp, kp, np.array([[0], [-1]]), np.array([3, 0]), 1.0, 16)
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    assert np.all(np.isnan(out[0]))  # page 0 is NaN here, and it is read


def test_empty_prefill():
    out, lse = oracle.prefill(np.zeros((0, 2, 4, 8)), np.zeros((0, 1, 4, 8)), np.zeros((0, 1, 4, 8)), 1.0)
    assert out.shape == (0, 2, 4, 8) and lse.shape == (0, 2, 4)
    out, lse = oracle.prefill(np.zeros((1, 2, 0, 8)), np.zeros((1, 1, 0, 8)), np.zeros((1, 1, 0, 8)), 1.0)
    assert out.shape == (1, 2, 0, 8)


def test_oracle_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.prefill(np.zeros((1, 3, 4, 8)), np.zeros((1, 2, 4, 8)), np.zeros((1, 2, 4, 8)), 1.0)
    with pytest.raises(ValueError):
        kp = np.zeros((1, 1, 16, 4))
        oracle.decode_paged(np.zeros((1, 1, 4)), kp, kp, np.array([[0]]), np.array([17]), 1.0, 16)
    with pytest.raises(ValueError):
        kp = np.zeros((1, 1, 16, 4))
        oracle.decode_paged(np.zeros((1, 1, 4)), kp, kp, np.array([[5]]), np.array([3]), 1.0, 16)
