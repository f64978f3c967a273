"""GPU parity of attn_prefill_paged_append (KV append + chunked prefill in one launch), through the C ABI.

Unused slots of the pools are NaN, and so are the chunk's own slots before the
call (stale values the launch must overwrite and never read): a read of
either shows up as NaN in the output.  Checked three ways: out / lse against
the fp64 oracle, the pools bit for bit against the oracle's append, and
everything bit for bit against the two-call path (attn_kv_append, then
attn_prefill_paged) on the same inputs.
"""

import numpy as np
import pytest
import torch

import attention_causal_gqa_amd as A
import oracle
from attention_causal_gqa_amd import synth
from tests._gpu import TOL_BF16, TOL_LSE, device, max_err, np64, say

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
NAN = float("nan")


def bits(t):
    return t.contiguous().view(torch.int16).numpy()


def run_fused(inp, scale):
    A.attn_validate_chunk_metadata(inp.block_table, inp.seq_lens, inp.page_size, inp.k_pages.shape[0],
                                   inp.q.shape[2])
    dev = device()
    kp, vp = inp.k_pages.to(dev), inp.v_pages.to(dev)
    out, lse = A.attn_prefill_paged_append(inp.q.to(dev), inp.k_new.to(dev), inp.v_new.to(dev), kp, vp,
                                           inp.block_table.to(dev), inp.seq_lens.to(dev), scale=scale)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), kp.cpu(), vp.cpu()


def run_two_calls(inp, scale):
    dev = device()
    kp, vp = inp.k_pages.to(dev), inp.v_pages.to(dev)
    bt, sl = inp.block_table.to(dev), inp.seq_lens.to(dev)
    A.attn_kv_append(inp.k_new.to(dev), inp.v_new.to(dev), kp, vp, bt, sl)
    out, lse = A.attn_prefill_paged(inp.q.to(dev), kp, vp, bt, sl, scale=scale)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), kp.cpu(), vp.cpu()


def check_pools(inp, kp, vp, what):
    k_ref, v_ref = oracle.kv_append(bits(inp.k_pages), bits(inp.v_pages), bits(inp.k_new), bits(inp.v_new),
                                    inp.block_table.numpy(), inp.seq_lens.numpy(), inp.page_size)
    assert np.array_equal(bits(kp), k_ref), f"{what}: K pool differs"
    assert np.array_equal(bits(vp), v_ref), f"{what}: V pool differs"


def check(inp, scale, what, rows=None):
    say(f"[fused] {what}: q{tuple(inp.q.shape)} pool{tuple(inp.k_pages.shape)} seq_lens {inp.seq_lens.tolist()[:8]}")
    out, lse, kp, vp = run_fused(inp, scale)
    check_pools(inp, kp, vp, what)
    ref_out, ref_lse, _, _ = oracle.prefill_paged_append(
        np64(inp.q), inp.k_new.float().numpy(), inp.v_new.float().numpy(), inp.k_pages.float().numpy(),
        inp.v_pages.float().numpy(), inp.block_table.numpy(), inp.seq_lens.numpy(), scale, inp.page_size, rows=rows)
    r_sel = slice(None) if rows is None else np.asarray(rows)
    e_o = max_err(np64(out)[:, :, r_sel], ref_out[:, :, r_sel], f"{what} out", TOL_BF16)
    e_l = max_err(np64(lse)[:, :, r_sel], ref_lse[:, :, r_sel], f"{what} lse", TOL_LSE)
    say(f"    max err out {e_o:.3e} lse {e_l:.3e}")
    return out, lse, kp, vp


@pytest.mark.parametrize("Hq,Hkv,d", [(8, 2, 128), (4, 4, 128), (32, 4, 128), (8, 1, 128), (8, 2, 64), (6, 3, 64),
                                      # B * Hkv a multiple of 8: the per-XCD pair order
                                      (8, 8, 128), (16, 8, 64)])
def test_fused_parity_group_sizes(Hq, Hkv, d):
    shp = synth.ChunkShape(3, Hq, Hkv, 100, d, synth.PAGE_SIZE, 100, 700, BF16)
    inp = synth.fused_inputs(shp, seed=1100 + Hq + Hkv + d, poison=NAN, stale=NAN)
    check(inp, synth.fp32_scale(d), f"Hq{Hq} Hkv{Hkv} d{d}")


# pos0 = L - Tq: 0 (the chunk is the whole sequence), mid-page, page-aligned, and values that put the
# chunk's first key inside a wave-wide DMA's rows (4 rows per DMA at d = 128, 8 at d = 64).
@pytest.mark.parametrize("Tq,lens,d", [
    (1, [1, 17, 302], 128),          # decode-like chunks
    (64, [64, 66, 129, 1000], 128),  # one tile of queries; pos0 = 0, 2, 65, 936
    (129, [129, 203, 513], 128),     # ragged query tail; pos0 = 0, 74, 384
    (300, [300, 305, 1025], 128),    # several query blocks
    (70, [70, 77, 141, 600], 64),    # pos0 = 0, 7, 71, 530
    (257, [257, 263, 900], 64),
])
def test_fused_lengths(Tq, lens, d):
    shp = synth.ChunkShape(len(lens), 8, 2, Tq, d, synth.PAGE_SIZE, 1, max(lens), BF16)
    inp = synth.fused_inputs(shp, seed=1200 + Tq + d, seq_lens=lens, poison=NAN, stale=NAN)
    check(inp, synth.fp32_scale(d), f"Tq {Tq} lens {lens} d {d}")


@pytest.mark.parametrize("scale", [0.0, -0.09])
def test_fused_scale_values(scale):
    shp = synth.ChunkShape(2, 8, 4, 90, 128, synth.PAGE_SIZE, 90, 400, BF16)
    inp = synth.fused_inputs(shp, seed=1300, poison=NAN, stale=NAN)
    check(inp, float(np.float32(scale)), f"scale {scale}")


@pytest.mark.parametrize("Hq,Hkv,Tq,lens,d", [
    (8, 2, 100, [100, 103, 357, 700], 128),
    (32, 8, 129, [129, 130, 1000], 128),
    (8, 2, 300, [301, 333, 1300], 64),
    (16, 1, 64, [64, 65, 97], 128),
])
def test_fused_equals_two_calls_bit_for_bit(Hq, Hkv, Tq, lens, d):
    """The fused launch must reproduce attn_kv_append + attn_prefill_paged exactly: same tiles, same
    arithmetic, the chunk's keys read from k_new / v_new instead of from the pools."""
    shp = synth.ChunkShape(len(lens), Hq, Hkv, Tq, d, synth.PAGE_SIZE, 1, max(lens), BF16)
    inp = synth.fused_inputs(shp, seed=1400 + Tq + d, seq_lens=lens, poison=NAN, stale=NAN)
    scale = synth.fp32_scale(d)
    say(f"[fused] vs two calls: Hq{Hq} Hkv{Hkv} Tq {Tq} lens {lens} d {d}")
    o1, l1, k1, v1 = run_fused(inp, scale)
    o2, l2, k2, v2 = run_two_calls(inp, scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert np.array_equal(bits(k1), bits(k2)) and np.array_equal(bits(v1), bits(v2))


def test_fused_chunks_rebuild_a_prefill():
    """Feed two sequences chunk by chunk into an empty (NaN) cache: each chunk's rows match the dense
    kernel's rows of the whole sequence, and the final cache is the sequences' K/V."""
    B, Hq, Hkv, d, L = 2, 16, 4, 128, 700
    q, k, v = synth.prefill_inputs(synth.PrefillShape(B, Hq, Hkv, L, d, BF16), seed=1500)
    dev = device()
    W = -(-L // synth.PAGE_SIZE)
    g = torch.Generator().manual_seed(1501)
    bt = torch.randperm(B * W, generator=g).to(torch.int32).reshape(B, W)
    kp = torch.full((B * W, Hkv, synth.PAGE_SIZE, d), NAN, dtype=BF16, device=dev)
    vp = torch.full_like(kp, NAN)
    scale = synth.fp32_scale(d)
    out_d, lse_d = A.attn_prefill(q.to(dev), k.to(dev), v.to(dev), scale=scale)
    start = 0
    for Tq in (13, 200, 64, 423):
        end = start + Tq
        say(f"[fused] chunk rows {start}..{end - 1}")
        sl = torch.full((B,), end, dtype=torch.int32)
        out, lse = A.attn_prefill_paged_append(q[:, :, start:end].contiguous().to(dev),
                                               k[:, :, start:end].contiguous().to(dev),
                                               v[:, :, start:end].contiguous().to(dev), kp, vp, bt.to(dev),
                                               sl.to(dev), scale=scale)
        torch.cuda.synchronize()
        max_err(np64(out.cpu()), np64(out_d[:, :, start:end].cpu()), f"rows {start}..{end - 1} out", TOL_BF16)
        max_err(np64(lse.cpu()), np64(lse_d[:, :, start:end].cpu()), f"rows {start}..{end - 1} lse", TOL_LSE)
        start = end
    assert start == L
    kc, vc = kp.cpu(), vp.cpu()
    for b in range(B):
        pos = torch.arange(L)
        pg = bt[b].long()[pos // synth.PAGE_SIZE]
        assert torch.equal(kc[pg, :, pos % synth.PAGE_SIZE].transpose(0, 1), k[b])
        assert torch.equal(vc[pg, :, pos % synth.PAGE_SIZE].transpose(0, 1), v[b])


def test_workload11_full():
    """The benchmark's fused workload at full size: pools bit for bit, bit-equal to the two-call path,
    and sampled rows of every sequence against the oracle."""
    shp = synth.WORKLOADS[11]["fused"]
    inp = synth.fused_inputs(shp, seed=11, poison=NAN, stale=NAN)
    scale = synth.fp32_scale(shp.d)
    say(f"[fused] workload 11: seq_lens {inp.seq_lens.tolist()}")
    o1, l1, k1, v1 = run_fused(inp, scale)
    check_pools(inp, k1, v1, "workload 11")
    o2, l2, k2, v2 = run_two_calls(inp, scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    rows = [0, 1, 255, 1024, 2046, 2047]
    ref_o, ref_l, _, _ = oracle.prefill_paged_append(
        np64(inp.q), inp.k_new.float().numpy(), inp.v_new.float().numpy(), inp.k_pages.float().numpy(),
        inp.v_pages.float().numpy(), inp.block_table.numpy(), inp.seq_lens.numpy(), scale, inp.page_size, rows=rows)
    e = max_err(np64(o1)[:, :, rows], ref_o[:, :, rows], "w11 out", TOL_BF16)
    max_err(np64(l1)[:, :, rows], ref_l[:, :, rows], "w11 lse", TOL_LSE)
    say(f"    max err out {e:.3e}")


def test_fused_longest_supported_context():
    """Contexts of 131072 tokens, the whole 8192-entry block table staged in LDS; sampled rows."""
    lens = [131072, 131072 - 5]
    shp = synth.ChunkShape(len(lens), 8, 2, 64, 128, synth.PAGE_SIZE, 1, 131072, BF16)
    inp = synth.fused_inputs(shp, seed=1600, seq_lens=lens, poison=NAN, stale=NAN)
    assert inp.block_table.shape[1] == 8192
    check(inp, synth.fp32_scale(128), "contexts of 131072 tokens (8192 pages)", rows=[0, 1, 31, 62, 63])


def test_fused_largest_group():
    """Hq / Hkv = 128: two chunk rows per workgroup."""
    shp = synth.ChunkShape(2, 128, 1, 37, 64, synth.PAGE_SIZE, 37, 300, BF16)
    inp = synth.fused_inputs(shp, seed=1700, poison=NAN, stale=NAN)
    check(inp, synth.fp32_scale(64), "Hq128 Hkv1 d64")
