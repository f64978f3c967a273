"""GPU parity of attn_prefill_paged (chunked prefill over a paged cache) against the fp64 oracle.

Called through the C ABI.  Unused slots of every page pool are NaN, so a read
outside a sequence's tokens shows up as NaN in the output.
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


def run_chunk(inp, scale):
    dev = device()
    q, kp, vp, bt, sl = (t.to(dev) for t in (inp.q, inp.k_pages, inp.v_pages, inp.block_table, inp.seq_lens))
    out, lse = A.attn_prefill_paged(q, kp, vp, bt, sl, scale=scale)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def oracle_chunk(inp, scale, rows=None, batches=None):
    batches = list(range(inp.q.shape[0])) if batches is None else batches
    idx = torch.tensor(batches, dtype=torch.long)
    return oracle.prefill_paged(np64(inp.q[idx]), inp.k_pages.float().numpy(), inp.v_pages.float().numpy(),
                                inp.block_table[idx].numpy(), inp.seq_lens[idx].numpy(), scale, inp.page_size,
                                rows=rows)


def check(inp, scale, what, rows=None, batches=None):
    A.attn_validate_chunk_metadata(inp.block_table, inp.seq_lens, inp.page_size, inp.k_pages.shape[0],
                                   inp.q.shape[2])
    say(f"[chunk] {what}: q{tuple(inp.q.shape)} pool{tuple(inp.k_pages.shape)} seq_lens {inp.seq_lens.tolist()[:8]}")
    out, lse = run_chunk(inp, scale)
    ref_out, ref_lse = oracle_chunk(inp, scale, rows, batches)
    b_sel = slice(None) if batches is None else torch.tensor(batches, dtype=torch.long)
    r_sel = slice(None) if rows is None else np.asarray(rows)
    e_o = max_err(np64(out[b_sel])[:, :, r_sel], ref_out[:, :, r_sel], f"{what} out", TOL_BF16)
    e_l = max_err(np64(lse[b_sel])[:, :, r_sel], ref_lse[:, :, r_sel], f"{what} lse", TOL_LSE)
    say(f"    max err out {e_o:.3e} lse {e_l:.3e}")
    return out, lse


@pytest.mark.parametrize("Hq,Hkv,d", [(8, 2, 128), (4, 4, 128), (16, 2, 128), (32, 4, 128), (8, 1, 128),
                                      (8, 2, 64), (6, 3, 64),
                                      # B * Hkv a multiple of 8: the per-XCD pair order
                                      (8, 8, 128), (16, 8, 64)])
def test_chunk_parity_group_sizes(Hq, Hkv, d):
    shp = synth.ChunkShape(3, Hq, Hkv, 100, d, synth.PAGE_SIZE, 100, 700, BF16)
    inp = synth.chunk_inputs(shp, seed=600 + Hq + Hkv + d, poison=float("nan"))
    check(inp, synth.fp32_scale(d), f"Hq{Hq} Hkv{Hkv} d{d}")


@pytest.mark.parametrize("Tq,lens", [
    (1, [1, 17, 300]),          # decode-like chunks
    (64, [64, 65, 128, 1000]),  # one tile of queries; L = Tq, L = Tq + 1, page-aligned L
    (129, [129, 200, 513]),     # ragged query tail
    (300, [300, 301, 1024]),    # several query blocks, L = Tq exactly
])
def test_chunk_lengths(Tq, lens):
    shp = synth.ChunkShape(len(lens), 8, 2, Tq, 128, synth.PAGE_SIZE, 1, max(lens), BF16)
    inp = synth.chunk_inputs(shp, seed=700 + Tq, seq_lens=lens, poison=float("nan"))
    check(inp, synth.fp32_scale(128), f"Tq {Tq} lens {lens}")


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.3])
def test_chunk_scale_values(scale):
    shp = synth.ChunkShape(2, 8, 4, 90, 128, synth.PAGE_SIZE, 90, 400, BF16)
    inp = synth.chunk_inputs(shp, seed=77, poison=float("nan"))
    check(inp, float(np.float32(scale)), f"scale {scale}")


def test_whole_sequence_chunk_is_the_dense_kernel_bit_for_bit():
    """L = Tq: the paged kernel reads the same K/V through pages and must equal attn_prefill exactly."""
    B, Hq, Hkv, T, d = 2, 16, 4, 333, 128
    q, k, v = synth.prefill_inputs(synth.PrefillShape(B, Hq, Hkv, T, d, BF16), seed=801)
    kp, vp, bt, sl = synth.paged_from_dense(k, v, [T] * B, synth.PAGE_SIZE, seed=802)
    dev = device()
    say(f"[chunk] whole-sequence chunk vs dense kernel: B{B} Hq{Hq} Hkv{Hkv} T{T}")
    out_d, lse_d = A.attn_prefill(q.to(dev), k.to(dev), v.to(dev), scale=synth.fp32_scale(d))
    out_p, lse_p = A.attn_prefill_paged(q.to(dev), kp.to(dev), vp.to(dev), bt.to(dev), sl.to(dev),
                                        scale=synth.fp32_scale(d))
    torch.cuda.synchronize()
    assert torch.equal(out_p.cpu(), out_d.cpu())
    assert torch.equal(lse_p.cpu(), lse_d.cpu())


def test_chunk_is_the_tail_of_the_dense_kernel():
    """Rows L-Tq.. of a dense prefill over the whole sequence, within tolerance of the chunk's rows."""
    B, Hq, Hkv, d, Tq = 2, 8, 2, 128, 150
    lens = [500, 731]
    T = max(lens)
    q, k, v = synth.prefill_inputs(synth.PrefillShape(B, Hq, Hkv, T, d, BF16), seed=811)
    kp, vp, bt, sl = synth.paged_from_dense(k, v, lens, synth.PAGE_SIZE, seed=812)
    dev = device()
    qc = torch.stack([q[b, :, lens[b] - Tq : lens[b]] for b in range(B)]).contiguous()
    out_p, lse_p = A.attn_prefill_paged(qc.to(dev), kp.to(dev), vp.to(dev), bt.to(dev), sl.to(dev),
                                        scale=synth.fp32_scale(d))
    torch.cuda.synchronize()
    say(f"[chunk] chunk vs dense tail: lens {lens} Tq {Tq}")
    for b in range(B):
        L = lens[b]
        out_d, lse_d = A.attn_prefill(q[b : b + 1, :, :L].contiguous().to(dev), k[b : b + 1, :, :L].contiguous().to(dev),
                                      v[b : b + 1, :, :L].contiguous().to(dev), scale=synth.fp32_scale(d))
        torch.cuda.synchronize()
        max_err(np64(out_p[b]), np64(out_d[0, :, L - Tq :]), f"b{b} out vs dense", TOL_BF16)
        max_err(np64(lse_p[b]), np64(lse_d[0, :, L - Tq :]), f"b{b} lse vs dense", TOL_LSE)


def test_page_permutation_is_bit_identical():
    shp = synth.ChunkShape(3, 8, 2, 120, 128, synth.PAGE_SIZE, 120, 600, BF16)
    inp = synth.chunk_inputs(shp, seed=821, poison=float("nan"))
    out1, lse1 = run_chunk(inp, synth.fp32_scale(128))
    k2, v2, t2 = synth.permute_pages(inp.k_pages, inp.v_pages, inp.block_table, seed=822)
    inp2 = synth.ChunkInputs(inp.q, k2, v2, t2, inp.seq_lens, inp.page_size)
    out2, lse2 = run_chunk(inp2, synth.fp32_scale(128))
    say("[chunk] page permutation")
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_workload6_full():
    """The benchmark's chunked-prefill workload at full size, every row (the oracle materialises a
    2048 x L score block per head, L up to 16384)."""
    shp = synth.WORKLOADS[6]["chunk"]
    inp = synth.chunk_inputs(shp, seed=6, poison=float("nan"))
    out, lse = run_chunk(inp, synth.fp32_scale(shp.d))
    worst = 0.0
    for b in range(shp.B):
        say(f"[chunk] workload 6, oracle for sequence {b} (L = {int(inp.seq_lens[b])})")
        ro, rl = oracle_chunk(inp, synth.fp32_scale(shp.d), batches=[b])
        worst = max(worst, max_err(np64(out[b : b + 1]), ro, f"w6 b{b} out", TOL_BF16))
        max_err(np64(lse[b : b + 1]), rl, f"w6 b{b} lse", TOL_LSE)
    say(f"    max err out {worst:.3e}")


def test_longest_supported_context():
    """Contexts of 131072 tokens: the whole 8192-entry block table the kernel stages in LDS is in use
    (the longest context the chunked prefill accepts), once with a ragged last page."""
    lens = [131072, 131072 - 5]
    shp = synth.ChunkShape(len(lens), 8, 2, 64, 128, synth.PAGE_SIZE, 1, 131072, BF16)
    inp = synth.chunk_inputs(shp, seed=131, seq_lens=lens, poison=float("nan"))
    assert inp.block_table.shape[1] == 8192
    check(inp, synth.fp32_scale(128), "contexts of 131072 tokens (8192 pages)", rows=[0, 1, 31, 62, 63])
