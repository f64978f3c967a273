"""GPU check of attn_kv_append (called through the C ABI): the whole pools, bit for bit, against the oracle.

Unused slots hold NaN; the comparison is on the raw 16-bit patterns, so every
slot, written or not, must match exactly.
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


def bits(t):
    return t.contiguous().view(torch.int16).numpy()


def run_append(inp):
    A.attn_validate_chunk_metadata(inp.block_table, inp.seq_lens, inp.page_size, inp.k_pages.shape[0],
                                   inp.k_new.shape[2])
    dev = device()
    kp, vp = inp.k_pages.to(dev), inp.v_pages.to(dev)
    A.attn_kv_append(inp.k_new.to(dev), inp.v_new.to(dev), kp, vp, inp.block_table.to(dev), inp.seq_lens.to(dev))
    torch.cuda.synchronize()
    return kp.cpu(), vp.cpu()


def check(inp, what):
    say(f"[append] {what}: new{tuple(inp.k_new.shape)} pool{tuple(inp.k_pages.shape)} seq_lens {inp.seq_lens.tolist()[:8]}")
    kp, vp = run_append(inp)
    # The oracle copies values; bf16 -> int16 views keep the exact bits (NaN payloads included).
    k_ref, v_ref = oracle.kv_append(bits(inp.k_pages), bits(inp.v_pages), bits(inp.k_new), bits(inp.v_new),
                                    inp.block_table.numpy(), inp.seq_lens.numpy(), inp.page_size)
    assert np.array_equal(bits(kp), k_ref), f"{what}: K pool differs"
    assert np.array_equal(bits(vp), v_ref), f"{what}: V pool differs"
    return kp, vp


@pytest.mark.parametrize("Tn,lens,d", [
    (1, [1, 16, 17, 300], 128),      # one decode step: first slot, page end, new page, mid-page
    (37, [37, 40, 100, 513], 128),   # chunks across page boundaries, L = Tn
    (200, [200, 215, 1000], 64),
    (16, [16, 32, 48], 64),          # page-aligned chunks
])
def test_append_bit_exact(Tn, lens, d):
    shp = synth.ChunkShape(len(lens), 8, 4, Tn, d, synth.PAGE_SIZE, 1, max(lens), BF16)
    inp = synth.append_inputs(shp, seed=900 + Tn + d, seq_lens=lens, poison=float("nan"))
    check(inp, f"Tn {Tn} lens {lens} d {d}")


def test_append_then_chunked_prefill():
    """Append a chunk's K/V, then attend over the cache: same as the oracle on the appended pool."""
    Tq, lens, Hq, Hkv, d = 96, [96, 250, 600], 8, 2, 128
    shp = synth.ChunkShape(len(lens), Hkv, Hkv, Tq, d, synth.PAGE_SIZE, 1, max(lens), BF16)
    inp = synth.append_inputs(shp, seed=950, seq_lens=lens, poison=float("nan"))
    kp, vp = check(inp, "append before chunked prefill")
    g = torch.Generator().manual_seed(951)
    q = torch.randn(len(lens), Hq, Tq, d, generator=g).to(BF16)
    dev = device()
    scale = synth.fp32_scale(d)
    out, lse = A.attn_prefill_paged(q.to(dev), kp.to(dev), vp.to(dev), inp.block_table.to(dev),
                                    inp.seq_lens.to(dev), scale=scale)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.prefill_paged(np64(q), kp.float().numpy(), vp.float().numpy(), inp.block_table.numpy(),
                                        inp.seq_lens.numpy(), scale, inp.page_size)
    max_err(np64(out.cpu()), ref_o, "append + chunk out", TOL_BF16)
    max_err(np64(lse.cpu()), ref_l, "append + chunk lse", TOL_LSE)


def test_workload7_bit_exact():
    shp = synth.WORKLOADS[7]["append"]
    inp = synth.append_inputs(shp, seed=7)
    check(inp, "workload 7 (B4 Hkv8 Tn2048 L~U[4096,16384])")
