"""GPU parity of attn_decode_paged_fp8 (FP8 E4M3 KV cache) against the fp64 oracle, through the C ABI.

Unused slots hold the NaN code 0x7F: a read outside a sequence's tokens
shows up as NaN in the output.
"""

import numpy as np
import pytest
import torch

import attention_causal_gqa_amd as A
import oracle
from attention_causal_gqa_amd import synth
from tests._gpu import TOL_BF16, TOL_LSE, device, max_err, np64, say

pytestmark = pytest.mark.gpu


def run(inp, scale, num_splits=0):
    A.attn_validate_paged_metadata(inp.block_table, inp.seq_lens, inp.page_size, inp.k_codes.shape[0])
    dev = device()
    out, lse = A.attn_decode_paged_fp8(inp.q.to(dev), inp.k_codes.to(dev), inp.v_codes.to(dev), inp.k_scale,
                                       inp.v_scale, inp.block_table.to(dev), inp.seq_lens.to(dev), scale=scale,
                                       num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def check(inp, scale, what, num_splits=0, batches=None):
    say(f"[decode fp8] {what}: B={inp.q.shape[0]} Hq={inp.q.shape[1]} pool={tuple(inp.k_codes.shape)} "
        f"scales {inp.k_scale:.4g}/{inp.v_scale:.4g} splits={num_splits}")
    out, lse = run(inp, scale, num_splits)
    idx = torch.arange(inp.q.shape[0]) if batches is None else torch.tensor(batches, dtype=torch.long)
    ref_o, ref_l = oracle.decode_paged_fp8(np64(inp.q[idx]), inp.k_codes.numpy(), inp.v_codes.numpy(), inp.k_scale,
                                           inp.v_scale, inp.block_table[idx].numpy(), inp.seq_lens[idx].numpy(),
                                           scale, inp.page_size)
    e_o = max_err(np64(out[idx]), ref_o, f"{what} out", TOL_BF16)
    e_l = max_err(np64(lse[idx]), ref_l, f"{what} lse", TOL_LSE)
    say(f"    max err out {e_o:.3e} lse {e_l:.3e}")


@pytest.mark.parametrize("Hq,Hkv,d", [(8, 8, 128), (16, 2, 128), (7, 1, 128), (8, 2, 64), (16, 1, 64)])
def test_fp8_decode_parity(Hq, Hkv, d):
    shp = synth.DecodeShape(5, Hq, Hkv, d, synth.PAGE_SIZE, 1, 700, torch.bfloat16)
    inp = synth.fp8_paged_inputs(shp, seed=1300 + Hq + d, poison_nan=True)
    check(inp, synth.fp32_scale(d), f"Hq{Hq} Hkv{Hkv} d{d}")


@pytest.mark.parametrize("num_splits", [1, 3, 0])
def test_fp8_decode_split_counts(num_splits):
    shp = synth.DecodeShape(4, 8, 2, 128, synth.PAGE_SIZE, 1, 900, torch.bfloat16)
    inp = synth.fp8_paged_inputs(shp, seed=1400, seq_lens=[1, 16, 17, 900], poison_nan=True)
    check(inp, synth.fp32_scale(128), f"splits {num_splits}", num_splits=num_splits)


def test_fp8_decode_equals_bf16_decode_of_exact_values():
    """Codes whose values bf16 holds exactly: the FP8 kernel and the bf16 kernel on the decoded,
    scaled values agree to accumulation rounding."""
    shp = synth.DecodeShape(4, 16, 4, 128, synth.PAGE_SIZE, 20, 500, torch.bfloat16)
    inp = synth.fp8_paged_inputs(shp, seed=1500)
    ks, vs = 2.0 ** -7, 2.0 ** -7  # powers of two keep value * scale exact in bf16; |values| <= 3.5
    kf = torch.from_numpy(oracle.fp8_e4m3_value(inp.k_codes.numpy()) * ks).to(torch.bfloat16)
    vf = torch.from_numpy(oracle.fp8_e4m3_value(inp.v_codes.numpy()) * vs).to(torch.bfloat16)
    inp2 = synth.Fp8PagedInputs(inp.q, inp.k_codes, inp.v_codes, ks, vs, inp.block_table, inp.seq_lens, 16)
    dev = device()
    scale = synth.fp32_scale(128)
    o8, l8 = run(inp2, scale)
    ob, lb = A.attn_decode_paged(inp.q.to(dev), kf.to(dev), vf.to(dev), inp.block_table.to(dev),
                                 inp.seq_lens.to(dev), scale=scale)
    torch.cuda.synchronize()
    say("[decode fp8] vs bf16 kernel on the decoded values")
    max_err(np64(o8), np64(ob.cpu()), "fp8 vs bf16 out", TOL_BF16)
    max_err(np64(l8), np64(lb.cpu()), "fp8 vs bf16 lse", 1e-5)


def test_workload9_full():
    shp = synth.WORKLOADS[9]["decode_fp8"]
    inp = synth.fp8_paged_inputs(shp, seed=109, poison_nan=True)
    check(inp, synth.fp32_scale(shp.d), "workload 9 (B64 Hq32 Hkv8 FP8, L~U[1024,8192])")
