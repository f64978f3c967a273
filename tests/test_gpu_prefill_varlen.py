"""GPU parity of attn_prefill_varlen (ragged batch packed along tokens), called through the C ABI."""

import numpy as np
import pytest
import torch

import attention_causal_gqa_amd as A
import oracle
from attention_causal_gqa_amd import synth
from tests._gpu import TOL_BF16, TOL_LSE, device, max_err, np64, say

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


def run_varlen(q, k, v, cu, max_seqlen, scale):
    A.attn_validate_varlen_metadata(cu, q.shape[0], max_seqlen)
    dev = device()
    out, lse = A.attn_prefill_varlen(q.to(dev), k.to(dev), v.to(dev), cu.to(dev), max_seqlen, scale=scale)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


@pytest.mark.parametrize("Hq,Hkv,d,lens", [
    (8, 2, 128, [1, 70, 300, 64, 129]),
    (4, 4, 128, [200, 3]),
    (32, 4, 128, [257, 31]),
    (8, 1, 64, [90, 1, 180]),
    (6, 3, 64, [65, 64, 63]),
    (8, 8, 128, [70, 300, 1]),        # Hkv a multiple of 8: each XCD serves its own kv head
    (16, 16, 64, [100, 1, 257, 64]),  # two kv heads per XCD
])
def test_varlen_parity(Hq, Hkv, d, lens):
    shp = synth.VarlenShape(len(lens), Hq, Hkv, d, 1, max(lens), BF16)
    q, k, v, cu, T = synth.varlen_inputs(shp, seed=1000 + Hq + d, lens=lens)
    scale = synth.fp32_scale(d)
    say(f"[varlen] Hq{Hq} Hkv{Hkv} d{d} lens {lens}")
    out, lse = run_varlen(q, k, v, cu, T, scale)
    ref_o, ref_l = oracle.prefill_varlen(np64(q), np64(k), np64(v), cu.numpy(), scale)
    max_err(np64(out), ref_o, "varlen out", TOL_BF16)
    max_err(np64(lse), ref_l, "varlen lse", TOL_LSE)


def test_varlen_empty_sequences_and_slack_max_seqlen():
    lens = [0, 50, 0, 0, 130, 0]
    shp = synth.VarlenShape(len(lens), 8, 2, 128, 0, 130, BF16)
    q, k, v, cu, T = synth.varlen_inputs(shp, seed=1100, lens=lens)
    scale = synth.fp32_scale(128)
    say("[varlen] empty sequences, max_seqlen larger than every length")
    out, lse = run_varlen(q, k, v, cu, T + 100, scale)
    ref_o, ref_l = oracle.prefill_varlen(np64(q), np64(k), np64(v), cu.numpy(), scale)
    max_err(np64(out), ref_o, "varlen out", TOL_BF16)
    max_err(np64(lse), ref_l, "varlen lse", TOL_LSE)


def dense_per_sequence(q, k, v, cu, scale):
    """Each sequence through the dense kernel (its own [1, H, T, d] tensors)."""
    dev = device()
    outs, lses = [], []
    for s in range(cu.numel() - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        qs = q[a:b].permute(1, 0, 2)[None].contiguous()
        ks = k[a:b].permute(1, 0, 2)[None].contiguous()
        vs = v[a:b].permute(1, 0, 2)[None].contiguous()
        o, l = A.attn_prefill(qs.to(dev), ks.to(dev), vs.to(dev), scale=scale)
        torch.cuda.synchronize()
        outs.append(o.cpu()[0].permute(1, 0, 2))
        lses.append(l.cpu()[0].permute(1, 0))
    return torch.cat(outs), torch.cat(lses)


def test_varlen_is_the_dense_kernel_bit_for_bit():
    lens = [333, 17, 512, 1]
    shp = synth.VarlenShape(len(lens), 16, 4, 128, 1, 512, BF16)
    q, k, v, cu, T = synth.varlen_inputs(shp, seed=1200, lens=lens)
    scale = synth.fp32_scale(128)
    say(f"[varlen] vs the dense kernel per sequence, lens {lens}")
    out, lse = run_varlen(q, k, v, cu, T, scale)
    od, ld = dense_per_sequence(q, k, v, cu, scale)
    assert torch.equal(out, od) and torch.equal(lse, ld)


def test_workload8_full():
    """The benchmark's ragged workload: bit for bit against the dense kernel, and every row against the oracle."""
    shp = synth.WORKLOADS[8]["varlen"]
    q, k, v, cu, T = synth.varlen_inputs(shp, seed=8)
    scale = synth.fp32_scale(shp.d)
    say(f"[varlen] workload 8: lens {(cu[1:] - cu[:-1]).tolist()}")
    out, lse = run_varlen(q, k, v, cu, T, scale)
    od, ld = dense_per_sequence(q, k, v, cu, scale)
    assert torch.equal(out, od) and torch.equal(lse, ld)
    say("    oracle over the packed batch")
    ref_o, ref_l = oracle.prefill_varlen(np64(q), np64(k), np64(v), cu.numpy(), scale)
    e_o = max_err(np64(out), ref_o, "w8 out", TOL_BF16)
    e_l = max_err(np64(lse), ref_l, "w8 lse", TOL_LSE)
    say(f"    max err out {e_o:.3e} lse {e_l:.3e}")
