"""GPU parity of attn_prefill against the fp64 oracle (called through the C ABI)."""

import math

import numpy as np
import pytest
import torch

import attention_causal_gqa_amd as A
import oracle
from attention_causal_gqa_amd import synth
from tests._gpu import TOL_BF16, TOL_F32, TOL_LSE, device, max_err, np64, say

pytestmark = pytest.mark.gpu


def run_prefill(q, k, v, scale):
    dev = device()
    out, lse = A.attn_prefill(q.to(dev), k.to(dev), v.to(dev), scale=scale)
    torch.cuda.synchronize()
    return out, lse


def check_full(q, k, v, scale, tol, what):
    say(f"[prefill] {what}: q{tuple(q.shape)} k{tuple(k.shape)} {q.dtype} scale={scale}")
    out, lse = run_prefill(q, k, v, scale)
    ref_out, ref_lse = oracle.prefill(np64(q), np64(k), np64(v), scale)
    e_out = max_err(np64(out), ref_out, f"{what} out", tol)
    e_lse = max_err(np64(lse), ref_lse, f"{what} lse", TOL_LSE)
    say(f"    max err out {e_out:.3e} lse {e_lse:.3e}")
    return out, lse


# ------------------------------------------------------------------ workloads 1 and 2, whole output
def test_workload1_fp32_mha():
    shp = synth.WORKLOADS[1]["prefill"]
    q, k, v = synth.prefill_inputs(shp, seed=1)
    check_full(q, k, v, synth.fp32_scale(shp.d), TOL_F32, "workload 1 (fp32 MHA T128 d64)")


def test_workload2_bf16_gqa():
    shp = synth.WORKLOADS[2]["prefill"]
    q, k, v = synth.prefill_inputs(shp, seed=2)
    check_full(q, k, v, synth.fp32_scale(shp.d), TOL_BF16, "workload 2 (bf16 GQA T512 d128)")


# ------------------------------------------------------------------ shapes: ragged T, every group size, d 64/128
BF16_SHAPES = [
    # B, Hq, Hkv, T, d
    (1, 1, 1, 1, 128),
    (2, 4, 2, 7, 128),
    (1, 8, 2, 63, 128),
    (1, 4, 1, 65, 128),
    (2, 6, 2, 200, 128),   # g = 3: 42 tokens x 3 heads per workgroup, two dead rows
    (1, 16, 2, 257, 128),  # g = 8
    (1, 3, 3, 100, 128),   # MHA
    (1, 32, 1, 40, 128),   # g = 32: 4 tokens per workgroup
    (1, 7, 1, 90, 128),    # g = 7
    (1, 8, 1, 130, 64),
    (2, 2, 2, 129, 64),
    (1, 12, 4, 300, 64),
]


@pytest.mark.parametrize("B,Hq,Hkv,T,d", BF16_SHAPES)
def test_bf16_shapes(B, Hq, Hkv, T, d):
    shp = synth.PrefillShape(B, Hq, Hkv, T, d, torch.bfloat16)
    q, k, v = synth.prefill_inputs(shp, seed=1000 + T + Hq)
    check_full(q, k, v, synth.fp32_scale(d), TOL_BF16, f"bf16 B{B} Hq{Hq} Hkv{Hkv} T{T} d{d}")


F32_SHAPES = [(1, 1, 1, 1, 64), (2, 4, 2, 100, 64), (1, 2, 2, 200, 128), (1, 6, 3, 129, 128)]


@pytest.mark.parametrize("B,Hq,Hkv,T,d", F32_SHAPES)
def test_f32_shapes(B, Hq, Hkv, T, d):
    shp = synth.PrefillShape(B, Hq, Hkv, T, d, torch.float32)
    q, k, v = synth.prefill_inputs(shp, seed=2000 + T)
    check_full(q, k, v, synth.fp32_scale(d), TOL_F32, f"fp32 B{B} Hq{Hq} Hkv{Hkv} T{T} d{d}")


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.5, 1e-3])
def test_bf16_scale_values(scale):
    shp = synth.PrefillShape(1, 4, 2, 150, 128, torch.bfloat16)
    q, k, v = synth.prefill_inputs(shp, seed=77)
    check_full(q, k, v, float(np.float32(scale)), TOL_BF16, f"bf16 scale {scale}")


@pytest.mark.parametrize("dtype,tol", [(torch.bfloat16, TOL_BF16), (torch.float32, TOL_F32)])
def test_zero_query_is_prefix_mean(dtype, tol):
    """q = 0: out_i = mean_{j<=i} v_j of the kv head h // g, lse_i = ln(i + 1)."""
    shp = synth.PrefillShape(2, 8, 2, 200, 128, dtype)
    _, k, v = synth.prefill_inputs(shp, seed=5)
    v[:, 1] += 3.0  # distinct values per kv head
    q = torch.zeros(2, 8, 200, 128, dtype=dtype)
    say(f"[prefill] q = 0 closed form {dtype}")
    out, lse = run_prefill(q, k, v, synth.fp32_scale(128))
    vv = np64(v)
    mean = np.cumsum(vv, axis=2) / np.arange(1, 201)[None, None, :, None]
    want = np.repeat(mean, 4, axis=1)
    max_err(np64(out), want, "q=0 out", tol)
    max_err(np64(lse), np.broadcast_to(np.log(np.arange(1, 201)), (2, 8, 200)), "q=0 lse", TOL_LSE)


def test_single_token_returns_v_exactly():
    shp = synth.PrefillShape(3, 8, 4, 1, 128, torch.bfloat16)
    q, k, v = synth.prefill_inputs(shp, seed=6)
    say("[prefill] T = 1")
    out, lse = run_prefill(q, k, v, synth.fp32_scale(128))
    assert torch.equal(out.cpu(), v.repeat_interleave(2, dim=1)), "T=1 must return v_0 bit for bit"
    dots = (np64(q) * np.repeat(np64(k), 2, axis=1)).sum(-1)
    max_err(np64(lse), synth.fp32_scale(128) * dots, "T=1 lse", TOL_LSE)


def test_row_zero_is_v0_for_long_rows():
    """Row 0 sees only key 0: out is v_0 exactly, whatever T is."""
    shp = synth.PrefillShape(1, 8, 2, 700, 128, torch.bfloat16)
    q, k, v = synth.prefill_inputs(shp, seed=8)
    say("[prefill] row 0 == v_0")
    out, _ = run_prefill(q, k, v, synth.fp32_scale(128))
    assert torch.equal(out[:, :, 0].cpu(), v[:, :, 0].repeat_interleave(4, dim=1))


def test_causality_future_keys_do_not_leak():
    shp = synth.PrefillShape(1, 4, 2, 300, 128, torch.bfloat16)
    q, k, v = synth.prefill_inputs(shp, seed=9)
    say("[prefill] causality")
    out1, lse1 = run_prefill(q, k, v, synth.fp32_scale(128))
    k2, v2 = k.clone(), v.clone()
    k2[:, :, 171:] = 7.0
    v2[:, :, 171:] = -9.0
    out2, lse2 = run_prefill(q, k2, v2, synth.fp32_scale(128))
    assert torch.equal(out1[:, :, :171].cpu(), out2[:, :, :171].cpu())
    assert torch.equal(lse1[:, :, :171].cpu(), lse2[:, :, :171].cpu())


def test_lse_is_optional_and_out_is_identical():
    shp = synth.PrefillShape(1, 4, 2, 97, 128, torch.bfloat16)
    q, k, v = synth.prefill_inputs(shp, seed=10)
    dev = device()
    say("[prefill] lse = NULL")
    o1, _ = A.attn_prefill(q.to(dev), k.to(dev), v.to(dev))
    o2, l2 = A.attn_prefill(q.to(dev), k.to(dev), v.to(dev), lse=False)
    torch.cuda.synchronize()
    assert l2 is None and torch.equal(o1.cpu(), o2.cpu())


# ------------------------------------------------------------------ many (sequence, kv head) pairs
# Batches with 100 and 256 (sequence, kv head) pairs, so the workgroup order
# cycles over many pairs (partial last blocks, d 64 and 128); each result is
# also compared bit for bit with the same sequence run alone, which launches
# a different set of workgroups.
PAIR_SHAPES = [
    # B, Hq, Hkv, T, d
    (16, 32, 16, 300, 128),  # 256 pairs, three blocks of 128 tokens per pair, the last of 44
    (2, 128, 16, 300, 128),  # 32 pairs, g = 8: 10 blocks of 32 tokens per pair
    (16, 16, 16, 520, 64),   # 256 pairs, d 64: blocks of 256, 256 and 8 tokens
    (25, 8, 4, 300, 64),     # 100 pairs
]


@pytest.mark.parametrize("B,Hq,Hkv,T,d", PAIR_SHAPES)
def test_bf16_many_pairs(B, Hq, Hkv, T, d):
    shp = synth.PrefillShape(B, Hq, Hkv, T, d, torch.bfloat16)
    q, k, v = synth.prefill_inputs(shp, seed=3000 + B + T)
    out, lse = check_full(q, k, v, synth.fp32_scale(d), TOL_BF16, f"bf16 many pairs B{B} Hq{Hq} Hkv{Hkv} T{T} d{d}")
    # The same sequence alone: its rows must come out bit for bit the same.
    for b in (0, B - 1):
        o1, l1 = run_prefill(q[b : b + 1], k[b : b + 1], v[b : b + 1], synth.fp32_scale(d))
        assert torch.equal(o1.cpu(), out[b : b + 1].cpu()), f"sequence {b} alone differs"
        assert torch.equal(l1.cpu(), lse[b : b + 1].cpu()), f"sequence {b} alone differs (lse)"


# ------------------------------------------------------------------ full-size workloads, whole output
@pytest.mark.parametrize("workload", [3, 5])
def test_full_size_prefill_whole_output(workload):
    """The benchmark's prefill workloads at full size, every element of out and lse against the oracle (one
    oracle call per batch: 32 heads x T x T scores in fp64, about 0.5 s per head at T = 8192)."""
    shp = synth.WORKLOADS[workload]["prefill"]
    q, k, v = synth.prefill_inputs(shp, seed=workload)
    scale = synth.fp32_scale(shp.d)
    say(f"[prefill] workload {workload} full size {shp}")
    out, lse = run_prefill(q, k, v, scale)
    out, lse = out.cpu(), lse.cpu()
    worst = 0.0
    for b in range(shp.B):
        say(f"    oracle, batch {b}")
        ro, rl = oracle.prefill(np64(q[b : b + 1]), np64(k[b : b + 1]), np64(v[b : b + 1]), scale)
        worst = max(worst, max_err(np64(out[b : b + 1]), ro, f"w{workload} b{b} out", TOL_BF16))
        max_err(np64(lse[b : b + 1]), rl, f"w{workload} b{b} lse", TOL_LSE)
    say(f"    max err out {worst:.3e}")


# ------------------------------------------------------------------ the lazy running-max rescale
def ramp_inputs(B, Hq, Hkv, T, d, slope, seed, dtype=torch.bfloat16):
    """Scores that rise (slope > 0) or fall along the keys: component 0 of key j is j * slope, every query is
    (8, small noise); other key components are small noise.  With scale 1/sqrt(d) the base-2 score of key j
    is about 1.02 * slope * j (d = 128)."""
    g = torch.Generator().manual_seed(seed)
    q = 0.05 * torch.randn(B, Hq, T, d, generator=g)
    q[..., 0] = 8.0
    k = 0.05 * torch.randn(B, Hkv, T, d, generator=g)
    k[..., 0] = slope * torch.arange(T, dtype=torch.float32)
    v = torch.randn(B, Hkv, T, d, generator=g)
    return q.to(dtype), k.to(dtype), v.to(dtype)


@pytest.mark.parametrize("slope", [0.25, 0.1, -0.25])
def test_running_max_moves_across_tiles(slope):
    """slope 0.25: each 64-key tile's max exceeds the previous one by about 16 (base 2), so the running max
    and the output rescale move in every tile; 0.1: about 6.5 per tile, so they move in some tiles and not
    in others (probabilities up to 2^8 against a stale max); -0.25: the max is key 0's and never moves."""
    q, k, v = ramp_inputs(1, 8, 2, 520, 128, slope, seed=31)
    check_full(q, k, v, synth.fp32_scale(128), TOL_BF16, f"bf16 score ramp, slope {slope}")
