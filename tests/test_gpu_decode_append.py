"""GPU parity of attn_decode_paged_append (the newest token's KV append fused into the paged decode), through
the C ABI.

Unused slots of the pools are NaN, and so is each sequence's newest-token slot before the call (a stale value
the call overwrites and must never read): a read of either shows up as NaN in the output.  Checked three ways:
out / lse against the fp64 oracle, the pools bit for bit against the oracle's append, and everything bit for bit
against the two-call path (attn_kv_append with one token, then attn_decode_paged) on the same inputs.
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


def run_fused(inp, kn, vn, scale, num_splits=0):
    A.attn_validate_paged_metadata(inp.block_table, inp.seq_lens, inp.page_size, inp.k_pages.shape[0])
    dev = device()
    kp, vp = inp.k_pages.to(dev), inp.v_pages.to(dev)
    out, lse = A.attn_decode_paged_append(inp.q.to(dev), kn.to(dev), vn.to(dev), kp, vp, inp.block_table.to(dev),
                                          inp.seq_lens.to(dev), scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), kp.cpu(), vp.cpu()


def run_two_calls(inp, kn, vn, scale, num_splits=0):
    dev = device()
    kp, vp = inp.k_pages.to(dev), inp.v_pages.to(dev)
    bt, sl = inp.block_table.to(dev), inp.seq_lens.to(dev)
    some = inp.seq_lens > 0  # the append needs a token to write
    idx = torch.nonzero(some).flatten()
    if idx.numel():
        A.attn_kv_append(kn[idx].unsqueeze(2).contiguous().to(dev), vn[idx].unsqueeze(2).contiguous().to(dev), kp,
                         vp, inp.block_table[idx].contiguous().to(dev), inp.seq_lens[idx].contiguous().to(dev))
    out, lse = A.attn_decode_paged(inp.q.to(dev), kp, vp, bt, sl, scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), kp.cpu(), vp.cpu()


def check(inp, kn, vn, scale, what, num_splits=0):
    say(f"[decode+append] {what}: B={inp.q.shape[0]} Hq={inp.q.shape[1]} pool={tuple(inp.k_pages.shape)} "
        f"splits={num_splits}")
    out, lse, kp, vp = run_fused(inp, kn, vn, scale, num_splits)
    ref_o, ref_l, _, _ = oracle.decode_paged_append(
        np64(inp.q), kn.float().numpy(), vn.float().numpy(), inp.k_pages.float().numpy(),
        inp.v_pages.float().numpy(), inp.block_table.numpy(), inp.seq_lens.numpy(), scale, inp.page_size)
    # the pools: the oracle's append of the 16-bit patterns (NaN payloads included)
    some = np.nonzero(inp.seq_lens.numpy() > 0)[0]
    kb, vb = oracle.kv_append(bits(inp.k_pages), bits(inp.v_pages), bits(kn)[some][:, :, None],
                              bits(vn)[some][:, :, None], inp.block_table.numpy()[some],
                              inp.seq_lens.numpy()[some], inp.page_size)
    assert np.array_equal(bits(kp), kb), f"{what}: K pool differs"
    assert np.array_equal(bits(vp), vb), f"{what}: V pool differs"
    e_o = max_err(np64(out), ref_o, f"{what} out", TOL_BF16)
    e_l = max_err(np64(lse), ref_l, f"{what} lse", TOL_LSE)
    say(f"    max err out {e_o:.3e} lse {e_l:.3e}")
    return out, lse


EDGE_LENS = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257, 1000, 2047, 2048]


@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_edge_lengths(num_splits):
    """The newest token first, last and inside a page, on pieces cut at split edges."""
    shp = synth.DecodeShape(len(EDGE_LENS), 8, 4, 128, 16, 1, 2048, BF16)
    inp, kn, vn = synth.decode_append_inputs(shp, seed=2000 + num_splits, seq_lens=EDGE_LENS, poison=NAN,
                                             stale=NAN)
    check(inp, kn, vn, synth.fp32_scale(128), f"edge lengths, splits={num_splits}", num_splits)


@pytest.mark.parametrize("Hq,Hkv,d", [(8, 8, 128), (16, 2, 128), (7, 1, 128), (32, 2, 128), (8, 2, 64),
                                      (16, 1, 64)])
def test_group_sizes_and_d(Hq, Hkv, d):
    shp = synth.DecodeShape(6, Hq, Hkv, d, 16, 1, 700, BF16)
    inp, kn, vn = synth.decode_append_inputs(shp, seed=2100 + Hq + Hkv + d, poison=NAN, stale=NAN)
    check(inp, kn, vn, synth.fp32_scale(d), f"Hq{Hq} Hkv{Hkv} d{d}")


@pytest.mark.parametrize("B", [65, 130])
def test_batches_past_64_with_empty_sequences(B):
    """B > 64 with zero-length sequences (nothing appended, out 0, lse -inf) and one-token sequences (the
    newest token is the whole cache)."""
    rng = np.random.default_rng(B)
    lens = rng.integers(1, 400, B)
    lens[::7] = 0
    lens[1::11] = 1
    lens = [int(x) for x in lens]
    shp = synth.DecodeShape(B, 8, 2, 128, 16, 0, max(lens), BF16)
    inp, kn, vn = synth.decode_append_inputs(shp, seed=2200 + B, seq_lens=lens, poison=NAN, stale=NAN)
    out, lse = check(inp, kn, vn, synth.fp32_scale(128), f"B={B} with empty sequences", num_splits=3)
    zero = torch.tensor([L == 0 for L in lens])
    assert torch.all(out[zero].float() == 0) and torch.all(torch.isneginf(lse[zero]))


@pytest.mark.parametrize("wl,seed", [(4, 2304), (5, 2305), (10, 2310)])
def test_workload_shapes_equal_two_calls_bit_for_bit(wl, seed):
    """The decode workloads' shapes at full size: the fused call equals attn_kv_append + attn_decode_paged
    bit for bit (out, lse and both pools)."""
    shp = synth.WORKLOADS[wl]["decode"]
    inp, kn, vn = synth.decode_append_inputs(shp, seed=seed, poison=NAN, stale=NAN)
    scale = synth.fp32_scale(shp.d)
    say(f"[decode+append] workload {wl} shape vs two calls")
    o1, l1, k1, v1 = run_fused(inp, kn, vn, scale)
    o2, l2, k2, v2 = run_two_calls(inp, kn, vn, scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert np.array_equal(bits(k1), bits(k2)) and np.array_equal(bits(v1), bits(v2))


def test_workload5_shape_against_the_oracle():
    shp = synth.WORKLOADS[5]["decode"]
    inp, kn, vn = synth.decode_append_inputs(shp, seed=2405, poison=NAN, stale=NAN)
    check(inp, kn, vn, synth.fp32_scale(shp.d), "workload 5 shape (B64 Hq32 Hkv8, L~U[1024,8192])")


def test_decode_steps_rebuild_a_prefill():
    """Decode two sequences token by token from an empty (NaN) cache through the fused call: each step's
    output matches the dense kernel's row of that token, and the cache ends up holding every token."""
    B, Hq, Hkv, d, T = 2, 16, 4, 128, 70
    q, k, v = synth.prefill_inputs(synth.PrefillShape(B, Hq, Hkv, T, d, BF16), seed=2500)
    dev = device()
    W = -(-T // synth.PAGE_SIZE)
    g = torch.Generator().manual_seed(2501)
    bt = torch.randperm(B * W, generator=g).to(torch.int32).reshape(B, W).to(dev)
    kp = torch.full((B * W, Hkv, synth.PAGE_SIZE, d), NAN, dtype=BF16, device=dev)
    vp = torch.full_like(kp, NAN)
    scale = synth.fp32_scale(d)
    out_d, lse_d = A.attn_prefill(q.to(dev), k.to(dev), v.to(dev), scale=scale)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    worst = 0.0
    for t in range(T):
        sl = torch.full((B,), t + 1, dtype=torch.int32, device=dev)
        out, lse = A.attn_decode_paged_append(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(),
                                              vd[:, :, t].contiguous(), kp, vp, bt, sl, scale=scale)
        torch.cuda.synchronize()
        worst = max(worst, max_err(np64(out.cpu()), np64(out_d[:, :, t].cpu()), f"step {t} out", TOL_BF16))
        max_err(np64(lse.cpu()), np64(lse_d[:, :, t].cpu()), f"step {t} lse", TOL_LSE)
    say(f"[decode+append] {T} steps, max err against the dense rows {worst:.3e}")
    kc, vc, btc = kp.cpu(), vp.cpu(), bt.cpu()
    pos = torch.arange(T)
    for b in range(B):
        pg = btc[b].long()[pos // synth.PAGE_SIZE]
        assert torch.equal(kc[pg, :, pos % synth.PAGE_SIZE].transpose(0, 1), k[b])
        assert torch.equal(vc[pg, :, pos % synth.PAGE_SIZE].transpose(0, 1), v[b])
