"""GPU parity of attn_decode_paged against the fp64 oracle (called through the C ABI)."""

import numpy as np
import pytest
import torch

import attention_causal_gqa_amd as A
import oracle
from attention_causal_gqa_amd import synth
from tests._gpu import TOL_BF16, TOL_LSE, device, max_err, np64, say

pytestmark = pytest.mark.gpu


def to_dev(inp):
    dev = device()
    return (inp.q.to(dev), inp.k_pages.to(dev), inp.v_pages.to(dev), inp.block_table.to(dev), inp.seq_lens.to(dev))


def run_decode(inp, scale, num_splits=0):
    q, kp, vp, bt, sl = to_dev(inp)
    out, lse = A.attn_decode_paged(q, kp, vp, bt, sl, scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def oracle_decode(inp, scale, batches=None):
    """Oracle over the chosen sequences (all by default); inputs upcast exactly."""
    batches = list(range(inp.q.shape[0])) if batches is None else batches
    idx = torch.tensor(batches, dtype=torch.long)
    return oracle.decode_paged(np64(inp.q[idx]), inp.k_pages.float().numpy(), inp.v_pages.float().numpy(),
                               inp.block_table[idx].numpy(), inp.seq_lens[idx].numpy(), scale, inp.page_size)


def check(inp, scale, what, num_splits=0, batches=None):
    A.attn_validate_paged_metadata(inp.block_table, inp.seq_lens, inp.page_size, inp.k_pages.shape[0])
    say(f"[decode] {what}: B={inp.q.shape[0]} Hq={inp.q.shape[1]} pool={tuple(inp.k_pages.shape)} "
        f"W={inp.max_pages_per_seq} splits={num_splits}")
    out, lse = run_decode(inp, scale, num_splits)
    ref_out, ref_lse = oracle_decode(inp, scale, batches)
    sel = slice(None) if batches is None else torch.tensor(batches, dtype=torch.long)
    e_o = max_err(np64(out[sel]), ref_out, f"{what} out", TOL_BF16)
    e_l = max_err(np64(lse[sel]), ref_lse, f"{what} lse", TOL_LSE)
    say(f"    max err out {e_o:.3e} lse {e_l:.3e}")
    return out, lse


# ------------------------------------------------------------------ workload 4, whole output
def test_workload4_full():
    shp = synth.WORKLOADS[4]["decode"]
    inp = synth.paged_inputs(shp, seed=104, poison=float("nan"))
    check(inp, synth.fp32_scale(shp.d), "workload 4 (B32 Hq16 Hkv8, L~U[32,2048], NaN-poisoned tails)")


def test_workload5_decode_full():
    shp = synth.WORKLOADS[5]["decode"]
    inp = synth.paged_inputs(shp, seed=105, poison=float("nan"))
    out, lse = check(inp, synth.fp32_scale(shp.d), "workload 5 decode (B64 Hq32 Hkv8, L~U[1024,8192])")
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


def test_workload10_serving_batch_full():
    shp = synth.WORKLOADS[10]["decode"]
    inp = synth.paged_inputs(shp, seed=110, poison=float("nan"))
    out, lse = check(inp, synth.fp32_scale(shp.d), "workload 10 (B1024 Hq32 Hkv8, L~U[16,512], NaN-poisoned tails)")
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


# ------------------------------------------------------------------ lengths at page and split edges
EDGE_LENS = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257, 1000, 2047, 2048]


@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_edge_lengths(num_splits):
    shp = synth.DecodeShape(len(EDGE_LENS), 8, 4, 128, 16, 1, 2048, torch.bfloat16)
    inp = synth.paged_inputs(shp, seed=7, seq_lens=EDGE_LENS, extra_pages=5, poison=float("nan"))
    check(inp, synth.fp32_scale(128), f"edge lengths, splits={num_splits}", num_splits=num_splits)


@pytest.mark.parametrize("Hq,Hkv,d", [(8, 8, 128), (6, 2, 128), (7, 1, 128), (16, 2, 128), (32, 2, 128), (8, 2, 64), (4, 4, 64), (16, 1, 64)])
def test_group_sizes_and_d(Hq, Hkv, d):
    shp = synth.DecodeShape(5, Hq, Hkv, d, 16, 1, 700, torch.bfloat16)
    inp = synth.paged_inputs(shp, seed=Hq * 10 + Hkv + d, poison=float("nan"))
    check(inp, synth.fp32_scale(d), f"Hq{Hq} Hkv{Hkv} d{d}")


def test_empty_sequence():
    shp = synth.DecodeShape(4, 4, 2, 128, 16, 1, 300, torch.bfloat16)
    inp = synth.paged_inputs(shp, seed=11, seq_lens=[0, 5, 0, 300], poison=float("nan"))
    out, lse = check(inp, synth.fp32_scale(128), "seq_len 0 rows")
    assert torch.all(out[[0, 2]].float() == 0) and torch.all(torch.isneginf(lse[[0, 2]]))


def test_zero_query_is_mean_of_cached_values():
    shp = synth.DecodeShape(6, 8, 2, 128, 16, 1, 900, torch.bfloat16)
    inp = synth.paged_inputs(shp, seed=12, poison=float("nan"))
    inp.q.zero_()
    say("[decode] q = 0 closed form")
    out, lse = run_decode(inp, synth.fp32_scale(128))
    for b in range(6):
        L = int(inp.seq_lens[b])
        for h in range(8):
            vals = oracle.gather_pages(inp.v_pages.float().numpy(), inp.block_table[b].numpy(), L, 16, h // 4)
            max_err(np64(out[b, h]), vals.mean(axis=0), f"q=0 b{b} h{h}", TOL_BF16)
        max_err(np64(lse[b]), np.full(8, np.log(L)), f"q=0 lse b{b}", TOL_LSE)


# ------------------------------------------------------------------ invariants on the GPU
def test_page_permutation_is_bit_identical():
    shp = synth.DecodeShape(9, 8, 2, 128, 16, 1, 1500, torch.bfloat16)
    inp = synth.paged_inputs(shp, seed=13, extra_pages=7, poison=float("nan"))
    k2, v2, t2 = synth.permute_pages(inp.k_pages, inp.v_pages, inp.block_table, seed=14)
    inp2 = synth.PagedInputs(inp.q, k2, v2, t2, inp.seq_lens, 16)
    assert not torch.equal(t2, inp.block_table)
    say("[decode] page permutation")
    for ns in (0, 2):
        o1, l1 = run_decode(inp, synth.fp32_scale(128), ns)
        o2, l2 = run_decode(inp2, synth.fp32_scale(128), ns)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"splits={ns}"


def test_split_count_invariance():
    shp = synth.DecodeShape(8, 8, 4, 128, 16, 500, 2048, torch.bfloat16)
    inp = synth.paged_inputs(shp, seed=15)
    ref_out, ref_lse = oracle_decode(inp, synth.fp32_scale(128))
    say("[decode] split invariance")
    outs = {}
    for ns in (1, 2, 5, 16, 128, 0):
        o, l = run_decode(inp, synth.fp32_scale(128), ns)
        max_err(np64(o), ref_out, f"splits={ns} out", TOL_BF16)
        max_err(np64(l), ref_lse, f"splits={ns} lse", TOL_LSE)
        outs[ns] = o
    max_err(np64(outs[1]), np64(outs[0]), "splits 1 vs auto", TOL_BF16)


def test_decode_equals_prefill_row():
    """Decode with L = t + 1 cached tokens equals prefill row t (each within tolerance of the oracle and of each other)."""
    shp = synth.PrefillShape(2, 8, 2, 320, 128, torch.bfloat16)
    q, k, v = synth.prefill_inputs(shp, seed=16)
    dev = device()
    say("[decode] decode(t) == prefill row t")
    pout, plse = A.attn_prefill(q.to(dev), k.to(dev), v.to(dev), scale=synth.fp32_scale(128))
    torch.cuda.synchronize()
    pout, plse = pout.cpu(), plse.cpu()
    ts = [0, 1, 15, 16, 17, 100, 255, 256, 319]
    for t in ts:
        kp, vp, bt, sl = synth.paged_from_dense(k, v, [t + 1, t + 1], 16, seed=t, W=20)
        inp = synth.PagedInputs(q[:, :, t].contiguous(), kp, vp, bt, sl, 16)
        dout, dlse = run_decode(inp, synth.fp32_scale(128))
        max_err(np64(dout), np64(pout[:, :, t]), f"decode vs prefill row {t} out", TOL_BF16)
        max_err(np64(dlse), np64(plse[:, :, t]), f"decode vs prefill row {t} lse", TOL_LSE)
        ro, rl = oracle.prefill_rows(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                     synth.fp32_scale(128), 1, 5, [t])
        max_err(np64(dout[1, 5])[None], ro, f"decode row {t} vs oracle", TOL_BF16)


def test_workspace_reuse_and_explicit_workspace():
    shp = synth.DecodeShape(3, 4, 2, 128, 16, 1, 400, torch.bfloat16)
    inp = synth.paged_inputs(shp, seed=17)
    q, kp, vp, bt, sl = to_dev(inp)
    need = A.attn_decode_workspace_bytes(3, 4, 2, 128, 16, inp.max_pages_per_seq, 0)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=q.device)  # garbage contents
    say("[decode] caller workspace")
    o1, l1 = A.attn_decode_paged(q, kp, vp, bt, sl, workspace=ws)
    o2, l2 = A.attn_decode_paged(q, kp, vp, bt, sl, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    with pytest.raises(A.AttnError) as ei:
        A.attn_decode_paged(q, kp, vp, bt, sl, workspace=ws[: need - 256])
    assert ei.value.status == A.ATTN_ERR_WORKSPACE


@pytest.mark.parametrize("num_splits", [0, 1])
def test_longest_context(num_splits):
    """A sequence of 131072 tokens (8192 pages) beside a shorter one, with the automatic plan and with a
    single split (one wave streams a whole (sequence, kv head) run)."""
    lens = [131072, 99999]
    shp = synth.DecodeShape(len(lens), 8, 2, 128, 16, 1, 131072, torch.bfloat16)
    inp = synth.paged_inputs(shp, seed=17, seq_lens=lens, poison=float("nan"))
    check(inp, synth.fp32_scale(128), f"contexts up to 131072 tokens, splits={num_splits}", num_splits=num_splits)


def test_combine_slot_counts_at_register_boundaries():
    """With one page per item, sequences of 64, 65, 128 and 129 pages give the combine exactly 64, 65, 128
    and 129 slots: the combine holds the first 128 slot values in registers and reads any later ones, so
    the pieces on both sides of slots 64 and 128 are merged by both paths."""
    lens = [1024, 1025, 2048, 2049]
    shp = synth.DecodeShape(len(lens), 4, 2, 128, 16, 1, 2049, torch.bfloat16)
    inp = synth.paged_inputs(shp, seed=31, seq_lens=lens, poison=float("nan"))
    W = inp.max_pages_per_seq
    assert A.attn_decode_num_splits(shp.B, shp.Hq, shp.Hkv, shp.d, shp.page_size, W, 0) == W  # one page per item
    for ns in (0, 1, 3):
        check(inp, synth.fp32_scale(128), f"combine slot counts 64/65/128/129, splits={ns}", num_splits=ns)


@pytest.mark.parametrize("slope", [0.25, 0.1, -0.25])
def test_running_max_moves_across_pages(slope):
    """Cached keys whose scores rise (or fall) with the position: component 0 of the key at position j is
    j * slope and every query is (8, small noise), so with slope 0.25 the running max of a split moves on
    every page group, with 0.1 only on some, with -0.25 never after the first."""
    shp = synth.DecodeShape(3, 8, 2, 128, 16, 1, 1500, torch.bfloat16)
    inp = synth.paged_inputs(shp, seed=29, seq_lens=[1500, 777, 64], poison=float("nan"))
    g = torch.Generator().manual_seed(30)
    q = 0.05 * torch.randn(inp.q.shape, generator=g)
    q[..., 0] = 8.0
    inp.q = q.to(torch.bfloat16)
    kp = inp.k_pages.float()
    for b in range(3):
        L = int(inp.seq_lens[b])
        pos = torch.arange(L)
        pages = inp.block_table[b, pos // 16].long()
        kp[pages, :, pos % 16, :] = 0.05 * torch.randn(L, shp.Hkv, shp.d, generator=g)
        kp[pages, :, pos % 16, 0] = (slope * pos.float())[:, None]
    inp.k_pages = kp.to(torch.bfloat16)
    for splits in (0, 1):
        check(inp, synth.fp32_scale(128), f"score ramp, slope {slope}, splits={splits}", num_splits=splits)


# ------------------------------------------------------------------ batches past one sequence per lane
def boundary_lens(B, seed):
    """Lengths 0..900 with zero-length and one-token sequences on both sides of every multiple of 64 and of
    the per-lane block size ceil(B / 64)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(2, 900, B)
    per = (B + 63) // 64
    for edge in sorted(set(range(64, B, 64)) | set(range(per, B, per))):
        lens[edge - 1] = 0
        lens[edge] = 1
        if edge + 1 < B:
            lens[edge + 1] = 0
    lens[0] = 1
    lens[-1] = 0
    return [int(x) for x in lens]


@pytest.mark.parametrize("B", [65, 130])
@pytest.mark.parametrize("num_splits", [0, 3])
def test_batches_past_64_sequences(B, num_splits):
    """B > 64: each lane of the streaming kernel's scan sums a block of ceil(B / 64) sequences, and the
    wave's share is found in two steps (block, then sequence).  Zero-length and one-token sequences sit at
    the block and 64-sequence boundaries."""
    lens = boundary_lens(B, seed=B + num_splits)
    shp = synth.DecodeShape(B, 8, 2, 128, 16, 0, max(lens), torch.bfloat16)
    inp = synth.paged_inputs(shp, seed=40 + B, seq_lens=lens, poison=float("nan"))
    out, lse = check(inp, synth.fp32_scale(128), f"B={B} across lane blocks, splits={num_splits}",
                     num_splits=num_splits)
    zero = torch.tensor([L == 0 for L in lens])
    assert torch.all(out[zero].float() == 0) and torch.all(torch.isneginf(lse[zero]))


@pytest.mark.parametrize("B,Hq,Hkv,lmax", [(1024, 8, 2, 512), (4096, 4, 1, 256)])
def test_serving_batch_sizes(B, Hq, Hkv, lmax):
    """Serving-size batches of short, ragged sequences (some empty), NaN in every unused slot; whole output
    against the oracle, with the automatic plan and with two splits."""
    rng = np.random.default_rng(B)
    lens = rng.integers(1, lmax + 1, B)
    lens[rng.random(B) < 0.05] = 0
    lens = [int(x) for x in lens]
    shp = synth.DecodeShape(B, Hq, Hkv, 128, 16, 0, lmax, torch.bfloat16)
    inp = synth.paged_inputs(shp, seed=B + 1, seq_lens=lens, poison=float("nan"))
    for ns in (0, 2):
        check(inp, synth.fp32_scale(128), f"B={B} serving batch, splits={ns}", num_splits=ns)
