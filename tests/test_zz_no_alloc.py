"""attn_decode_paged_noalloc (static per-GPU scratch, no allocation) against attn_decode_paged (caller
workspace) and the fp64 oracle, through the C ABI: two calls in a row, the second on a smaller input, so the
second reads a scratch that still holds the first call's pieces and run records."""

import pytest
import torch

import attention_causal_gqa_amd as A
import oracle
from attention_causal_gqa_amd import synth
from tests._gpu import TOL_BF16, TOL_LSE, device, max_err, np64, say

pytestmark = pytest.mark.gpu


def run_both(inp, num_splits):
    dev = device()
    q, kp, vp, bt, sl = (t.to(dev) for t in (inp.q, inp.k_pages, inp.v_pages, inp.block_table, inp.seq_lens))
    scale = synth.fp32_scale(q.shape[2])
    ref_o, ref_l = A.attn_decode_paged(q, kp, vp, bt, sl, scale=scale, num_splits=num_splits)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((q.shape[0], q.shape[1]), float("nan"), dtype=torch.float32, device=dev)
    A.attn_decode_paged_noalloc(q, kp, vp, bt, sl, out, lse, scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), ref_o.cpu(), ref_l.cpu(), scale


@pytest.mark.parametrize("num_splits", [0, 3])
def test_noalloc_matches_caller_workspace_on_two_calls(num_splits):
    first = synth.DecodeShape(64, 32, 8, 128, 16, 1024, 4096, torch.bfloat16)
    second = synth.DecodeShape(9, 8, 2, 128, 16, 1, 700, torch.bfloat16)
    for what, shp, seed in (("first call", first, 501), ("second call, smaller", second, 502)):
        inp = synth.paged_inputs(shp, seed=seed + num_splits, poison=float("nan"))
        say(f"[noalloc] {what}: B={shp.B} Hq={shp.Hq} Hkv={shp.Hkv} splits={num_splits}")
        out, lse, ref_o, ref_l, scale = run_both(inp, num_splits)
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"{what}: differs from attn_decode_paged"
        want_o, want_l = oracle.decode_paged(np64(inp.q), inp.k_pages.float().numpy(), inp.v_pages.float().numpy(),
                                             inp.block_table.numpy(), inp.seq_lens.numpy(), scale, 16)
        e_o = max_err(np64(out), want_o, f"{what} out", TOL_BF16)
        e_l = max_err(np64(lse), want_l, f"{what} lse", TOL_LSE)
        say(f"    bit-identical to the caller-workspace call; max err out {e_o:.3e} lse {e_l:.3e}")


def test_noalloc_rejects_shapes_past_the_scratch():
    dev = device()
    B, Hq, Hkv = 3525, 32, 8  # needs just over 64 MiB of workspace
    q = torch.zeros(B, Hq, 128, dtype=torch.bfloat16, device=dev)
    kp = torch.zeros(1, Hkv, 16, 128, dtype=torch.bfloat16, device=dev)
    bt = torch.zeros(B, 1, dtype=torch.int32, device=dev)
    sl = torch.ones(B, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    say("[noalloc] shape past the 64 MiB scratch")
    with pytest.raises(A.AttnError) as ei:
        A.attn_decode_paged_noalloc(q, kp, kp, bt, sl, out)
    assert ei.value.status == A.ATTN_ERR_WORKSPACE
