"""The hot path under HIP graph capture: replays match eager launches bit for bit (called through the C ABI)."""

import pytest
import torch

import attention_causal_gqa_amd as A
from attention_causal_gqa_amd import synth
from tests._gpu import device, say

pytestmark = pytest.mark.gpu


def test_prefill_and_decode_graph_replays_match_eager():
    dev = device()
    pshape = synth.PrefillShape(1, 8, 2, 300, 128, torch.bfloat16)
    q, k, v = (t.to(dev) for t in synth.prefill_inputs(pshape, seed=21))
    out = torch.empty_like(q)
    lse = torch.empty(1, 8, 300, dtype=torch.float32, device=dev)
    dshape = synth.DecodeShape(6, 8, 2, 128, 16, 1, 900, torch.bfloat16)
    inp = synth.paged_inputs(dshape, seed=22, poison=float("nan"))
    dq, kp, vp, bt, sl = (t.to(dev) for t in (inp.q, inp.k_pages, inp.v_pages, inp.block_table, inp.seq_lens))
    dout = torch.empty_like(dq)
    dlse = torch.empty(6, 8, dtype=torch.float32, device=dev)
    need = A.attn_decode_workspace_bytes(6, 8, 2, 128, 16, inp.max_pages_per_seq, 0)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    scale = synth.fp32_scale(128)

    def work():
        A.attn_prefill(q, k, v, out=out, lse=lse, scale=scale)
        A.attn_decode_paged(dq, kp, vp, bt, sl, out=dout, lse=dlse, scale=scale, workspace=ws)

    say("[graph] eager reference")
    work()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, dout, dlse)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for r in range(4):
        say(f"[graph] replay {r}")
        for t in (out, lse, dout, dlse):
            t.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("out", "lse", "dout", "dlse"), (out, lse, dout, dlse), ref):
            assert torch.equal(got, want), f"replay {r}: {name} differs from the eager launch"


def test_fused_append_graph_replays_rewrite_the_cache():
    """The fused append + chunked prefill under capture: before every replay the chunk's slots are set back
    to NaN and the outputs cleared, and every replay must write the same slots and outputs as the eager call."""
    dev = device()
    shp = synth.ChunkShape(3, 8, 2, 100, 128, synth.PAGE_SIZE, 100, 700, torch.bfloat16)
    inp = synth.fused_inputs(shp, seed=23, poison=float("nan"), stale=float("nan"))
    q, kn, vn, kp, vp, bt, sl = (t.to(dev) for t in (inp.q, inp.k_new, inp.v_new, inp.k_pages, inp.v_pages,
                                                     inp.block_table, inp.seq_lens))
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    pages, slots = (t.to(dev) for t in synth.chunk_slots(inp.block_table, inp.seq_lens, 100, synth.PAGE_SIZE))
    scale = synth.fp32_scale(128)

    def work():
        A.attn_prefill_paged_append(q, kn, vn, kp, vp, bt, sl, out=out, lse=lse, scale=scale)

    say("[graph] fused append: eager reference")
    work()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, kp, vp)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for r in range(4):
        say(f"[graph] fused append: replay {r}")
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        kp[pages, :, slots] = float("nan")  # eager work between replays: the chunk's slots are stale again
        vp[pages, :, slots] = float("nan")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("out", "lse", "k_pages", "v_pages"), (out, lse, kp, vp), ref):
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want), \
                f"replay {r}: {name} differs from the eager launch"


def test_decode_append_graph_replays_rewrite_the_cache():
    """The decode with the fused append under capture: before every replay the newest tokens' slots are set
    back to NaN and the outputs cleared; every replay must write the same slots and outputs as the eager call."""
    dev = device()
    shp = synth.DecodeShape(6, 8, 2, 128, 16, 1, 900, torch.bfloat16)
    inp, kn, vn = synth.decode_append_inputs(shp, seed=24, poison=float("nan"), stale=float("nan"))
    q, kp, vp, bt, sl = (t.to(dev) for t in (inp.q, inp.k_pages, inp.v_pages, inp.block_table, inp.seq_lens))
    kn, vn = kn.to(dev), vn.to(dev)
    out = torch.empty_like(q)
    lse = torch.empty(6, 8, dtype=torch.float32, device=dev)
    ws = torch.empty(A.attn_decode_workspace_bytes(6, 8, 2, 128, 16, inp.max_pages_per_seq, 0), dtype=torch.uint8,
                     device=dev)
    L = inp.seq_lens.long()
    pages = inp.block_table.long()[torch.arange(6), (L - 1) // 16].to(dev)
    slots = ((L - 1) % 16).to(dev)
    scale = synth.fp32_scale(128)

    def work():
        A.attn_decode_paged_append(q, kn, vn, kp, vp, bt, sl, out=out, lse=lse, scale=scale, workspace=ws)

    say("[graph] decode append: eager reference")
    work()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, kp, vp)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for r in range(4):
        say(f"[graph] decode append: replay {r}")
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        kp[pages, :, slots] = float("nan")
        vp[pages, :, slots] = float("nan")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("out", "lse", "k_pages", "v_pages"), (out, lse, kp, vp), ref):
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want), \
                f"replay {r}: {name} differs from the eager launch"
