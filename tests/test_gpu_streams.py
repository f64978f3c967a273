"""Prefill and decode on two HIP streams (the benchmark's step schedule) give the outputs of one stream, bit for bit
(called through the C ABI)."""

import pytest
import torch

import attention_causal_gqa_amd as A
from attention_causal_gqa_amd import synth
from tests._gpu import device, say

pytestmark = pytest.mark.gpu


def test_prefill_and_decode_on_two_streams_match_one_stream():
    dev = device()
    pshape = synth.PrefillShape(1, 8, 2, 1000, 128, torch.bfloat16)
    q, k, v = (t.to(dev) for t in synth.prefill_inputs(pshape, seed=41))
    out = torch.empty_like(q)
    lse = torch.empty(1, 8, 1000, dtype=torch.float32, device=dev)
    dshape = synth.DecodeShape(16, 8, 2, 128, 16, 1, 3000, torch.bfloat16)
    inp = synth.paged_inputs(dshape, seed=42, poison=float("nan"))
    dq, kp, vp, bt, sl = (t.to(dev) for t in (inp.q, inp.k_pages, inp.v_pages, inp.block_table, inp.seq_lens))
    dout = torch.empty_like(dq)
    dlse = torch.empty(16, 8, dtype=torch.float32, device=dev)
    need = A.attn_decode_workspace_bytes(16, 8, 2, 128, 16, inp.max_pages_per_seq, 0)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    scale = synth.fp32_scale(128)

    def prefill(stream=None):
        A.attn_prefill(q, k, v, out=out, lse=lse, scale=scale, stream=stream)

    def decode(stream=None):
        A.attn_decode_paged(dq, kp, vp, bt, sl, out=dout, lse=dlse, scale=scale, workspace=ws, stream=stream)

    say("[streams] one stream")
    decode()
    prefill()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, dout, dlse)]
    main = torch.cuda.current_stream()
    sp, sd = torch.cuda.Stream(), torch.cuda.Stream()
    for r in range(5):
        say(f"[streams] two streams, step {r}")
        for t in (out, lse, dout, dlse):
            t.fill_(float("nan"))
        start = torch.cuda.Event()
        start.record(main)
        sd.wait_event(start)
        sp.wait_event(start)
        decode(sd)
        prefill(sp)
        done_d, done_p = torch.cuda.Event(), torch.cuda.Event()
        done_d.record(sd)
        done_p.record(sp)
        main.wait_event(done_d)
        main.wait_event(done_p)
        torch.cuda.synchronize()
        for got, want in zip((out, lse, dout, dlse), ref):
            assert torch.equal(got, want)


def test_decode_on_a_side_stream_without_workspace():
    """workspace=None on a stream other than the current one: the binding allocates the workspace on the
    launch stream, so memory the current stream allocates and overwrites right after the call (the same
    size, freed and reused at once by torch's caching allocator if the two shared a pool) cannot be the
    workspace the kernels are still using."""
    dev = device()
    dshape = synth.DecodeShape(64, 32, 8, 128, 16, 2000, 4000, torch.bfloat16)
    inp = synth.paged_inputs(dshape, seed=43, poison=float("nan"))
    dq, kp, vp, bt, sl = (t.to(dev) for t in (inp.q, inp.k_pages, inp.v_pages, inp.block_table, inp.seq_lens))
    scale = synth.fp32_scale(128)
    ref_o, ref_l = A.attn_decode_paged(dq, kp, vp, bt, sl, scale=scale)
    torch.cuda.synchronize()
    need = A.attn_decode_workspace_bytes(64, 32, 8, 128, 16, inp.max_pages_per_seq, 0)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    for r in range(4):
        say(f"[streams] side-stream decode without workspace, round {r}")
        out = torch.empty_like(dq)
        lse = torch.empty(64, 32, dtype=torch.float32, device=dev)
        side.wait_stream(main)
        A.attn_decode_paged(dq, kp, vp, bt, sl, out=out, lse=lse, scale=scale, stream=side)
        junk = torch.empty(need, dtype=torch.uint8, device=dev)  # on the current stream
        junk.fill_(0xFF)
        main.wait_stream(side)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
