"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path over the mixed long-context workload:
causal GQA prefill (B1 Hq32 Hkv8 T8192 d128, bf16) and paged single-token
decode (B64 Hq32 Hkv8 d128, page 16, seq_lens ~ U[1024, 8192]), i.e. the
prefill kernel, the split-KV decode kernel and the LSE combine kernel.  The
two parts are independent, so by default they run on two HIP streams (the
HBM-bound decode launched first, beside the MFMA-bound prefill) joined once
per step; ``--sequential`` runs them one after the other.  Inputs are seeded
synthetic tensors, resident in HBM before timing.

Prints one JSON line.  ``value`` is the step's roofline fraction: the time the
step's algorithmic work takes at MI355X peak (prefill flops at the bf16 MFMA
peak plus decode bytes at the HBM peak) divided by the measured step time.
After the warm-up, untimed steps run until 30 have run in all and the GPU
has been busy for 0.5 s (its speed settles over the first tens of ms).  The timed region is exactly K
steps between two synchronizations: ``ms_per_step`` is their host-clock
time, and ``kernel_ms_per_step`` the time between two timing markers on the
launch stream before the first and after the last of those steps (with
``--flush``, a marker pair around each step, after its flush).  The
per-step median, p90 and minimum in ``step_events`` come from a later pass
of K steps with one marker at each step's end.
Per-part times come from a later pass of K steps with events around each
part; in the two-stream step those events slow the step, so per-part times
there are upper bounds.  A workload with a single part also times K
back-to-back launches between one pair of events, and in a two-part step
the dominant kernel is timed alone that way: ``roofline.achieved`` is its
average launch duration.  These passes run in the steady state the timed
region leaves (no GPU sleep before them, which would let the idle GPU boost
its clock), except where the host issues a step more slowly than the GPU
runs it.  ``environment`` names the GPU, ROCm and torch, and the GFX clock
amdsmi reports while the dominant kernel runs.

    python bench.py [--steps K] [--warmup W] [--workload 5|3|4|6|7|8|9|10|11|12] [--no-cpu-baseline] [--flush]

``--flush`` reads a 512 MiB buffer before every step (outside the events),
so that a decode whose K/V would fit in the 256 MB MALL (workload 4) starts
cold; ``value`` then comes from the kernels' event time.

Workload 6 (not the default) times the chunked prefill over a paged cache:
2048-token chunks at the end of four sequences of 4096..16384 cached tokens.
Workload 7 times the KV append that writes such chunks into the cache, and
workload 11 the two in one launch (the chunk's keys and values arriving as
dense tensors, read from there and written into the cache by the prefill).
Workload 12 times workload 4's decode with each sequence's newest token
appended by the same two launches.
Workload 8 times the ragged prefill of 16 sequences of 256..4096 tokens
packed along the token axis.  Workload 9 times the paged decode of workload
5 over an FP8 E4M3 cache (algorithmic bytes: one byte per cached value).
Workload 10 times a serving-size decode batch: 1024 sequences of 16..512
tokens (Hq32 Hkv8 d128).
    python bench.py --copy-calibration   # plain 1 GiB copy, reference for HBM byte counters
    python bench.py --read-ceiling       # plain reads: 2 GiB, and the decode slices of workloads 5 and 9
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import attention_causal_gqa_amd as A  # noqa: E402
from attention_causal_gqa_amd import synth  # noqa: E402

PEAK_BF16_FLOPS = 2.5e15  # MI355X dense bf16 MFMA, published
PEAK_HBM_BYTES = 8.0e12   # MI355X HBM3E, published
METRIC = "prefill TFLOP/s and paged-decode HBM GB/s, as fraction of MI355X peak"
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
SETTLE_STEPS = 30  # untimed steps (warm-up included) before the timed region, at least
SETTLE_SECONDS = 0.5  # and at least this much GPU-busy time


def environment():
    """GPU, ROCm and torch versions of this run."""
    props = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"gpu": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "rocm": rocm, "hip_runtime": torch.version.hip,
            "torch": torch.__version__}


def sample_gfx_clock(launch, seconds=1.5, skip=0.8):
    """GFX clock (MHz) and socket power (W) that amdsmi reports while `launch` runs back to back for `seconds`,
    or None when amdsmi is not usable on this host.  The firmware's metrics table lags the GPU by about half a
    second (the reading stayed at its idle value for ~0.5 s after a kernel loop started), so samples from the
    first `skip` seconds are dropped.  Per-XCD current clocks when the table has them, else the single current
    clock; the power cap beside the power, so a kernel held at the cap shows as such."""
    try:
        import threading

        import amdsmi

        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
        samples, watts, done = [], [], threading.Event()
        t_start = time.perf_counter()

        def power():
            try:
                w = amdsmi.amdsmi_get_power_info(handle).get("current_socket_power")
                return float(w) if isinstance(w, (int, float)) and w > 0 else None
            except Exception:
                return None

        def read():
            try:
                xcds = amdsmi.amdsmi_get_gpu_metrics_info(handle).get("current_gfxclks")
                xcds = [float(c) for c in xcds if isinstance(c, (int, float)) and 0 < c < 65535]
                if xcds:
                    return xcds
            except Exception:
                pass
            c = amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.GFX)["clk"]
            return [float(c)] if isinstance(c, (int, float)) and c > 0 else None

        def poll():
            while not done.is_set():
                t = time.perf_counter() - t_start
                try:
                    v = read()
                    if v is not None and t >= skip:
                        samples.append(v)
                    w = power() if t >= skip else None
                    if w is not None:
                        watts.append(w)
                except Exception:
                    pass
                time.sleep(0.01)

        torch.cuda.synchronize()
        th = threading.Thread(target=poll)
        th.start()
        while time.perf_counter() - t_start < seconds:
            for _ in range(8):
                launch()
            torch.cuda.synchronize()
        done.set()
        th.join()
        cap = None
        try:
            c = amdsmi.amdsmi_get_power_cap_info(handle).get("power_cap")
            cap = round(float(c) / 1e6, 1) if isinstance(c, (int, float)) and c > 0 else None  # reported in uW
        except Exception:
            pass
        amdsmi.amdsmi_shut_down()
        if not samples:
            return None
        means = [float(np.mean(v)) for v in samples]
        return {"mhz_median": round(float(np.median(means)), 1), "mhz_min": round(float(min(means)), 1),
                "per_xcd_last": samples[-1], "samples": len(samples),
                "socket_w_median": round(float(np.median(watts)), 1) if watts else None, "power_cap_w": cap,
                "note": f"amdsmi current GFX clock (mean over XCDs) and socket power while the dominant kernel ran "
                        f"back to back; samples after the first {skip} s of {seconds} s"}
    except Exception:
        return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", type=int, default=5, choices=(3, 4, 5, 6, 7, 8, 9, 10, 11, 12))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--sequential", action="store_true",
                   help="run the parts of a two-part step (workload 5) one after the other on one stream; by default "
                        "the decode and the prefill run on two HIP streams, joined once per step")
    p.add_argument("--flush", action="store_true",
                   help="read a 512 MiB buffer before each step (outside the kernel events) to evict L2/MALL")
    p.add_argument("--no-clock", action="store_true",
                   help="skip the GFX clock sample (1.5 s of the dominant kernel back to back after the timed region); "
                        "the kernel-trace profiles use it so that their per-kernel averages cover the benchmark's "
                        "own launches only")
    p.add_argument("--read-ceiling", action="store_true",
                   help="only time plain reads: a 2 GiB buffer, and workload 5's K/V page slices in decode order")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy ten times (reference for the HBM byte counters)")
    return p.parse_args()


COPY_BYTES = 1 << 30


def copy_calibration():
    """A plain copy of known size: every launch reads and writes COPY_BYTES.  Profiling this run with
    rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) gives the scale from counter bytes to HBM bytes."""
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_launch": COPY_BYTES, "bytes_written_per_launch": COPY_BYTES,
                                           "launches": 10}}), flush=True)


def read_ceiling(args):
    """The practical HBM read ceiling: a kernel that only reads (libattn_probe.so), timed with HIP events
    over K launches, on (1) a 2 GiB buffer in 4 KiB slices, (2) the 4 KiB K and V slices of workload 5's
    decode pool and (3) the 2 KiB K and V slices of workload 9's FP8 pool, (sequence, kv head, page) in the
    streaming decode's order, from pools far larger than the MALL; each with ordinary and with non-temporal
    16-byte loads.  Context for the decode's rate, not a replacement for the 8 TB/s peak."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "attention_causal_gqa_amd", "libattn_probe.so"))
    vp = ctypes.c_void_p
    lib.probe_read_slices.argtypes = [vp, vp, ctypes.c_longlong, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, vp]
    lib.probe_read_slices.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count * 8
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def timed(base, offs, n, slice_bytes, nt):
        def go():
            rc = lib.probe_read_slices(base.data_ptr(), None if offs is None else offs.data_ptr(), n, slice_bytes,
                                       sink.data_ptr(), blocks, nt, ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"probe_read_slices failed: {rc}")
        for _ in range(args.warmup):
            go()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            go()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        return {"slices": int(n), "slice_bytes": slice_bytes, "bytes": int(n) * slice_bytes,
                "loads": "non-temporal" if nt else "ordinary", "ms": round(ms, 4),
                "gbps": round(n * slice_bytes / (ms / 1e3) / 1e9, 1)}

    def both(name, base, offs, n, slice_bytes):
        out[name] = timed(base, offs, n, slice_bytes, 0)
        out[name + "_nt"] = timed(base, offs, n, slice_bytes, 1)

    def decode_slices(seq_lens, block_table, P, Hkv, page_size, slice_bytes):
        """Byte offsets of the K and V slices one decode reads, in its order, in a K pool then V pool."""
        offs = []
        for b in range(seq_lens.shape[0]):
            n = (int(seq_lens[b]) + page_size - 1) // page_size
            pages = block_table[b, :n].long()
            for kvh in range(Hkv):
                ko = (pages * Hkv + kvh) * slice_bytes
                offs.append(torch.stack([ko, ko + P * Hkv * slice_bytes], dim=1).reshape(-1))
        return torch.cat(offs).to(dev)

    out = {}
    big = torch.ones(2 << 30, dtype=torch.uint8, device=dev)
    both("contiguous", big, None, big.numel() // 4096, 4096)
    del big
    shp = synth.WORKLOADS[5]["decode"]
    inp = synth.paged_inputs(shp, seed=105)
    P = inp.k_pages.shape[0]
    sb = shp.page_size * shp.d * 2
    pool = torch.ones(2 * P * shp.Hkv * sb, dtype=torch.uint8, device=dev)  # K pool, then V pool
    offs = decode_slices(inp.seq_lens, inp.block_table, P, shp.Hkv, shp.page_size, sb)
    both("decode_pages_w5", pool, offs, offs.numel(), sb)
    del pool, inp
    shp = synth.WORKLOADS[9]["decode_fp8"]
    inp = synth.fp8_paged_inputs(shp, seed=109)
    P = inp.k_codes.shape[0]
    sb = shp.page_size * shp.d
    pool = torch.ones(2 * P * shp.Hkv * sb, dtype=torch.uint8, device=dev)
    offs = decode_slices(inp.seq_lens, inp.block_table, P, shp.Hkv, shp.page_size, sb)
    both("decode_pages_w9_fp8", pool, offs, offs.numel(), sb)
    out.update({"blocks": blocks, "steps": args.steps})
    print(json.dumps({"read_ceiling": out}), flush=True)


def kernel_source_hash(names):
    """Hash of the kernels' code (comments and blank lines removed, so that a comment edit keeps it)."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "attention_causal_gqa_amd", "csrc", n)) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel, src_hash):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it was taken on this source."""
    if not os.path.exists(PROFILE_COUNTERS):
        return None
    for line in open(PROFILE_COUNTERS):
        parts = line.split()
        if len(parts) == 5 and parts[0] == "traffic" and parts[1] == str(workload) and parts[2] == kernel \
                and parts[3] == src_hash:
            return int(parts[4])
    return None


def cpu_baseline(pre_inputs, pre_shape, dec_inputs, budget_s=20.0):
    """Time the fp64 oracle, as it stands, on a bounded sample of the same workload."""
    import oracle
    from threadpoolctl import threadpool_info

    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    q, k, v = pre_inputs
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    scale = synth.fp32_scale(pre_shape.d)
    g = pre_shape.Hq // pre_shape.Hkv
    t0 = time.perf_counter()
    heads = 0
    flops = 0
    # prefill, one query head at a time (with its kv head), until half the budget is used
    while heads < pre_shape.Hq and (heads == 0 or time.perf_counter() - t0 < budget_s / 2):
        h = heads
        oracle.prefill(qn[:, h:h + 1], kn[:, h // g:h // g + 1], vn[:, h // g:h // g + 1], scale)
        flops += 2 * pre_shape.B * pre_shape.d * pre_shape.T * (pre_shape.T + 1)
        heads += 1
    t_pre = time.perf_counter() - t0
    seqs = 0
    dbytes = 0
    t1 = time.perf_counter()
    kp, vp = dec_inputs.k_pages.float().numpy(), dec_inputs.v_pages.float().numpy()
    t_conv = time.perf_counter() - t1
    t1 = time.perf_counter()
    B, Hq, d = dec_inputs.q.shape
    Hkv = dec_inputs.k_pages.shape[1]
    while seqs < B and (seqs == 0 or time.perf_counter() - t1 < budget_s / 2):
        b = seqs
        oracle.decode_paged(dec_inputs.q[b:b + 1].float().numpy(), kp, vp, dec_inputs.block_table[b:b + 1].numpy(),
                            dec_inputs.seq_lens[b:b + 1].numpy(), scale, dec_inputs.page_size)
        L = int(dec_inputs.seq_lens[b])
        dbytes += 2 * L * Hkv * d * 2 + 2 * Hq * d * 2 + 4 * (-(-L // 16)) + 4
        seqs += 1
    t_dec = time.perf_counter() - t1
    frac = (flops / PEAK_BF16_FLOPS + dbytes / PEAK_HBM_BYTES) / (t_pre + t_dec)
    return {
        "value": frac,
        "unit": "fraction of MI355X roofline",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"fp64 oracle: prefill of {heads} of {pre_shape.Hq} query heads at T={pre_shape.T} "
                   f"({t_pre:.2f} s) + paged decode of {seqs} of {B} sequences, all {Hq} heads ({t_dec:.2f} s); "
                   f"same seeded inputs"),
        "prefill_tflops": flops / t_pre / 1e12,
        "decode_gbps": dbytes / t_dec / 1e9,
        "host_cpu_count": os.cpu_count(),
        "pool_upcast_s": round(t_conv, 2),
    }


def cpu_baseline_chunk(inp, budget_s=20.0):
    """Time the fp64 oracle on a bounded sample of the chunked-prefill workload: sequence 0, head by head."""
    import oracle
    from threadpoolctl import threadpool_info

    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    B, Hq, Tq, d = inp.q.shape
    Hkv = inp.k_pages.shape[1]
    g = Hq // Hkv
    kp, vp = inp.k_pages.float().numpy(), inp.v_pages.float().numpy()
    L = int(inp.seq_lens[0])
    scale = synth.fp32_scale(d)
    t0 = time.perf_counter()
    heads = 0
    while heads < Hq and (heads == 0 or time.perf_counter() - t0 < budget_s):
        h = heads
        oracle.prefill_paged(inp.q[0:1, h:h + 1].float().numpy(), kp[:, h // g:h // g + 1], vp[:, h // g:h // g + 1],
                             inp.block_table[0:1].numpy(), inp.seq_lens[0:1].numpy(), scale, inp.page_size)
        heads += 1
    t = time.perf_counter() - t0
    flops = heads * synth.chunk_flops(1, d, Tq, [L])
    return {"value": flops / t / PEAK_BF16_FLOPS, "unit": "fraction of MI355X roofline", "cores": threads,
            "kind": "oracle",
            "sample": f"fp64 oracle: chunked prefill of sequence 0 (L={L}), {heads} of {Hq} query heads ({t:.2f} s)",
            "chunk_tflops": flops / t / 1e12, "host_cpu_count": os.cpu_count()}


def cpu_baseline_fused(inp, budget_s=20.0):
    """Time the fp64 oracle on a bounded sample of the fused workload: sequence 0, query head by query
    head, each call appending that head's kv-head slice of the chunk and attending over the result."""
    import oracle
    from threadpoolctl import threadpool_info

    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    B, Hq, Tq, d = inp.q.shape
    Hkv = inp.k_pages.shape[1]
    g = Hq // Hkv
    kp, vp = inp.k_pages.float().numpy(), inp.v_pages.float().numpy()
    kn, vn = inp.k_new.float().numpy(), inp.v_new.float().numpy()
    L = int(inp.seq_lens[0])
    scale = synth.fp32_scale(d)
    t0 = time.perf_counter()
    heads = 0
    while heads < Hq and (heads == 0 or time.perf_counter() - t0 < budget_s):
        h, kv = heads, heads // g
        oracle.prefill_paged_append(inp.q[0:1, h:h + 1].float().numpy(), kn[0:1, kv:kv + 1], vn[0:1, kv:kv + 1],
                                    kp[:, kv:kv + 1], vp[:, kv:kv + 1], inp.block_table[0:1].numpy(),
                                    inp.seq_lens[0:1].numpy(), scale, inp.page_size)
        heads += 1
    t = time.perf_counter() - t0
    flops = heads * synth.chunk_flops(1, d, Tq, [L])
    return {"value": flops / t / PEAK_BF16_FLOPS, "unit": "fraction of MI355X roofline", "cores": threads,
            "kind": "oracle",
            "sample": f"fp64 oracle: KV append + chunked prefill of sequence 0 (L={L}), {heads} of {Hq} query heads "
                      f"({t:.2f} s)",
            "chunk_tflops": flops / t / 1e12, "host_cpu_count": os.cpu_count()}


def cpu_baseline_append(inp):
    """Time the oracle's KV append on the whole workload (bf16 values moved as 16-bit patterns)."""
    import oracle

    bits = lambda t: t.contiguous().view(torch.int16).numpy()
    kp, vp, kn, vn = bits(inp.k_pages), bits(inp.v_pages), bits(inp.k_new), bits(inp.v_new)
    t0 = time.perf_counter()
    oracle.kv_append(kp, vp, kn, vn, inp.block_table.numpy(), inp.seq_lens.numpy(), inp.page_size)
    t = time.perf_counter() - t0
    nbytes = inp.algorithmic_bytes()
    return {"value": nbytes / t / PEAK_HBM_BYTES, "unit": "fraction of MI355X roofline", "cores": 1, "kind": "oracle",
            "sample": f"oracle KV append of the whole workload ({t:.2f} s, including its copies of both pools)",
            "append_gbps": nbytes / t / 1e9, "host_cpu_count": os.cpu_count()}


def cpu_baseline_varlen(var_in, shape, budget_s=20.0):
    """Time the fp64 oracle on a bounded sample of the ragged workload: whole sequences, shortest first."""
    import oracle
    from threadpoolctl import threadpool_info

    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    q, k, v, cu, _ = var_in
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    cu = cu.numpy()
    order = np.argsort(cu[1:] - cu[:-1])
    scale = synth.fp32_scale(shape.d)
    t0 = time.perf_counter()
    done = []
    for s in order:
        if done and time.perf_counter() - t0 > budget_s:
            break
        a, b = int(cu[s]), int(cu[s + 1])
        oracle.prefill_varlen(qn[a:b], kn[a:b], vn[a:b], np.array([0, b - a]), scale)
        done.append(b - a)
    t = time.perf_counter() - t0
    flops = synth.varlen_flops(shape.Hq, shape.d, done)
    return {"value": flops / t / PEAK_BF16_FLOPS, "unit": "fraction of MI355X roofline", "cores": threads,
            "kind": "oracle",
            "sample": f"fp64 oracle: {len(done)} of {len(order)} sequences, shortest first (lengths {done}; {t:.2f} s)",
            "varlen_tflops": flops / t / 1e12, "host_cpu_count": os.cpu_count()}


def cpu_baseline_decode_append(inp, kn, vn, budget_s=20.0):
    """Time the fp64 oracle's decode with the fused append on a bounded sample: sequences one at a time."""
    import oracle
    from threadpoolctl import threadpool_info

    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    kp, vp = inp.k_pages.float().numpy(), inp.v_pages.float().numpy()
    kn, vn = kn.float().numpy(), vn.float().numpy()
    scale = synth.fp32_scale(inp.q.shape[2])
    B, Hq, d = inp.q.shape
    Hkv = kp.shape[1]
    t0 = time.perf_counter()
    seqs = nbytes = 0
    while seqs < B and (seqs == 0 or time.perf_counter() - t0 < budget_s):
        b = seqs
        oracle.decode_paged_append(inp.q[b:b + 1].float().numpy(), kn[b:b + 1], vn[b:b + 1], kp, vp,
                                   inp.block_table[b:b + 1].numpy(), inp.seq_lens[b:b + 1].numpy(), scale,
                                   inp.page_size)
        L = int(inp.seq_lens[b])
        nbytes += 2 * L * Hkv * d * 2 + 2 * Hq * d * 2 + 4 * (-(-L // 16)) + 4 + 2 * Hkv * d * 2
        seqs += 1
    t = time.perf_counter() - t0
    return {"value": nbytes / t / PEAK_HBM_BYTES, "unit": "fraction of MI355X roofline", "cores": threads,
            "kind": "oracle", "sample": f"fp64 oracle decode with the append of {seqs} of {B} sequences ({t:.2f} s, "
                                        f"each call copying both pools)",
            "decode_gbps": nbytes / t / 1e9, "host_cpu_count": os.cpu_count()}


def cpu_baseline_fp8(inp, budget_s=20.0):
    """Time the fp64 oracle's FP8 decode on a bounded sample: sequences one at a time."""
    import oracle
    from threadpoolctl import threadpool_info

    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    kc, vc = inp.k_codes.numpy(), inp.v_codes.numpy()
    scale = synth.fp32_scale(inp.q.shape[2])
    B, Hq, d = inp.q.shape
    Hkv = kc.shape[1]
    t0 = time.perf_counter()
    seqs = nbytes = 0
    while seqs < B and (seqs == 0 or time.perf_counter() - t0 < budget_s):
        b = seqs
        oracle.decode_paged_fp8(inp.q[b:b + 1].float().numpy(), kc, vc, inp.k_scale, inp.v_scale,
                                inp.block_table[b:b + 1].numpy(), inp.seq_lens[b:b + 1].numpy(), scale, inp.page_size)
        L = int(inp.seq_lens[b])
        nbytes += 2 * L * Hkv * d + 2 * Hq * d * 2 + 4 * (-(-L // 16)) + 4
        seqs += 1
    t = time.perf_counter() - t0
    return {"value": nbytes / t / PEAK_HBM_BYTES, "unit": "fraction of MI355X roofline", "cores": threads,
            "kind": "oracle", "sample": f"fp64 oracle FP8 decode of {seqs} of {B} sequences ({t:.2f} s, pools "
                                        f"decoded from codes inside each call)",
            "decode_gbps": nbytes / t / 1e9, "host_cpu_count": os.cpu_count()}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the attention path has no multi-GPU "
                                   "code; run without --gpus or with --gpus 1"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.read_ceiling:
        read_ceiling(args)
        return
    dev = torch.device("cuda:0")
    A.load_library()
    wl = synth.WORKLOADS[args.workload]
    pre_shape = wl.get("prefill")
    dec_shape = wl.get("decode")
    chunk_shape = wl.get("chunk")
    app_shape = wl.get("append")
    var_shape = wl.get("varlen")
    f8_shape = wl.get("decode_fp8")
    fu_shape = wl.get("fused")
    da_shape = wl.get("decode_append")

    pre_inputs = dec_inputs = chunk_in = app_in = var_in = f8_in = fu_in = da_in = None
    work = {}
    if pre_shape is not None:
        pre_inputs = synth.prefill_inputs(pre_shape, seed=args.workload)
        q, k, v = (t.to(dev) for t in pre_inputs)
        out = torch.empty_like(q)
        lse = torch.empty(pre_shape.B, pre_shape.Hq, pre_shape.T, dtype=torch.float32, device=dev)
        scale = synth.fp32_scale(pre_shape.d)
        work["prefill"] = lambda: A.attn_prefill(q, k, v, out=out, lse=lse, scale=scale)
    if dec_shape is not None:
        dec_inputs = synth.paged_inputs(dec_shape, seed=100 + args.workload)
        dq, kp, vp, bt, sl = (t.to(dev) for t in (dec_inputs.q, dec_inputs.k_pages, dec_inputs.v_pages,
                                                  dec_inputs.block_table, dec_inputs.seq_lens))
        dout = torch.empty_like(dq)
        dlse = torch.empty(dq.shape[0], dq.shape[1], dtype=torch.float32, device=dev)
        W = dec_inputs.max_pages_per_seq
        need = A.attn_decode_workspace_bytes(dec_shape.B, dec_shape.Hq, dec_shape.Hkv, dec_shape.d,
                                             dec_shape.page_size, W, 0)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        dscale = synth.fp32_scale(dec_shape.d)
        work["decode"] = lambda: A.attn_decode_paged(dq, kp, vp, bt, sl, out=dout, lse=dlse, scale=dscale,
                                                     workspace=ws)
    if chunk_shape is not None:
        chunk_in = synth.chunk_inputs(chunk_shape, seed=args.workload)
        cq, ckp, cvp, cbt, csl = (t.to(dev) for t in (chunk_in.q, chunk_in.k_pages, chunk_in.v_pages,
                                                      chunk_in.block_table, chunk_in.seq_lens))
        cout = torch.empty_like(cq)
        clse = torch.empty(cq.shape[:3], dtype=torch.float32, device=dev)
        cscale = synth.fp32_scale(chunk_shape.d)
        work["chunk"] = lambda: A.attn_prefill_paged(cq, ckp, cvp, cbt, csl, out=cout, lse=clse, scale=cscale)
    if app_shape is not None:
        app_in = synth.append_inputs(app_shape, seed=args.workload)
        akn, avn, akp, avp, abt, asl = (t.to(dev) for t in (app_in.k_new, app_in.v_new, app_in.k_pages,
                                                            app_in.v_pages, app_in.block_table, app_in.seq_lens))
        work["append"] = lambda: A.attn_kv_append(akn, avn, akp, avp, abt, asl)
    if fu_shape is not None:
        # The launch rewrites the chunk's slots with the same values at every
        # step, and reads the chunk's keys from k_new / v_new: steps repeat
        # exactly.
        fu_in = synth.fused_inputs(fu_shape, seed=args.workload)
        uq, ukn, uvn, ukp, uvp, ubt, usl = (t.to(dev) for t in (fu_in.q, fu_in.k_new, fu_in.v_new, fu_in.k_pages,
                                                                fu_in.v_pages, fu_in.block_table, fu_in.seq_lens))
        uout = torch.empty_like(uq)
        ulse = torch.empty(uq.shape[:3], dtype=torch.float32, device=dev)
        uscale = synth.fp32_scale(fu_shape.d)
        work["fused"] = lambda: A.attn_prefill_paged_append(uq, ukn, uvn, ukp, uvp, ubt, usl, out=uout, lse=ulse,
                                                            scale=uscale)
    if da_shape is not None:
        # Every step writes the same newest tokens into the same slots, and
        # the decode reads them from k_new / v_new: steps repeat exactly.
        da_in, da_kn, da_vn = synth.decode_append_inputs(da_shape, seed=100 + args.workload)
        eq, ekp, evp, ebt, esl, ekn, evn = (t.to(dev) for t in (da_in.q, da_in.k_pages, da_in.v_pages,
                                                                da_in.block_table, da_in.seq_lens, da_kn, da_vn))
        eout = torch.empty_like(eq)
        else_ = torch.empty(eq.shape[0], eq.shape[1], dtype=torch.float32, device=dev)
        eneed = A.attn_decode_workspace_bytes(da_shape.B, da_shape.Hq, da_shape.Hkv, da_shape.d, da_shape.page_size,
                                              da_in.max_pages_per_seq, 0)
        ews = torch.empty(eneed, dtype=torch.uint8, device=dev)
        escale = synth.fp32_scale(da_shape.d)
        work["decode_append"] = lambda: A.attn_decode_paged_append(eq, ekn, evn, ekp, evp, ebt, esl, out=eout,
                                                                   lse=else_, scale=escale, workspace=ews)
    if var_shape is not None:
        var_in = synth.varlen_inputs(var_shape, seed=args.workload)
        vq, vk, vv, vcu = (t.to(dev) for t in var_in[:4])
        vT = var_in[4]
        vout = torch.empty_like(vq)
        vlse = torch.empty(vq.shape[:2], dtype=torch.float32, device=dev)
        vscale = synth.fp32_scale(var_shape.d)
        work["varlen"] = lambda: A.attn_prefill_varlen(vq, vk, vv, vcu, vT, out=vout, lse=vlse, scale=vscale)
    if f8_shape is not None:
        f8_in = synth.fp8_paged_inputs(f8_shape, seed=100 + args.workload)
        fq, fkc, fvc, fbt, fsl = (t.to(dev) for t in (f8_in.q, f8_in.k_codes, f8_in.v_codes, f8_in.block_table,
                                                      f8_in.seq_lens))
        fout = torch.empty_like(fq)
        flse = torch.empty(fq.shape[0], fq.shape[1], dtype=torch.float32, device=dev)
        fneed = A.attn_decode_workspace_bytes(f8_shape.B, f8_shape.Hq, f8_shape.Hkv, f8_shape.d, f8_shape.page_size,
                                              f8_in.block_table.shape[1], 0)
        fws = torch.empty(fneed, dtype=torch.uint8, device=dev)
        fscale = synth.fp32_scale(f8_shape.d)
        work["decode_fp8"] = lambda: A.attn_decode_paged_fp8(fq, fkc, fvc, f8_in.k_scale, f8_in.v_scale, fbt, fsl,
                                                             out=fout, lse=flse, scale=fscale, workspace=fws)
    # --flush: a 512 MiB buffer, written once here and then only read before
    # each step.  Reading evicts the decode's K/V from L2 and the 256 MB MALL
    # without leaving dirty lines, whose write-back the timed kernels would
    # otherwise pay (a 512 MiB write before each step more than doubled the
    # workload-4 decode).
    flush_buf = torch.ones(128 << 20, dtype=torch.float32, device=dev) if args.flush else None
    flush_sink = torch.empty((), dtype=torch.float32, device=dev) if args.flush else None

    names = list(work)
    stream = torch.cuda.current_stream()
    # A two-part step (prefill of new tokens, decode of running sequences:
    # independent work) runs its parts on two HIP streams by default, the
    # HBM-bound decode launched first, so that it overlaps the MFMA-bound
    # prefill; the step ends when both are done.  Default stream priority.
    concurrent = len(names) > 1 and not args.sequential
    order = sorted(names, key=lambda n: 0 if n == "decode" else 1) if concurrent else names
    part_streams = {n: torch.cuda.Stream() for n in names} if concurrent else {}
    start_ev = torch.cuda.Event()
    done_ev = {n: torch.cuda.Event() for n in names}

    def step(events=None, seq=False, mark=None):
        """One step.  events: {part: (start, end)}, recorded around each part on the stream it runs on;
        mark: (start or None, end), recorded on the launch stream after the step's flush and at its end."""
        if flush_buf is not None:
            torch.sum(flush_buf, dim=0, out=flush_sink)
        if mark is not None and mark[0] is not None:
            mark[0].record(stream)
        if not concurrent or seq:
            for n in names:
                if events is not None:
                    events[n][0].record(stream)
                work[n]()
                if events is not None:
                    events[n][1].record(stream)
        else:
            start_ev.record(stream)
            for n in order:
                ps = part_streams[n]
                ps.wait_event(start_ev)
                with torch.cuda.stream(ps):
                    if events is not None:
                        events[n][0].record(ps)
                    work[n]()
                    if events is not None:
                        events[n][1].record(ps)
                done_ev[n].record(ps)
            for n in order:
                stream.wait_event(done_ev[n])
        if mark is not None:
            mark[1].record(stream)

    def timing_event():
        return torch.cuda.Event(enable_timing=True)

    def new_events():
        return {n: (timing_event(), timing_event()) for n in names}

    for _ in range(args.warmup):
        step()
    # Settling: the GPU's speed takes some time to settle once it is busy (the
    # step's event span fell from 0.83-0.89 ms to 0.78 ms over the first ~25
    # steps of workload 5; back-to-back workload-3 prefills took 95 us each
    # at first and ~80 us after some 100 launches), so untimed steps are
    # added until SETTLE_STEPS have run in all and the GPU has been busy for
    # SETTLE_SECONDS (steps issued in batches, each batch synchronized).
    settle = max(0, SETTLE_STEPS - args.warmup)
    for _ in range(settle):
        step()
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < SETTLE_SECONDS:
        for _ in range(8):
            step()
        settle += 8
        torch.cuda.synchronize()

    # Timed region: exactly K steps between two synchronizations on the host
    # clock, with one timing marker on the launch stream before the first
    # step and one after the last (with --flush, a marker after each step's
    # flush and one at each step's end, so that the flush stays out).  Events
    # around the parts on their own streams slowed the two-stream step of
    # workload 5 by about 7%, so they stay out of it.
    marks = [timing_event() for _ in range(args.steps + 1)]
    starts = [timing_event() if flush_buf is not None else None for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record(stream)
    for s in range(args.steps):
        step(mark=(starts[s], marks[s + 1]) if flush_buf is not None else None)
    if flush_buf is None:
        marks[args.steps].record(stream)
    issued = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if flush_buf is not None:
        step_events = np.asarray([starts[s].elapsed_time(marks[s + 1]) for s in range(args.steps)])
        step_ms = float(step_events.mean())
    else:
        step_ms = marks[0].elapsed_time(marks[args.steps]) / args.steps
        # The per-step distribution: K more steps with a marker at each end.
        marks2 = [timing_event() for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        marks2[0].record(stream)
        for s in range(args.steps):
            step(mark=(None, marks2[s + 1]))
        torch.cuda.synchronize()
        step_events = np.asarray([marks2[s].elapsed_time(marks2[s + 1]) for s in range(args.steps)])

    # The passes below time kernels back to back in the steady state the
    # timed region left behind.  A GPU sleep before a pass would let the
    # host queue every launch first, but the idle GPU then gains power
    # headroom and runs the following kernels at a boosted clock (workload 3:
    # 78 us per launch behind a sleep against 80-95 us back to back), so the
    # sleep is used only where the host issues a step more slowly than the GPU
    # runs it (then back-to-back launches would time the host).
    host_bound = issued / args.steps > 0.5 * step_ms / 1e3

    def lead_in():
        if host_bound:
            torch.cuda._sleep(200_000 * args.steps)

    # Per-part times (diagnostic, after the timed region): K more steps with
    # events around every part.  In a two-stream step these events slow the
    # step (see above): the per-part times inside it are upper bounds.
    evs = [new_events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    lead_in()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    per = {n: [evs[s][n][0].elapsed_time(evs[s][n][1]) for s in range(args.steps)] for n in names}
    ms = {n: float(np.mean(per[n])) for n in names}

    ms_alone = None
    if concurrent:  # each part alone (one after the other), for reference
        evs2 = [new_events() for _ in range(args.steps)]
        torch.cuda.synchronize()
        lead_in()
        for s in range(args.steps):
            step(evs2[s], seq=True)
        torch.cuda.synchronize()
        ms_alone = {n: float(np.mean([evs2[s][n][0].elapsed_time(evs2[s][n][1]) for s in range(args.steps)]))
                    for n in names}
    dom_block_ms = None
    if len(names) > 1 and flush_buf is None:
        # The dominant kernel alone, K back-to-back launches between one pair of
        # events on the launch stream: its average launch duration, which the
        # roofline uses (a per-step event pair would also hold the gap after
        # the other part's last kernel).
        dom = max(names, key=lambda n: ms[n])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        for _ in range(3):  # back to the steady state after the synchronization
            work[dom]()
        e0.record(stream)
        for _ in range(args.steps):
            work[dom]()
        e1.record(stream)
        torch.cuda.synchronize()
        dom_block_ms = e0.elapsed_time(e1) / args.steps
    if len(names) == 1 and flush_buf is None:
        # One part per step: also time K back-to-back launches between one pair of
        # events, so that a short kernel's time does not carry the cost of an
        # event pair per launch (a few microseconds).  (With --flush the
        # per-step event pairs are kept: they leave out each step's flush.)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        lead_in()
        if not host_bound:
            for _ in range(3):  # back to the steady state after the synchronization
                step()
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms[names[0]] = e0.elapsed_time(e1) / args.steps
    wall_seq = None
    if concurrent:  # the same K steps with the parts one after the other, for reference
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(seq=True)
        torch.cuda.synchronize()
        wall_seq = time.perf_counter() - t0
    # The shader clock while the dominant kernel runs back to back (sampled
    # through amdsmi, when the host offers it).
    dom_name = max(names, key=lambda n: ms[n])
    sclk = None if args.no_clock else sample_gfx_clock(work[dom_name])

    kernel_ms = step_ms
    ms_per_step = wall * 1e3 / args.steps

    def spread(n):
        """Min, median and 90th percentile of a part's per-step event times (the per-part pass)."""
        x = np.asarray(per[n])
        return {"ms_min": round(float(x.min()), 4), "ms_median": round(float(np.median(x)), 4),
                "ms_p90": round(float(np.percentile(x, 90)), 4)}

    result = {"metric": METRIC}
    at_peak = 0.0
    parts = {}
    if pre_shape is not None:
        flops = pre_shape.flops()
        t = ms["prefill"] / 1e3
        at_peak += flops / PEAK_BF16_FLOPS
        parts["prefill"] = {"ms": round(ms["prefill"], 4), **spread("prefill"),
                            "tflops": round(flops / t / 1e12, 1), "frac_of_peak": round(flops / t / PEAK_BF16_FLOPS, 4),
                            "flops_per_launch": flops}
    if dec_shape is not None:
        nbytes = dec_inputs.algorithmic_bytes()
        t = ms["decode"] / 1e3
        at_peak += nbytes / PEAK_HBM_BYTES
        parts["decode"] = {"ms": round(ms["decode"], 4), **spread("decode"),
                           "gbps": round(nbytes / t / 1e9, 1), "frac_of_peak": round(nbytes / t / PEAK_HBM_BYTES, 4),
                           "bytes_per_launch": nbytes, "kernels": "stream + combine",
                           "num_splits": A.attn_decode_num_splits(dec_shape.B, dec_shape.Hq, dec_shape.Hkv,
                                                                  dec_shape.d, dec_shape.page_size,
                                                                  dec_inputs.max_pages_per_seq, 0)}
    if chunk_shape is not None:
        flops = synth.chunk_flops(chunk_shape.Hq, chunk_shape.d, chunk_shape.Tq, chunk_in.seq_lens.tolist())
        t = ms["chunk"] / 1e3
        at_peak += flops / PEAK_BF16_FLOPS
        parts["chunk"] = {"ms": round(ms["chunk"], 4), **spread("chunk"),
                          "tflops": round(flops / t / 1e12, 1), "frac_of_peak": round(flops / t / PEAK_BF16_FLOPS, 4),
                          "flops_per_launch": flops}
    if da_shape is not None:
        # the decode's bytes (the newest token's K/V counted once, read from
        # k_new / v_new) plus the append's write of that token into the pools
        nbytes = da_in.algorithmic_bytes() + 2 * da_kn.numel() * da_kn.element_size()
        t = ms["decode_append"] / 1e3
        at_peak += nbytes / PEAK_HBM_BYTES
        parts["decode_append"] = {"ms": round(ms["decode_append"], 4), **spread("decode_append"),
                                  "gbps": round(nbytes / t / 1e9, 1),
                                  "frac_of_peak": round(nbytes / t / PEAK_HBM_BYTES, 4), "bytes_per_launch": nbytes,
                                  "kernels": "stream + combine (append forms)"}
    if fu_shape is not None:
        flops = synth.chunk_flops(fu_shape.Hq, fu_shape.d, fu_shape.Tq, fu_in.seq_lens.tolist())
        t = ms["fused"] / 1e3
        at_peak += flops / PEAK_BF16_FLOPS
        parts["fused"] = {"ms": round(ms["fused"], 4), **spread("fused"),
                          "tflops": round(flops / t / 1e12, 1), "frac_of_peak": round(flops / t / PEAK_BF16_FLOPS, 4),
                          "flops_per_launch": flops,
                          "append_bytes_per_launch": 2 * fu_in.k_new.numel() * fu_in.k_new.element_size()}
    if var_shape is not None:
        lens = (var_in[3][1:] - var_in[3][:-1]).tolist()
        flops = synth.varlen_flops(var_shape.Hq, var_shape.d, lens)
        t = ms["varlen"] / 1e3
        at_peak += flops / PEAK_BF16_FLOPS
        parts["varlen"] = {"ms": round(ms["varlen"], 4), **spread("varlen"),
                           "tflops": round(flops / t / 1e12, 1), "frac_of_peak": round(flops / t / PEAK_BF16_FLOPS, 4),
                           "flops_per_launch": flops}
    if f8_shape is not None:
        nbytes = f8_in.algorithmic_bytes()
        t = ms["decode_fp8"] / 1e3
        at_peak += nbytes / PEAK_HBM_BYTES
        parts["decode_fp8"] = {"ms": round(ms["decode_fp8"], 4), **spread("decode_fp8"),
                               "gbps": round(nbytes / t / 1e9, 1), "frac_of_peak": round(nbytes / t / PEAK_HBM_BYTES, 4),
                               "bytes_per_launch": nbytes, "kernels": "stream (FP8 form) + combine"}
    if app_shape is not None:
        nbytes = app_in.algorithmic_bytes()
        t = ms["append"] / 1e3
        at_peak += nbytes / PEAK_HBM_BYTES
        parts["append"] = {"ms": round(ms["append"], 4), **spread("append"),
                           "gbps": round(nbytes / t / 1e9, 1), "frac_of_peak": round(nbytes / t / PEAK_HBM_BYTES, 4),
                           "bytes_per_launch": nbytes}
    # With --flush the host-clock step includes the 512 MiB cache-evicting
    # write, which is not part of the path: the step is then the kernels'
    # event time.
    value = at_peak / ((kernel_ms if flush_buf is not None else ms_per_step) / 1e3)
    if ms_alone is not None:
        for n, pt in parts.items():
            pt["ms_alone"] = round(ms_alone[n], 4)
            pt["frac_of_peak_alone"] = round(pt["frac_of_peak"] * ms[n] / ms_alone[n], 4)

    # Dominant kernel's roofline (the one with the larger share of the step).
    dom = max(names, key=lambda n: ms[n])
    if dom in ("prefill", "chunk", "varlen", "fused"):
        src = kernel_source_hash(["prefill_bf16.hip", "device_common.h"])
        form = {"prefill": "", "chunk": " (paged form)", "varlen": " (packed form)", "fused": " (append form)"}[dom]
        roof = {"kernel": "prefill_bf16_kernel" + form, "bound": "mfma",
                "achieved": parts[dom]["tflops"], "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                "frac": round(parts[dom]["tflops"] * 1e12 / PEAK_BF16_FLOPS, 4),
                "traffic": measured_traffic(args.workload, "prefill_bf16_kernel", src), "source_hash": src}
    elif dom == "decode_fp8":
        src = kernel_source_hash(["decode_paged.hip", "device_common.h"])
        roof = {"kernel": "decode_stream_kernel+decode_combine_kernel (FP8 form)", "bound": "hbm",
                "achieved": parts["decode_fp8"]["gbps"], "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                "frac": round(parts["decode_fp8"]["gbps"] * 1e9 / PEAK_HBM_BYTES, 4),
                "traffic": measured_traffic(args.workload, "decode_stream_kernel+decode_combine_kernel", src),
                "source_hash": src}
    elif dom == "decode_append":
        src = kernel_source_hash(["decode_paged.hip", "device_common.h"])
        roof = {"kernel": "decode_stream_kernel+decode_combine_kernel (append form)", "bound": "hbm",
                "achieved": parts[dom]["gbps"], "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                "frac": round(parts[dom]["gbps"] * 1e9 / PEAK_HBM_BYTES, 4),
                "traffic": measured_traffic(args.workload, "decode_stream_kernel+decode_combine_kernel", src),
                "source_hash": src}
    elif dom == "append":
        src = kernel_source_hash(["kv_append.hip", "device_common.h"])
        roof = {"kernel": "kv_append_kernel", "bound": "hbm", "achieved": parts["append"]["gbps"],
                "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                "frac": round(parts["append"]["gbps"] * 1e9 / PEAK_HBM_BYTES, 4),
                "traffic": measured_traffic(args.workload, "kv_append_kernel", src), "source_hash": src}
    else:
        src = kernel_source_hash(["decode_paged.hip", "device_common.h"])
        roof = {"kernel": "decode_stream_kernel+decode_combine_kernel", "bound": "hbm",
                "achieved": parts["decode"]["gbps"], "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                "frac": round(parts["decode"]["gbps"] * 1e9 / PEAK_HBM_BYTES, 4),
                "traffic": measured_traffic(args.workload, "decode_stream_kernel+decode_combine_kernel", src),
                "source_hash": src}
    if dom_block_ms is not None:
        # In a two-part step the kernel's own rate is its average launch
        # duration alone (K back-to-back launches, measured in this run); with two
        # streams its duration inside the step is longer, as the parts share
        # the chip (achieved_in_step).
        r = ms[dom] / dom_block_ms
        roof["achieved_in_step"] = roof["achieved"]
        roof["achieved"] = round(roof["achieved"] * r, 1)
        roof["frac"] = round(roof["frac"] * r, 4)
        roof["timed"] = f"alone: {args.steps} back-to-back launches between one pair of HIP events"

    cfg = {"workload": synth.WORKLOAD_NAMES[args.workload]}
    if pre_shape is not None:
        cfg["seed_prefill"] = args.workload
    if dec_inputs is not None:
        cfg["seed_decode"] = 100 + args.workload
        cfg["decode_tokens"] = int(dec_inputs.seq_lens.sum())
    if f8_in is not None:
        cfg["seed_decode"] = 100 + args.workload
        cfg["decode_tokens"] = int(f8_in.seq_lens.sum())
        cfg["kv_format"] = "FP8 E4M3, per-tensor scales"
    if var_in is not None:
        cfg["seed_varlen"] = args.workload
        cfg["varlen_lens"] = (var_in[3][1:] - var_in[3][:-1]).tolist()
    if app_in is not None:
        cfg["seed_append"] = args.workload
        cfg["append_seq_lens"] = app_in.seq_lens.tolist()
    if chunk_in is not None:
        cfg["seed_chunk"] = args.workload
        cfg["chunk_seq_lens"] = chunk_in.seq_lens.tolist()
    if da_in is not None:
        cfg["seed_decode"] = 100 + args.workload
        cfg["decode_tokens"] = int(da_in.seq_lens.sum())
    if fu_in is not None:
        cfg["seed_fused"] = args.workload
        cfg["fused_seq_lens"] = fu_in.seq_lens.tolist()
    result.update({
        "value": round(value, 4),
        "unit": "fraction of MI355X roofline (step time at peak / measured step time)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "kernel_ms_per_step": round(kernel_ms, 4),
        "step_events": {"ms_median": round(float(np.median(step_events)), 4),
                        "ms_p90": round(float(np.percentile(step_events, 90)), 4),
                        "ms_min": round(float(step_events.min()), 4),
                        "note": ("marker pairs around each of the K timed steps, after the step's flush"
                                 if flush_buf is not None else
                                 "a later pass of K steps with a timing marker at each step's end")},
        "settle_steps": settle,
        "host_issue_ms_per_step": round(issued * 1e3 / args.steps, 4),
        **({"schedule": "decode and prefill on two HIP streams, joined once per step",
            "ms_per_step_sequential": round(wall_seq * 1e3 / args.steps, 4),
            "parts_timing": "per-part events in a later pass of K two-stream steps (events on the part streams "
                            "slow the step, so each part's ms is an upper bound); ms_alone: each part alone"}
           if concurrent else {}),
        **({"flush": "512 MiB read before each step (outside the kernel events); value from kernel_ms_per_step"}
           if flush_buf is not None else {}),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": cfg,
        "parts": parts,
        "roofline": roof,
        "environment": {**environment(), "gfx_clock_running_dominant": sclk},
    })
    if not args.no_cpu_baseline and args.workload == 5:
        result["cpu_baseline"] = cpu_baseline(pre_inputs, pre_shape, dec_inputs)
    if not args.no_cpu_baseline and args.workload == 6:
        result["cpu_baseline"] = cpu_baseline_chunk(chunk_in)
    if not args.no_cpu_baseline and args.workload == 7:
        result["cpu_baseline"] = cpu_baseline_append(app_in)
    if not args.no_cpu_baseline and args.workload == 12:
        result["cpu_baseline"] = cpu_baseline_decode_append(da_in, da_kn, da_vn)
    if not args.no_cpu_baseline and args.workload == 11:
        result["cpu_baseline"] = cpu_baseline_fused(fu_in)
    if not args.no_cpu_baseline and args.workload == 9:
        result["cpu_baseline"] = cpu_baseline_fp8(f8_in)
    if not args.no_cpu_baseline and args.workload == 8:
        result["cpu_baseline"] = cpu_baseline_varlen(var_in, var_shape)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
