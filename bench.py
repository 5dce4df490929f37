"""Benchmark of the exact-attention hot path on one MI355X.

One *step* is one ``mfa_fwd`` call over the dense causal prefill workload
(B=2, H=8, Nq=Nk=4096, D=128, fp16, causal; seeded synthetic inputs resident in HBM
before timing).  ``value`` is its throughput in TFLOP/s, counting 4*D FLOP per
*visible* (query, key) pair.  In the same run the other workloads are timed the same
way and reported under ``workloads``: the GQA long-context prefill (bf16, N=16384),
the sliding-window prefill (window (512, 0)), the paged split-KV decode (HBM
GB/s over the algorithmic bytes: every cached K/V byte once, plus q, out, LSE, the
block-table entries used and seq_lens), and the packed variable-length causal prefill
(``mfa_fwd_varlen``, 16 sequences of 256..4096 tokens, TFLOP/s over visible pairs), and
chunked prefill over the paged cache (``mfa_fwd_varlen_paged``, 8 sequences, new chunks
of 512..2048 tokens after 1024..16384 cached ones), and the 4-token verification decode
(``mfa_decode_paged_multi`` over the decode workload's cache shape, HBM GB/s), and the
block-sparse causal prefill (``mfa_fwd_ext`` with a 25%-dense 128 x 128 block mask,
TFLOP/s over the computed visible pairs), and the backward over the dense causal prefill
shape in bf16 (``mfa_bwd``: dQ and dK/dV launches; TFLOP/s at 10*D FLOP per visible
pair).

Timing: HIP events on the stream the kernels run on; per workload, W untimed warm-up
steps (continued until at least 30 ms of back-to-back calls have run, so that the clock
has settled), then K timed steps as one block between two events, then K more with each
call between its own pair of events; ``torch.cuda.synchronize()`` on both
sides of each timed region.  ``ms_per_step`` and ``value`` cover the block of K calls
(launch gaps included); the mean, median and min of the per-call event times are reported
beside it, and ``roofline.achieved`` divides the algorithmic work by the mean per-call
time (the kernel's average launch duration).  The dense-layout prefill entries also
carry ``roofline_model``: FLOP per algorithmic byte, the attainable TFLOP/s at that
intensity (the lesser of the MFMA peak and intensity x 8 TB/s) and the fraction reached.
``cpu_baseline`` times the float64 CPU oracle on this host over whole heads of the
same prefill workload, for about 10 s, scales to TFLOP/s, names the CPU model, and
reports the max-abs difference between the GPU's O and LSE and the oracle's on those
heads.

Usage: python bench.py [--steps K] [--warmup W] [--workloads NAME,...] [--no-cpu-baseline]
(workload names as in attn_inputs.WORKLOADS; default: all but tiny_dense)
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import attn_inputs as A  # noqa: E402

PEAK_MFMA_F16 = 2500.0   # TFLOP/s, MI355X dense fp16/bf16
PEAK_HBM = 8000.0        # GB/s, MI355X HBM3E

METRIC = "attn fwd TFLOP/s (D=128 causal fp16) + paged decode HBM GB/s, % roofline"
HEAD = "dense_causal_prefill"   # the workload whose throughput is `value`

# HBM traffic per launch measured with rocprofv3 counters (FETCH_SIZE / WRITE_SIZE,
# scaled by a plain copy kernel of known size) is kept in profiles/traffic.json
# together with a hash of the kernel sources it was measured on; it is reported only
# while the sources are unchanged.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "fwd": ["mfa_fwd.hip", "mfa_device.h", "mfa_geometry.h", "mfa_tile.h"],
    "decode": ["mfa_decode.hip", "mfa_device.h"],
    "bwd": ["mfa_bwd.hip", "mfa_device.h", "mfa_geometry.h", "mfa_tile.h"],
}


def sources_hash(kind):
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "exact_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(key, kind):
    """Bytes per launch recorded for `key`, or None if absent or measured on other sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("sources_sha256") != sources_hash(kind):
        return None
    return rec.get("bytes_per_launch")


def visible_pairs(Nq, Nk, causal, left, right) -> int:
    """Number of visible (query, key) pairs of one head (inclusive window ends)."""
    i = np.arange(Nq, dtype=np.int64)
    off = Nk - Nq
    lo = np.zeros(Nq, dtype=np.int64) if left < 0 else np.maximum(0, i + off - left)
    hi = np.full(Nq, Nk - 1, dtype=np.int64)
    if causal:
        hi = np.minimum(hi, i + off)
    if right >= 0:
        hi = np.minimum(hi, i + off + right)
    return int(np.maximum(hi - lo + 1, 0).sum())


def to_dev(bits, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16)


def time_calls(fn, steps):
    """Time `steps` back-to-back calls, twice.

    First as one block between two HIP events (ms per call with the launch gaps, the
    whole-job rate), then each call between its own pair of events (mean, median and min of
    the per-call times: the kernels' own duration).  Events are recorded on the current
    stream, the one the library launches on, with torch.cuda.synchronize() on both sides of
    each pass.  An event between every two calls adds a few microseconds of gap on this
    hardware, which is why the block is timed separately."""
    import torch
    torch.cuda.synchronize()
    b0 = torch.cuda.Event(enable_timing=True)
    b1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    b0.record()
    for _ in range(steps):
        fn()
    b1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for e0, e1 in ev:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    per = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    return {"ms_per_call": b0.elapsed_time(b1) / steps, "mean_ms": float(per.mean()),
            "median_ms": float(np.median(per)), "min_ms": float(per.min()), "wall_ms": wall}


WARM_MS = 30.0   # back-to-back work that brings the clock up after an idle gap


def warm_up(fn, n):
    """n untimed calls right before a workload's timed calls, continued (in groups of four)
    until at least WARM_MS of back-to-back calls have run: after an idle gap the clock
    takes some 20 ms of load to settle, which would otherwise show in the first timed
    calls of a long kernel."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        fn()
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < WARM_MS:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def timing_fields(t):
    return {k: t[k] for k in ("ms_per_call", "mean_ms", "median_ms", "min_ms", "wall_ms")}


def setup_prefill(name):
    """Device inputs and one step (one mfa_fwd call) of the named dense prefill workload."""
    import torch
    import exact_attention_amd as ea
    c = A.workload(name)
    x = A.workload_inputs(name)
    q, k, v = (to_dev(t, c["dtype"]) for t in (x.q, x.k, x.v))
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    del x

    step = ea.prepare(ea.mfa_fwd, q, k, v, scale=c["scale"], causal=c["causal"], win_left=c["left"],
                      win_right=c["right"], out=out, lse=lse)
    step.out, step.lse = out, lse
    return step


def prefill_bytes(c) -> int:
    """Algorithmic bytes of a dense prefill: q, k, v and out once each (2 bytes per element)
    and the fp32 LSE."""
    rows_q = c["B"] * c["Hq"] * c["Nq"]
    return 2 * c["D"] * (2 * rows_q + 2 * c["B"] * c["Hkv"] * c["Nk"]) + 4 * rows_q


def roofline_model(flop, nbytes, tflops):
    """The roofline at this workload's arithmetic intensity: attainable TFLOP/s is the lesser
    of the MFMA peak and intensity x peak HBM bandwidth (ridge 312.5 FLOP/B)."""
    inten = flop / nbytes
    att = min(PEAK_MFMA_F16, inten * PEAK_HBM / 1e3)
    return {"flop_per_byte": inten, "ridge_flop_per_byte": PEAK_MFMA_F16 * 1e3 / PEAK_HBM,
            "bound": "mfma" if att >= PEAK_MFMA_F16 else "hbm", "attainable_tflops": att,
            "frac_of_attainable": tflops / att}


def bench_prefill(name, step, steps):
    import exact_attention_amd as ea
    c = A.workload(name)
    t = time_calls(step, steps)
    ms = t["ms_per_call"]
    info = ea.mfa_last_dispatch()
    flop = 4.0 * c["D"] * visible_pairs(c["Nq"], c["Nk"], c["causal"], c["left"], c["right"]) \
        * c["B"] * c["Hq"]
    tf = flop / (ms * 1e-3) / 1e12
    tk = flop / (t["mean_ms"] * 1e-3) / 1e12
    return {
        "workload": f"{c['name']} B={c['B']} Hq={c['Hq']} Hkv={c['Hkv']} N={c['Nq']} D={c['D']} "
                    f"{c['dtype']} causal={int(c['causal'])} window=({c['left']},{c['right']})",
        "tflops": tf, **timing_fields(t), "flop": flop,
        "roofline": {"bound": "mfma", "achieved": tk, "peak": PEAK_MFMA_F16, "unit": "TFLOP/s",
                     "frac": tk / PEAK_MFMA_F16,
                     "traffic": measured_traffic(name, "fwd")},
        "roofline_model": roofline_model(flop, prefill_bytes(c), tk),
        "kernel": info["kernel"], "grid": info["grid"], "planned_tiles": info["planned"],
        "dtype": c["dtype"],
    }


def setup_varlen():
    """Device inputs and one step (one mfa_fwd_varlen call) of the packed workload."""
    import torch
    import exact_attention_amd as ea
    c = A.workload("packed_varlen_causal_prefill")
    x = A.workload_inputs("packed_varlen_causal_prefill")
    q, k, v = (to_dev(t, c["dtype"]) for t in (x.q, x.k, x.v))
    cq = torch.from_numpy(x.cu_seqlens_q).to("cuda")
    ck = torch.from_numpy(x.cu_seqlens_k).to("cuda")
    lq, lk = np.diff(x.cu_seqlens_q), np.diff(x.cu_seqlens_k)
    out = torch.empty_like(q)
    lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device="cuda")

    step = ea.prepare(ea.mfa_fwd_varlen, q, k, v, cq, ck, int(lq.max()), int(lk.max()),
                      scale=c["scale"], causal=c["causal"], win_left=c["left"],
                      win_right=c["right"], out=out, lse=lse)
    step.lens = (lq, lk)
    return step


def bench_varlen(step, steps):
    import exact_attention_amd as ea
    c = A.workload("packed_varlen_causal_prefill")
    t = time_calls(step, steps)
    ms = t["ms_per_call"]
    info = ea.mfa_last_dispatch()
    lq, lk = step.lens
    pairs = sum(visible_pairs(int(a), int(b), c["causal"], c["left"], c["right"]) for a, b in zip(lq, lk))
    flop = 4.0 * c["D"] * pairs * c["Hq"]
    tf = flop / (ms * 1e-3) / 1e12
    tk = flop / (t["mean_ms"] * 1e-3) / 1e12
    return {
        "workload": f"{c['name']} B={c['B']} Hq={c['Hq']} Hkv={c['Hkv']} D={c['D']} {c['dtype']} "
                    f"causal={int(c['causal'])} lengths in [{c['len_lo']},{c['len_hi']}] "
                    f"(total {int(lq.sum())} tokens)",
        "tflops": tf, **timing_fields(t), "flop": flop,
        "roofline": {"bound": "mfma", "achieved": tk, "peak": PEAK_MFMA_F16, "unit": "TFLOP/s",
                     "frac": tk / PEAK_MFMA_F16, "traffic": measured_traffic("packed_varlen_causal_prefill", "fwd")},
        "kernel": info["kernel"], "grid": info["grid"], "dtype": c["dtype"],
    }


def setup_chunked():
    """Device inputs and one step (one mfa_fwd_varlen_paged call) of the chunked prefill."""
    import torch
    import exact_attention_amd as ea
    c = A.workload("paged_chunked_prefill")
    p = A.workload_inputs("paged_chunked_prefill")
    q = to_dev(p.q, c["dtype"])
    kp = to_dev(p.k_pages, c["dtype"])
    vp = to_dev(p.v_pages, c["dtype"])
    bt = torch.from_numpy(p.block_table).to("cuda")
    sl = torch.from_numpy(p.seq_lens_k).to("cuda")
    cq = torch.from_numpy(p.cu_seqlens_q).to("cuda")
    lq = np.diff(p.cu_seqlens_q)
    out = torch.empty_like(q)
    lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device="cuda")

    step = ea.prepare(ea.mfa_fwd_varlen_paged, q, kp, vp, bt, sl, cq, int(lq.max()),
                      int(p.seq_lens_k.max()), scale=c["scale"], causal=c["causal"],
                      win_left=c["left"], win_right=c["right"], out=out, lse=lse)
    step.lens = (lq, p.seq_lens_k.astype(np.int64))
    return step


def bench_chunked(step, steps):
    import exact_attention_amd as ea
    c = A.workload("paged_chunked_prefill")
    t = time_calls(step, steps)
    ms = t["ms_per_call"]
    info = ea.mfa_last_dispatch()
    lq, lk = step.lens
    pairs = sum(visible_pairs(int(a), int(b), c["causal"], c["left"], c["right"]) for a, b in zip(lq, lk))
    flop = 4.0 * c["D"] * pairs * c["Hq"]
    tf = flop / (ms * 1e-3) / 1e12
    tk = flop / (t["mean_ms"] * 1e-3) / 1e12
    return {
        "workload": f"{c['name']} B={c['B']} Hq={c['Hq']} Hkv={c['Hkv']} D={c['D']} {c['dtype']} "
                    f"page=16 new tokens {int(lq.sum())} in chunks of [{c['new_lo']},{c['new_hi']}], "
                    f"cached keys {int(lk.sum())}",
        "tflops": tf, **timing_fields(t), "flop": flop,
        "roofline": {"bound": "mfma", "achieved": tk, "peak": PEAK_MFMA_F16, "unit": "TFLOP/s",
                     "frac": tk / PEAK_MFMA_F16, "traffic": measured_traffic("paged_chunked_prefill", "fwd")},
        "kernel": info["kernel"], "grid": info["grid"], "dtype": c["dtype"],
    }


def decode_bytes(p, Hkv, D, Hq, Nq=1):
    L = p.seq_lens.astype(np.int64)
    kv = int(L.sum()) * Hkv * D * 2 * 2
    B = len(L)
    qo = 2 * B * Nq * Hq * D * 2
    lse = B * Nq * Hq * 4
    bt = 4 * int(np.ceil(L / p.page_size).sum())
    return kv + qo + lse + bt + 4 * B


def setup_decode():
    """Device inputs and one step (one mfa_decode_paged call) of the paged decode workload."""
    import torch
    import exact_attention_amd as ea
    c = A.workload("paged_splitkv_decode")
    p = A.workload_inputs("paged_splitkv_decode")
    q = to_dev(p.q, c["dtype"])
    kp = to_dev(p.k_pages, c["dtype"])
    vp = to_dev(p.v_pages, c["dtype"])
    bt = torch.from_numpy(p.block_table).to("cuda")
    sl = torch.from_numpy(p.seq_lens).to("cuda")
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    nbytes = ea.mfa_decode_workspace_bytes(c["B"], c["Hq"], c["D"], 16, bt.shape[1], 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    step = ea.prepare(ea.mfa_decode_paged, q, kp, vp, bt, sl, scale=c["scale"], out=out, lse=lse,
                      workspace=ws)
    step.seq_lens = p.seq_lens
    step.page_size = p.page_size
    return step


def bench_decode(step, steps):
    import exact_attention_amd as ea
    c = A.workload("paged_splitkv_decode")
    t = time_calls(step, steps)
    ms = t["ms_per_call"]
    info = ea.mfa_last_dispatch()
    nb = decode_bytes(step, c["Hkv"], c["D"], c["Hq"])
    gbs = nb / (ms * 1e-3) / 1e9
    gk = nb / (t["mean_ms"] * 1e-3) / 1e9
    return {
        "workload": f"{c['name']} B={c['B']} Hq={c['Hq']} Hkv={c['Hkv']} D={c['D']} bf16 "
                    f"page=16 seq_lens in [1024,32768] (sum={int(step.seq_lens.sum())})",
        "gbs": gbs, **timing_fields(t), "bytes": nb,
        "roofline": {"bound": "hbm", "achieved": gk, "peak": PEAK_HBM, "unit": "GB/s",
                     "frac": gk / PEAK_HBM, "traffic": measured_traffic("paged_splitkv_decode", "decode")},
        "kernel": info["kernel"], "grid": info["grid"], "num_splits": info["num_splits"],
        "chunk_tokens": info["chunk_tokens"], "dtype": c["dtype"],
    }


def setup_multi():
    """Device inputs and one step (one mfa_decode_paged_multi call) of the 4-token decode."""
    import torch
    import exact_attention_amd as ea
    c = A.workload("paged_multi_query_decode")
    p = A.workload_inputs("paged_multi_query_decode")
    q = to_dev(p.q, c["dtype"])
    kp = to_dev(p.k_pages, c["dtype"])
    vp = to_dev(p.v_pages, c["dtype"])
    bt = torch.from_numpy(p.block_table).to("cuda")
    sl = torch.from_numpy(p.seq_lens).to("cuda")
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    nbytes = ea.mfa_decode_multi_workspace_bytes(c["B"], c["Nq"], c["Hq"], c["D"], 16, bt.shape[1], 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    step = ea.prepare(ea.mfa_decode_paged_multi, q, kp, vp, bt, sl, scale=c["scale"], out=out,
                      lse=lse, workspace=ws)
    step.seq_lens = p.seq_lens
    step.page_size = p.page_size
    return step


def bench_multi(step, steps):
    import exact_attention_amd as ea
    c = A.workload("paged_multi_query_decode")
    t = time_calls(step, steps)
    ms = t["ms_per_call"]
    info = ea.mfa_last_dispatch()
    nb = decode_bytes(step, c["Hkv"], c["D"], c["Hq"], c["Nq"])
    gbs = nb / (ms * 1e-3) / 1e9
    gk = nb / (t["mean_ms"] * 1e-3) / 1e9
    return {
        "workload": f"{c['name']} B={c['B']} Nq={c['Nq']} Hq={c['Hq']} Hkv={c['Hkv']} D={c['D']} bf16 "
                    f"page=16 seq_lens in [1024,32768] (sum={int(step.seq_lens.sum())})",
        "gbs": gbs, **timing_fields(t), "bytes": nb,
        "roofline": {"bound": "hbm", "achieved": gk, "peak": PEAK_HBM, "unit": "GB/s",
                     "frac": gk / PEAK_HBM, "traffic": measured_traffic("paged_multi_query_decode", "decode")},
        "kernel": info["kernel"], "grid": info["grid"], "num_splits": info["num_splits"],
        "chunk_tokens": info["chunk_tokens"], "dtype": c["dtype"],
    }


def block_sparse_pairs(bm, Nq, Nk, bq, bk):
    """Visible (query, key) pairs of a causal (Nq == Nk) attention under a block mask with
    square blocks: a block below the diagonal holds bq * bk pairs, a diagonal block
    bq (bq + 1) / 2 (full blocks only)."""
    assert Nq == Nk and bq == bk and Nq % bq == 0
    r = np.arange(bm.shape[-2])[:, None]
    c = np.arange(bm.shape[-1])[None, :]
    per_block = np.where(c < r, bq * bk, np.where(c == r, bq * (bq + 1) // 2, 0))
    return int((bm.astype(np.int64) * per_block).sum())


def setup_sparse():
    """Device inputs and one step (one mfa_fwd_ext call) of the block-sparse prefill."""
    import torch
    import exact_attention_amd as ea
    c = A.workload("block_sparse_causal_prefill")
    x = A.workload_inputs("block_sparse_causal_prefill")
    bm = A.block_mask_inputs(c["B"], c["Hq"], c["Nq"], c["Nk"], c["block_q"], c["block_k"],
                             c["density"], c["seed"] + 1000)
    q, k, v = (to_dev(t, c["dtype"]) for t in (x.q, x.k, x.v))
    bmd = torch.from_numpy(bm).to("cuda")
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")

    step = ea.prepare(ea.mfa_fwd_ext, q, k, v, scale=c["scale"], causal=True, block_mask=bmd,
                      block_q=c["block_q"], block_k=c["block_k"], out=out, lse=lse)
    step.pairs = block_sparse_pairs(bm, c["Nq"], c["Nk"], c["block_q"], c["block_k"])
    step.density = float(bm.mean())
    return step


def bench_sparse(step, steps):
    import exact_attention_amd as ea
    c = A.workload("block_sparse_causal_prefill")
    t = time_calls(step, steps)
    ms = t["ms_per_call"]
    info = ea.mfa_last_dispatch()
    flop = 4.0 * c["D"] * step.pairs
    tf = flop / (ms * 1e-3) / 1e12
    tk = flop / (t["mean_ms"] * 1e-3) / 1e12
    dense = 4.0 * c["D"] * visible_pairs(c["Nq"], c["Nk"], True, -1, -1) * c["B"] * c["Hq"]
    return {
        "workload": f"{c['name']} B={c['B']} H={c['Hq']} N={c['Nq']} D={c['D']} {c['dtype']} causal, "
                    f"{c['block_q']}x{c['block_k']} block mask, {step.density:.3f} of blocks on "
                    f"({step.pairs / (dense / (4.0 * c['D'])):.3f} of the causal pairs)",
        "tflops": tf, **timing_fields(t), "flop": flop,
        "roofline": {"bound": "mfma", "achieved": tk, "peak": PEAK_MFMA_F16, "unit": "TFLOP/s",
                     "frac": tk / PEAK_MFMA_F16, "traffic": measured_traffic("block_sparse_causal_prefill", "fwd")},
        "kernel": info["kernel"], "grid": info["grid"], "dtype": c["dtype"],
    }


def setup_backward():
    """Device inputs, the forward's O and LSE, and one step (one mfa_bwd call) of the
    backward over the dense causal prefill shape."""
    import torch
    import exact_attention_amd as ea
    c = A.workload("dense_causal_backward")
    x = A.workload_inputs("dense_causal_backward")
    q, k, v = (to_dev(t, c["dtype"]) for t in (x.q, x.k, x.v))
    do = to_dev(A.grad_inputs(c["B"], c["Hq"], c["Nq"], c["D"], c["dtype"], c["seed"] + 1000),
                c["dtype"])
    out, lse = ea.mfa_fwd(q, k, v, scale=c["scale"], causal=c["causal"])
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(int(ea.lib().mfa_bwd_workspace_bytes(c["B"], c["Hq"], c["Nq"])),
                     dtype=torch.uint8, device="cuda")

    step = ea.prepare(ea.mfa_bwd, q, k, v, out, do, lse, scale=c["scale"], causal=c["causal"],
                      dq=dq, dk=dk, dv=dv, workspace=ws)
    return step


def bench_backward(step, steps):
    import exact_attention_amd as ea
    c = A.workload("dense_causal_backward")
    t = time_calls(step, steps)
    ms = t["ms_per_call"]
    info = ea.mfa_last_dispatch()
    # 10 D FLOP per visible pair: the five products S = Q K^T, dP = dO V^T, dV = P^T dO,
    # dQ = dS K and dK = dS^T Q (2 D each)
    flop = 10.0 * c["D"] * visible_pairs(c["Nq"], c["Nk"], c["causal"], -1, -1) * c["B"] * c["Hq"]
    tf = flop / (ms * 1e-3) / 1e12
    tk = flop / (t["mean_ms"] * 1e-3) / 1e12
    return {
        "workload": f"{c['name']} B={c['B']} Hq={c['Hq']} Hkv={c['Hkv']} N={c['Nq']} D={c['D']} "
                    f"{c['dtype']} causal=1 (dQ + dK/dV launches)",
        "tflops": tf, **timing_fields(t), "flop": flop,
        "roofline": {"bound": "mfma", "achieved": tk, "peak": PEAK_MFMA_F16, "unit": "TFLOP/s",
                     "frac": tk / PEAK_MFMA_F16,
                     "traffic": measured_traffic("dense_causal_backward", "bwd")},
        "kernel": info["kernel"], "grid": info["grid"], "dtype": c["dtype"],
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(gpu_out=None, budget_s=10.0):
    """The float64 oracle on this host over whole heads of the dense causal prefill.

    With gpu_out = (O, LSE) of the GPU run on the same inputs, the heads the oracle
    finished are also compared with it (max-abs error of O and of LSE)."""
    import oracle
    from threadpoolctl import threadpool_info
    c = A.workload("dense_causal_prefill")
    x = A.workload_inputs("dense_causal_prefill")
    q, k, v = (oracle.widen(t, c["dtype"]) for t in (x.q, x.k, x.v))
    pairs = visible_pairs(c["Nq"], c["Nk"], True, -1, -1)
    done = []
    t0 = time.perf_counter()
    for b in range(c["B"]):
        for h in range(c["Hq"]):
            O, L = oracle.attention(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                                    c["scale"], True)
            done.append((b, h, O[0, 0], L[0, 0]))
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flop = 4.0 * c["D"] * pairs * len(done)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    res = {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{len(done)} of 16 (b,h) heads of the B=2 H=8 N=4096 D=128 causal workload, "
                     f"float64 numpy oracle, {dt:.1f} s wall, BLAS threads={threads}, "
                     f"os.cpu_count()={os.cpu_count()}",
           "cpu_model": cpu_model()}
    if gpu_out is not None:
        Ob, Lg = gpu_out
        eo = max(float(np.abs(oracle.widen(Ob[b, h], c["dtype"]) - O).max()) for b, h, O, _ in done)
        el = max(float(np.abs(Lg[b, h] - L).max()) for b, h, _, L in done)
        res["max_abs_err_vs_gpu"] = {"O": eo, "LSE": el, "heads": len(done),
                                     "bound": {"O": 2e-3, "LSE": 1e-3}}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workloads", default=",".join(w for w in A.WORKLOADS if w != "tiny_dense"))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_amd as ea
    if not os.path.exists(ea.LIB_PATH):
        from exact_attention_amd.build import build
        build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ea.lib()

    wl = [s for s in args.workloads.split(",") if s]
    for name in wl:
        if name not in A.WORKLOADS:
            raise SystemExit(f"unknown workload {name!r}; known: {', '.join(A.WORKLOADS)}")
    if HEAD not in wl:
        wl = [HEAD] + wl
    setup = {"paged_splitkv_decode": setup_decode, "packed_varlen_causal_prefill": setup_varlen,
             "paged_chunked_prefill": setup_chunked, "paged_multi_query_decode": setup_multi,
             "block_sparse_causal_prefill": setup_sparse, "dense_causal_backward": setup_backward}
    timed = {"paged_splitkv_decode": bench_decode, "packed_varlen_causal_prefill": bench_varlen,
             "paged_chunked_prefill": bench_chunked, "paged_multi_query_decode": bench_multi,
             "block_sparse_causal_prefill": bench_sparse, "dense_causal_backward": bench_backward}
    steps = {n: (setup[n]() if n in setup else setup_prefill(n)) for n in wl}
    res = {}
    for n in wl:
        warm_up(steps[n], args.warmup)
        res[n] = timed[n](steps[n], args.steps) if n in timed else bench_prefill(n, steps[n], args.steps)
        print(f"# workload {n}: " + json.dumps(res[n]), file=sys.stderr, flush=True)

    head = res[HEAD]
    line = {
        "metric": METRIC,
        "value": round(head["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_call"], 5),
        "per_call_ms": {"mean": round(head["mean_ms"], 5), "median": round(head["median_ms"], 5),
                        "min": round(head["min_ms"], 5)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded N(0,1) Q/K/V)",
        "config": {"workload": head["workload"], "global_batch": 2, "seq_len": 4096,
                   "parallelism": "none (1 GPU)"},
        "roofline": head["roofline"],
    }
    if not args.no_cpu_baseline:
        bits = steps[HEAD].out.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        line["cpu_baseline"] = cpu_baseline((bits, steps[HEAD].lse.cpu().numpy()))
    line["workloads"] = {
        n: {k: (round(v, 6) if isinstance(v, float) else v) for k, v in r.items()}
        for n, r in res.items()}
    if "paged_splitkv_decode" in res:
        line["decode_gbs"] = round(res["paged_splitkv_decode"]["gbs"], 1)
        line["decode_roofline"] = res["paged_splitkv_decode"]["roofline"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
