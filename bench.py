#!/usr/bin/env python3
"""Throughput of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]

One step is one pass of the hot path over the batched-MHA workload
(B=4, H=16, N=2048, d=128, bf16, scale 1/sqrt(128)) in both of its modes,
non-causal and causal.  ``value`` is the step's algorithmic TFLOP/s
(4*B*H*Nq*Nk*d, halved for the causal pass) with inputs already resident in
device memory.  The timed region issues the K steps' non-causal launches
back to back, then their causal launches, with a HIP event on the launch
stream at its start, between the two runs and at its end: the two averages
are the kernels' launch-to-launch times, with no event between launches of a
run.  ``roofline`` reports the dominant kernel (the non-causal forward)
against the MI355X dense bf16 MFMA peak.  ``cpu_baseline`` times the fp64 CPU oracle on a bounded
sample of the same workload.  ``other_workloads`` adds the long causal GQA,
varlen and split-KV decode workloads (TFLOP/s, or GB/s for decode).

Prints exactly one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
METRIC = "attention fwd TFLOP/s (4·B·H·Nq·Nk·d, causal halved) and % of bf16 MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "exact_attention_84_amd", "csrc")


def device_mfma_peak(torch_cus: int):
    """Dense bf16 MFMA peak of device 0 from its CU count and peak shader clock
    (hipDeviceGetAttribute), at 4096 flop per clock per CU (four SIMDs, one
    32x32x16 product per 32 clocks each): (TFLOP/s, CUs, MHz), or None when
    the runtime's answer does not check out against torch's CU count."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        val = ctypes.c_int(0)
        # hipDeviceAttributeClockRate (kHz) and hipDeviceAttributeMultiprocessorCount
        # in ROCm 7.2's hip_runtime_api.h
        if hip.hipDeviceGetAttribute(ctypes.byref(val), 63, 0) != 0 or val.value != torch_cus:
            return None
        cus = val.value
        if hip.hipDeviceGetAttribute(ctypes.byref(val), 5, 0) != 0 or val.value <= 0:
            return None
        mhz = val.value / 1000.0
        return round(cus * 4096 * mhz * 1e6 / 1e12, 1), cus, mhz
    except OSError:  # pragma: no cover
        return None


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def code_without_comments(text: str) -> str:
    """C/C++ source with comments, trailing blanks and blank lines removed
    (the sources hold no comment markers inside string literals)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(l.rstrip() for l in text.splitlines() if l.strip())


def unit_files(unit: str, csrc: str = CSRC) -> list:
    """The files a kernel's code comes from: its translation unit, the host
    code that fills its parameters (fa_api.hip, when present), and every
    local header they include, recursively."""
    todo = [unit] + (["fa_api.hip"] if os.path.exists(os.path.join(csrc, "fa_api.hip")) else [])
    seen = []
    while todo:
        f = todo.pop()
        if f in seen or not os.path.exists(os.path.join(csrc, f)):
            continue
        seen.append(f)
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            todo += re.findall(r'^\s*#\s*include\s+"([^"]+)"', fh.read(), re.M)
    return sorted(seen)


def kernel_source_hash(unit: str = "fa_fwd.hip", csrc: str = CSRC) -> str:
    """Hash of the code a kernel is built from (its unit's files, comments
    removed) and of the unit's compiler options: a change to either, not to
    comments, makes recorded counter figures for that kernel stale."""
    h = hashlib.sha256()
    for f in unit_files(unit, csrc):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + code_without_comments(fh.read()).encode())
    try:
        from exact_attention_84_amd import build as B
        # options as written in the build script, with the checkout's own
        # path left out (it differs between machines)
        opts = [o.replace(B.ROOT, "<root>") for o in B.flags() + B.SOURCE_FLAGS.get(unit, [])]
        h.update(" ".join(opts).encode())
    except ImportError:  # pragma: no cover
        pass
    return h.hexdigest()[:16]


# kernel-name pattern -> (traffic.json tag, translation unit)
TRAFFIC_KERNELS = {
    "fwd_wide_kernel<4, false, false>": ("fwd_noncausal_d128", "fa_fwd_wide.hip"),
    "fwd_wide_kernel<4, true, true>": ("fwd_causal_d128", "fa_fwd_wide.hip"),
    "decode_kernel<128>": ("decode_d128", "fa_decode.hip"),
    "bwd_dkdv_kernel<128, false>": ("bwd_dkdv_noncausal_d128", "fa_bwd.hip"),
    "bwd_dq_kernel<128, 4, false>": ("bwd_dq_noncausal_d128", "fa_bwd.hip"),
    "fwd_fp8_kernel<4, false>": ("fwd_fp8_noncausal_d128", "fa_fwd_fp8.hip"),
}


def measured_traffic(tag: str):
    """HBM bytes per launch of one kernel from committed rocprofv3 counter
    runs, if they were taken on that kernel's current sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    k = t.get("kernels", {}).get(tag)
    if k is None or k.get("source_hash") != kernel_source_hash(k.get("unit", "")):
        return None
    # counters of another kernel (a different instance, or an old tag) do not count
    if not any(t_ == tag and pat in k.get("kernel", "") and u == k.get("unit")
               for pat, (t_, u) in TRAFFIC_KERNELS.items()):
        return None
    return k.get("bytes_per_launch")


def write_traffic(fetch_dir: str, write_dir: str) -> dict:
    """Turn two rocprofv3 counter runs of ``bench.py --probe`` (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch) into HBM bytes per launch of the forward
    kernels.  Each counter is scaled by what it reads for the probe's plain
    1 GiB copy, which reads and writes exactly 1 GiB."""
    import csv
    import statistics

    def per_kernel(d, counter):
        vals = {}
        with open(os.path.join(d, "run_counter_collection.csv")) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    copy_bytes = float(1 << 30)
    out = {"kernels": {}, "scale": {}}
    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = per_kernel(d, counter)
        # the 1 GiB copy is the largest copy dispatch (setting up the inputs
        # launches small ones too)
        copy = [max(v) for k, v in vals.items() if "copyBuffer" in k]
        if not copy:
            raise SystemExit(f"no copy kernel in {d}: run bench.py --probe under rocprofv3")
        factor = copy_bytes / (max(copy) * 1024.0)
        kib = {k: statistics.mean(v) for k, v in vals.items()}
        out["scale"][counter] = round(factor, 4)
        for k, v in kib.items():
            per.setdefault(k, {})[counter] = v * 1024.0 * factor
    for k, v in per.items():
        for pat, (tag, unit) in TRAFFIC_KERNELS.items():
            if pat in k and "FETCH_SIZE" in v and "WRITE_SIZE" in v:
                rd, wr = round(v["FETCH_SIZE"]), round(v["WRITE_SIZE"])
                out["kernels"][tag] = {"kernel": k, "unit": unit,
                                       "source_hash": kernel_source_hash(unit),
                                       "read_bytes": rd, "write_bytes": wr,
                                       "bytes_per_launch": rd + wr}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    return out


def to_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def time_calls(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def other_workloads(fa, steps, warmup):
    import torch
    res = {}
    for wid in (3, 4):
        w = W.WORKLOADS[wid]
        inp = W.make_workload(w, seed=0)
        q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
        kw = {}
        if w.kind == "varlen":
            cu = torch.from_numpy(inp["cu_q"]).cuda()
            kw = dict(cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=int(inp["lengths"].max()),
                      max_seqlen_k=int(inp["lengths"].max()))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
        ms = time_calls(lambda: fa.attention(q, k, v, causal=True, scale=w.scale, out=o, lse=lse,
                                             **kw), steps, warmup)
        fl = W.flops(w, inp.get("lengths"))
        tf = fl / (ms * 1e-3) / 1e12
        res[w.name] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                       "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4), "gflop": round(fl / 1e9, 1)}
        log(w.name, res[w.name])
        del q, k, v, o, lse
    w = W.WORKLOADS[5]
    lens, args, kw = decode_inputs(fa, w)
    ms = time_calls(lambda: fa.decode(*args, scale=w.scale, **kw), steps, warmup)
    by = W.decode_bytes(w, lens)
    gbs = by / (ms * 1e-3) / 1e9
    res[w.name] = {"ms": round(ms, 4), "gbs": round(gbs, 1),
                   "frac_of_hbm": round(gbs / PEAK_HBM_GBS, 4), "gbytes": round(by / 1e9, 3)}
    log(w.name, res[w.name])
    return res


def kvcache_workload(fa, w, steps, warmup):
    """The decode workload as one KV-cache step per call: the cache paged in
    256-row blocks handed out in a shuffled order, the new token's key and
    value appended at each sequence's position, and rotary embedding (the
    usual 10000-base tables) on its query and key.  Sequence b holds its
    drawn length minus one before the call, so the step attends to exactly
    the drawn lengths.  The cache contents are seeded N(0, 1) draws made on
    the device (their values do not affect the time).  Algorithmic bytes: the
    attended K and V rows once, the appended rows written once, q, k_new and
    v_new read, the rotated queries written and read back, two table rows per
    sequence, and O and LSE."""
    import torch
    lens = W.workload_lengths(w, seed=0) - 1
    page = 256
    nblk = w.seqlen_k // page
    rng = np.random.default_rng(0)
    table = torch.from_numpy(
        rng.permutation(w.batch * nblk).reshape(w.batch, nblk).astype(np.int32)).cuda()
    g = torch.Generator(device="cuda").manual_seed(0)
    kc = torch.empty((w.batch * nblk, page, w.heads_kv, w.head_dim), dtype=torch.bfloat16,
                     device="cuda")
    kc.normal_(generator=g)
    vc = torch.empty_like(kc).normal_(generator=g)
    q = to_dev(W.decode_q(w.batch, w.heads_q, w.head_dim, seed=0, wid=w.wid))
    kn = torch.empty((w.batch, w.heads_kv, w.head_dim), dtype=torch.bfloat16,
                     device="cuda").normal_(generator=g)
    vn = torch.empty_like(kn).normal_(generator=g)
    inv = 10000.0 ** (-torch.arange(0, w.head_dim, 2, dtype=torch.float64) / w.head_dim)
    ang = torch.outer(torch.arange(w.seqlen_k, dtype=torch.float64), inv)
    cos, sin = ang.cos().float().cuda(), ang.sin().float().cuda()
    cl = torch.from_numpy(lens.astype(np.int32)).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((w.batch, w.heads_q), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.decode_kvcache_workspace_size(w.batch, w.heads_q, w.seqlen_k,
                                                      w.head_dim), dtype=torch.uint8,
                     device="cuda")
    ms = time_calls(lambda: fa.decode_kvcache(q, kc, vc, cl, k_new=kn, v_new=vn,
                                              block_table=table, rotary_cos=cos, rotary_sin=sin,
                                              scale=w.scale, out=o, lse=lse, workspace=ws),
                    steps, warmup)
    row = w.heads_kv * w.head_dim * 2
    extra = (2 * w.batch * row                                   # appended rows written
             + 2 * w.batch * row                                 # k_new, v_new read
             + 2 * w.batch * w.heads_q * w.head_dim * 2          # rotated q written, read
             + 2 * w.batch * w.head_dim * 4)                     # cos and sin rows
    by = W.decode_bytes(w, lens + 1) + extra
    gbs = by / (ms * 1e-3) / 1e9
    res = {"ms": round(ms, 4), "gbs": round(gbs, 1), "frac_of_hbm": round(gbs / PEAK_HBM_GBS, 4),
           "gbytes": round(by / 1e9, 3), "page_size": page}
    log("decode_kvcache (paged, append, rotary)", res)
    del kc, vc
    return res


def window_workload(fa, w, steps, warmup):
    """The long causal GQA workload through the score-variant kernel: a
    4096-key causal sliding window, then the same window with ALiBi slopes
    (2^(-8 h / Hq)) and a softcap of 30.  Algorithmic flops: 4 d per
    admissible (query, key) pair, i.e. 4 d Hq sum_i min(i + 1, 4096)."""
    import torch
    inp = W.make_workload(w, seed=0)
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
    win = 4096
    pairs = sum(min(i + 1, win) for i in range(w.seqlen_q))
    fl = 4.0 * w.head_dim * w.heads_q * w.batch * pairs
    slopes = (2.0 ** (-8.0 * torch.arange(1, w.heads_q + 1) / w.heads_q)).float().cuda()
    res = {}
    for name, kw in (("window4096", {}), ("window4096_alibi_softcap30",
                                          dict(alibi_slopes=slopes, softcap=30.0))):
        ms = time_calls(lambda: fa.attention(q, k, v, causal=True, scale=w.scale,
                                             window=(win - 1, 0), out=o, lse=lse, **kw),
                        steps, warmup)
        tf = fl / (ms * 1e-3) / 1e12
        res[name] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                     "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4), "gflop": round(fl / 1e9, 1)}
        log("sliding window", w.name, name, res[name])
    return res


def fp8_workload(fa, w, steps, warmup):
    """The headline workload's shape with E4M3 inputs (N(0,1) draws scaled per
    tensor and cast; descales 1/32, 1/16, 1/64) through the FP8 forward,
    non-causal and causal.  Algorithmic flops as the bf16 forward's; the
    share is of the dense FP8 peak."""
    import torch
    q8, k8, v8, ds = W.make_fixed_fp8(w.batch, w.heads_q, w.heads_kv, w.seqlen_q, w.seqlen_k,
                                      w.head_dim, seed=0, wid=w.wid)
    q, k, v = (torch.from_numpy(x).cuda() for x in (q8, k8, v8))
    o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
    res = {}
    for causal in (False, True):
        fl = W.flops(w, causal=causal)
        ms = time_calls(lambda: fa.attention_fp8(q, k, v, q_descale=ds[0], k_descale=ds[1],
                                                 v_descale=ds[2], causal=causal, scale=w.scale,
                                                 out=o, lse=lse),
                        steps, warmup)
        tf = fl / (ms * 1e-3) / 1e12
        res["causal" if causal else "noncausal"] = {
            "ms": round(ms, 4), "tflops": round(tf, 1),
            "frac_of_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4), "gflop": round(fl / 1e9, 1)}
        if not causal:
            res["noncausal"]["traffic"] = measured_traffic("fwd_fp8_noncausal_d128")
        log("fp8 forward", w.name, "causal" if causal else "non-causal",
            res["causal" if causal else "noncausal"])
    return res


def backward_workload(fa, w, steps, warmup):
    """The attention backward (preprocess, dK/dV and dQ kernels) on the
    headline workload, non-causal and causal, from the forward's own O and
    LSE.  Algorithmic flops: the five products S, dP, dV, dK, dQ of
    2 N_q N_k d each per head, 2.5 times the forward's (halved when causal)."""
    import torch
    inp = W.make_workload(w, seed=0)
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    do = to_dev(W.make_dout(inp["q"].shape, seed=0, wid=w.wid))
    ws = torch.empty(fa.bwd_workspace_size(w.batch, w.heads_q, w.seqlen_q), dtype=torch.uint8,
                     device="cuda")
    res = {}
    for causal in (False, True):
        o, lse = fa.attention(q, k, v, causal=causal, scale=w.scale)
        ms = time_calls(lambda: fa.attention_backward(q, k, v, o, lse, do, causal=causal,
                                                      scale=w.scale, workspace=ws,
                                                      grad_dtype=torch.bfloat16),
                        steps, warmup)
        fl = 2.5 * W.flops(w, causal=causal)
        tf = fl / (ms * 1e-3) / 1e12
        res["causal" if causal else "noncausal"] = {
            "ms": round(ms, 4), "tflops": round(tf, 1),
            "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4), "gflop": round(fl / 1e9, 1)}
        log("backward", w.name, "causal" if causal else "non-causal", res[
            "causal" if causal else "noncausal"])
    return res


def cold_launches(fn, n, flush):
    """Average event-timed duration of `fn` when each launch follows a write
    of `flush` (512 MiB, twice the 256 MB last-level cache), so that its
    inputs start in HBM rather than in the MALL."""
    import torch
    ts = []
    for _ in range(n):
        flush.zero_()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        ts.append((a, b))
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ts) / n


def decode_inputs(fa, w):
    """Device inputs of the split-KV decode workload (seed 0): query, caches
    filled up to each drawn length, lengths, outputs and workspace."""
    import torch
    lens = W.workload_lengths(w, seed=0)
    qd = to_dev(W.decode_q(w.batch, w.heads_q, w.head_dim, seed=0, wid=w.wid))
    kc = torch.zeros((w.batch, w.seqlen_k, w.heads_kv, w.head_dim), dtype=torch.bfloat16,
                     device="cuda")
    vc = torch.zeros_like(kc)
    for b in range(w.batch):
        kb, vb = W.decode_kv_slice(b, int(lens[b]), w.heads_kv, w.head_dim, seed=0, wid=w.wid)
        kc[b, :int(lens[b])] = to_dev(kb)
        vc[b, :int(lens[b])] = to_dev(vb)
    o = torch.empty_like(qd)
    lse = torch.empty((w.batch, w.heads_q), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.decode_workspace_size(w.batch, w.heads_q, w.seqlen_k, w.head_dim),
                     dtype=torch.uint8, device="cuda")
    return lens, (qd, kc, vc, torch.from_numpy(lens).cuda()), dict(out=o, lse=lse, workspace=ws)


def probe(fa, w, steps, warmup):
    """Launches for rocprofv3 counter runs: the headline workload's non-causal
    and causal forward, the split-KV decode workload, the headline workload's
    non-causal backward (bf16 gradients), its non-causal FP8 forward, then a 1 GiB
    device-to-device copy (a kernel that reads and writes exactly 1 GiB each,
    to scale the byte counters)."""
    import torch
    inp = W.make_workload(w, seed=0)
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
    for causal in (False, True):
        for _ in range(warmup + steps):
            fa.attention(q, k, v, causal=causal, scale=w.scale, out=o, lse=lse)
    del q, k, v, o, lse
    wd = W.WORKLOADS[5]
    _, args, kw = decode_inputs(fa, wd)
    for _ in range(warmup + steps):
        fa.decode(*args, scale=wd.scale, **kw)
    del args, kw
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    do = to_dev(W.make_dout(inp["q"].shape, seed=0, wid=w.wid))
    o, lse = fa.attention(q, k, v, causal=False, scale=w.scale)
    ws = torch.empty(fa.bwd_workspace_size(w.batch, w.heads_q, w.seqlen_q), dtype=torch.uint8,
                     device="cuda")
    for _ in range(warmup + steps):
        fa.attention_backward(q, k, v, o, lse, do, causal=False, scale=w.scale, workspace=ws,
                              grad_dtype=torch.bfloat16)
    del q, k, v, do, o, lse, ws
    q8, k8, v8, ds = W.make_fixed_fp8(w.batch, w.heads_q, w.heads_kv, w.seqlen_q, w.seqlen_k,
                                      w.head_dim, seed=0, wid=w.wid)
    q, k, v = (torch.from_numpy(x).cuda() for x in (q8, k8, v8))
    o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
    for _ in range(warmup + steps):
        fa.attention_fp8(q, k, v, q_descale=ds[0], k_descale=ds[1], v_descale=ds[2],
                         causal=False, scale=w.scale, out=o, lse=lse)
    del q, k, v, o, lse
    a = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"probe: {warmup + steps} non-causal, causal, decode, backward and FP8 launches, "
        f"{steps} copies of {a.numel() * 4} bytes")


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return None


def _peak_rss_mib():
    import resource
    return round(resource.getrusage(resource.RUSAGE_SELF).ru_maxrss / 1024.0, 1)  # KiB on Linux


def _oracle_slices(w, budget_s, step):
    """Runs step(i) -> (work units) for i = 0, 1, ... until budget_s seconds of
    work are done (at least one call); returns (units, calls, seconds)."""
    done, n = 0.0, 0
    t0 = time.perf_counter()
    while n == 0 or time.perf_counter() - t0 < budget_s:
        done += step(n)
        n += 1
    return done, n, time.perf_counter() - t0


def cpu_baseline(w, budget_s=8.0, per_config_s=3.0):
    """The fp64 oracle timed on this host.  The headline figure is the
    workload bench.py times, on (sequence, head) slices in both modes, taken
    in order over every sequence and head (wrapping around) until
    ``budget_s`` seconds are done.  ``per_config`` times the other workloads
    the same way on slices of a few seconds each: the single head in full,
    heads of the long GQA sequence, (sequence, head) pairs of the packed
    batch, and (sequence, kv head) groups of the decode batch (whose caches
    are drawn one sequence at a time, never whole)."""
    import oracle
    per = {}

    # batched MHA (the headline): both modes per (sequence, head)
    inp = W.make_workload(w, seed=0)
    g = w.heads_q // w.heads_kv
    slices = [(b, h) for b in range(w.batch) for h in range(w.heads_q)]

    def mha(n):
        b, h = slices[n % len(slices)]
        qh = oracle.to_f64(inp["q"][b, :, h])
        kh = oracle.to_f64(inp["k"][b, :, h // g])
        vh = oracle.to_f64(inp["v"][b, :, h // g])
        fl = 0.0
        for causal in (False, True):
            oracle.head_attention(qh, kh, vh, w.scale, causal)
            fl += (0.5 if causal else 1.0) * 4.0 * w.seqlen_q * w.seqlen_k * w.head_dim
        return fl

    done, n, dt = _oracle_slices(w, budget_s, mha)
    head = {"value": round(done / dt / 1e12, 6), "unit": "TFLOP/s",
            "sample": f"{n} (sequence, head) slices of the {len(slices)} in {w.name} "
                      f"(batch-major order), each non-causal and causal, {dt:.1f} s"}
    per[w.name] = head
    del inp

    # single head: the whole call
    w1 = W.WORKLOADS[1]
    i1 = W.make_workload(w1, seed=0)
    done, n, dt = _oracle_slices(
        w1, min(1.0, per_config_s),
        lambda _: (oracle.attention(i1["q"], i1["k"], i1["v"], w1.scale, w1.causal),
                   W.flops(w1))[1])
    per[w1.name] = {"value": round(done / dt / 1e12, 6), "unit": "TFLOP/s",
                    "sample": f"the whole call, {n} times, {dt:.1f} s"}

    # long causal GQA: whole query heads
    w3 = W.WORKLOADS[3]
    i3 = W.make_workload(w3, seed=0)
    g3 = w3.heads_q // w3.heads_kv

    def gqa(n):
        h = n % w3.heads_q
        oracle.head_attention(oracle.to_f64(i3["q"][0, :, h]), oracle.to_f64(i3["k"][0, :, h // g3]),
                              oracle.to_f64(i3["v"][0, :, h // g3]), w3.scale, True)
        return 0.5 * 4.0 * w3.seqlen_q * w3.seqlen_k * w3.head_dim

    done, n, dt = _oracle_slices(w3, per_config_s, gqa)
    per[w3.name] = {"value": round(done / dt / 1e12, 6), "unit": "TFLOP/s",
                    "sample": f"{n} of its {w3.heads_q} query heads, causal, {dt:.1f} s"}
    del i3

    # packed batch: (sequence, head) pairs, causal within each sequence
    w4 = W.WORKLOADS[4]
    i4 = W.make_workload(w4, seed=0)
    g4 = w4.heads_q // w4.heads_kv
    cu = i4["cu_q"]
    pairs = [(s, h) for s in range(w4.batch) for h in range(0, w4.heads_q, g4)]

    def packed(n):
        s_, h = pairs[n % len(pairs)]
        a, b = int(cu[s_]), int(cu[s_ + 1])
        oracle.head_attention(oracle.to_f64(i4["q"][a:b, h]), oracle.to_f64(i4["k"][a:b, h // g4]),
                              oracle.to_f64(i4["v"][a:b, h // g4]), w4.scale, True)
        return 0.5 * 4.0 * (b - a) * (b - a) * w4.head_dim

    done, n, dt = _oracle_slices(w4, per_config_s, packed)
    per[w4.name] = {"value": round(done / dt / 1e12, 6), "unit": "TFLOP/s",
                    "sample": f"{n} (sequence, head) pairs of its {w4.batch * w4.heads_q}, "
                              f"sequence-major, one head per kv group, {dt:.1f} s"}
    del i4

    # split-KV decode: (sequence, kv head) groups, each sequence's cache drawn alone
    w5 = W.WORKLOADS[5]
    lens = W.workload_lengths(w5, 0)
    q5 = W.decode_q(w5.batch, w5.heads_q, w5.head_dim, seed=0, wid=w5.wid)
    g5 = w5.heads_q // w5.heads_kv
    cache = {}

    def dec(n):
        b = (n // w5.heads_kv) % w5.batch
        kvh = n % w5.heads_kv
        if b not in cache:
            cache.clear()
            cache[b] = W.decode_kv_slice(b, int(lens[b]), w5.heads_kv, w5.head_dim, seed=0,
                                         wid=w5.wid)
        kb, vb = cache[b]
        kf, vf = oracle.to_f64(kb[:, kvh]), oracle.to_f64(vb[:, kvh])
        for h in range(kvh * g5, (kvh + 1) * g5):
            oracle.head_attention(oracle.to_f64(q5[b, h])[None, :], kf, vf, w5.scale, False)
        return 2.0 * int(lens[b]) * w5.head_dim * 2  # K and V rows of the group, bf16

    done, n, dt = _oracle_slices(w5, per_config_s, dec)
    per[w5.name] = {"value": round(done / dt / 1e9, 4), "unit": "GB/s",
                    "sample": f"{n} (sequence, kv head) groups of its {w5.batch * w5.heads_kv}, "
                              f"each with its {g5} query heads, {dt:.1f} s "
                              f"(including drawing each sequence's cache)"}
    threads = _blas_threads()
    return {"value": head["value"], "unit": "TFLOP/s",
            # the matrix products run on the BLAS threads, the rest on one
            "cores": threads if threads else 1, "host_cpus": os.cpu_count(),
            "blas_threads": threads, "kind": "oracle",
            "sample": head["sample"] + ", fp64 numpy", "peak_rss_mib": _peak_rss_mib(),
            "per_config": per}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--probe", action="store_true",
                    help="counter-collection mode: only the timed launches of the headline "
                         "workload plus a plain 1 GiB device copy (the scale for HBM byte "
                         "counters); prints no JSON")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc runs of --probe "
                         "(FETCH_SIZE, then WRITE_SIZE) and exit; needs no GPU")
    a = ap.parse_args()
    if a.write_traffic:
        print(json.dumps(write_traffic(*a.write_traffic), indent=1))
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(the attention forward here runs whole on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_84_amd as fa
    fa.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    props = torch.cuda.get_device_properties(0)
    log("device", props.name, getattr(props, "gcnArchName", ""), "CUs",
        props.multi_processor_count)
    dev_peak = device_mfma_peak(props.multi_processor_count)
    log("bf16 MFMA peak from the device", dev_peak, "against the published", PEAK_BF16_TFLOPS)

    w = W.WORKLOADS[2]
    if a.probe:
        probe(fa, w, a.steps, a.warmup)
        return
    inp = W.make_workload(w, seed=0)
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    o_nc, o_c = torch.empty_like(q), torch.empty_like(q)
    lse_nc = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
    lse_c = torch.empty_like(lse_nc)
    fl_nc = W.flops(w, causal=False)
    fl_c = W.flops(w, causal=True)

    def noncausal():
        fa.attention(q, k, v, causal=False, scale=w.scale, out=o_nc, lse=lse_nc)

    def causal():
        fa.attention(q, k, v, causal=True, scale=w.scale, out=o_c, lse=lse_c)

    for _ in range(a.warmup):
        noncausal()
        causal()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    wall0 = time.perf_counter()
    ev[0].record()
    for _ in range(a.steps):
        noncausal()
    ev[1].record()
    for _ in range(a.steps):
        causal()
    ev[2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = ev[0].elapsed_time(ev[2]) / a.steps
    ms_nc = ev[0].elapsed_time(ev[1]) / a.steps
    ms_c = ev[1].elapsed_time(ev[2]) / a.steps
    assert torch.isfinite(o_nc.float()).all() and torch.isfinite(o_c.float()).all()
    value = (fl_nc + fl_c) / (ms_step * 1e-3) / 1e12
    flush = torch.empty(1 << 29, dtype=torch.uint8, device="cuda")
    ms_cold = cold_launches(lambda: fa.attention(q, k, v, causal=False, scale=w.scale, out=o_nc,
                                                 lse=lse_nc), 20, flush)
    del flush
    ach = fl_nc / (ms_nc * 1e-3) / 1e12
    log(f"step {ms_step:.4f} ms ({wall / a.steps * 1e3:.4f} ms wall), non-causal {ms_nc:.4f} ms "
        f"({ach:.1f} TFLOP/s), causal {ms_c:.4f} ms ({fl_c / (ms_c * 1e-3) / 1e12:.1f} TFLOP/s)")

    kname = "fwd_wide_kernel<4, false, false>"
    traffic = measured_traffic("fwd_noncausal_d128")
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name + " (non-causal + causal)", "batch": w.batch,
                   "heads_q": w.heads_q, "heads_kv": w.heads_kv, "seq_len": w.seqlen_q,
                   "head_dim": w.head_dim, "scale": round(w.scale, 6),
                   "inputs": "bf16 N(0,1), seed 0", "o_dtype": "bf16"},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "kernel": kname, "achieved": round(ach, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "device_peak": ({"tflops": dev_peak[0], "cus": dev_peak[1],
                                      "max_clock_mhz": dev_peak[2]} if dev_peak else None),
                     "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "avg_launch_ms": round(ms_nc, 5),
                     "flop_per_launch": fl_nc},
        "causal_launch": {"avg_launch_ms": round(ms_c, 5),
                          "tflops": round(fl_c / (ms_c * 1e-3) / 1e12, 2)},
        "noncausal_launch_ms": {"cold_cache_avg": round(ms_cold, 5),
                                "cold_cache_tflops": round(fl_nc / (ms_cold * 1e-3) / 1e12, 2)},
    }
    del o_nc, o_c, lse_nc, lse_c
    if not a.no_extra:
        res["other_workloads"] = other_workloads(fa, max(5, a.steps // 5), max(3, a.warmup // 5))
        res["other_workloads"]["decode_kvcache_paged_append_rotary_b64_h32kv8_cache32k_d128"] = \
            kvcache_workload(fa, W.WORKLOADS[5], max(5, a.steps // 5), max(3, a.warmup // 5))
        res["other_workloads"]["gqa_causal_b1_h32kv8_n8192_d128_sliding_window"] = \
            window_workload(fa, W.WORKLOADS[3], max(5, a.steps // 5), max(3, a.warmup // 5))
        res["fp8_forward"] = {"workload": w.name, "dtype": "e4m3 inputs, fp32 accumulation",
                              "o_dtype": "bf16",
                              **fp8_workload(fa, w, max(5, a.steps // 5), max(3, a.warmup // 5))}
        res["backward"] = {"workload": w.name, "grad_dtype": "bf16",
                           **backward_workload(fa, w, max(5, a.steps // 5),
                                               max(3, a.warmup // 5))}
    if not a.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w)
        log("cpu_baseline", res["cpu_baseline"])
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res, ensure_ascii=False), flush=True)


if __name__ == "__main__":
    main()
