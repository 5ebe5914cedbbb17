#!/usr/bin/env python3
"""Benchmark of the GLA chunkwise forward (and backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one forward pass of the layer over the GLA-340M layer shape (B=8,
H=4, L=2048, d_k=128, d_v=256, bf16 I/O, chunk 64, sub-chunk 16) on seeded
synthetic inputs: the library's per-chunk prep pass, then its chunk
recurrence, producing o and hT.  The inputs already sit in device memory when
the timed region starts.  Steps rotate over several copies of the inputs whose
total size exceeds the 256 MB Infinity Cache, so each step reads its inputs
from HBM (a "warm" figure with one set reused is reported beside it).

Printed (one JSON line on stdout):
* value: tokens/s of the forward step; tflops by the stated count
  2*L*C*(dk+dv) + 4*L*dk*dv per head;
* roofline: the dominant kernel against the 8 TB/s HBM peak, counting only
  the method's compulsory bytes that the kernel moves (q, k, v, log alpha
  read once; o, hT written once; h0 read), over its average duration from HIP
  events recorded by the library on the launch stream; the bytes of the
  intermediate records that the two passes exchange are reported apart
  (overhead_bytes), and rocprofv3's measured HBM bytes as traffic;
* step_roofline: the whole step's compulsory bytes over the step time;
* legs at the GLA-1.3B layer shape and the long-sequence shape (forward) and
  the backward at the GLA-340M shape, each with tokens/s, TFLOP/s and the
  fraction of its roofline; a one-token decode figure; the general gate
  G = alpha^T beta; the op-level layer; and the fp64 oracle on the host cores
  (a baseline, not a target).

The GPU leaves its idle clock state only after some milliseconds of work, so
the streaming-copy measurement (copy_gbps) runs just before the warm-up steps.
Progress goes to stderr.

Counter records: `--ingest-counters FETCH_DIR WRITE_DIR WORKLOAD` reads the
rocprofv3 FETCH_SIZE and WRITE_SIZE runs of one workload (plus the
`--calibrate-copy` runs in CAL_FETCH_DIR CAL_WRITE_DIR given with
--calibration) and writes profiles/traffic.json, which the bench reports as
`traffic` while the kernels' sources are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
INFINITY_CACHE_BYTES = 256 << 20

METRIC = "GLA chunkwise fwd TFLOP/s + tokens/s, B8 H4 L2048 dk128 dv256 bf16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CALIBRATE_BYTES = 1 << 30     # plain device copy used to scale the HBM byte counters
KERNEL_SOURCES = [
    "chunkwise_linear_rnn_gla_amd/csrc/gla_prep.hip",
    "chunkwise_linear_rnn_gla_amd/csrc/gla_recur.hip",
    "chunkwise_linear_rnn_gla_amd/csrc/gla_records.h",
    "chunkwise_linear_rnn_gla_amd/csrc/gla_common.h",
    "chunkwise_linear_rnn_gla_amd/csrc/gla_internal.h",
    "chunkwise_linear_rnn_gla_amd/csrc/gla_pblock.h",
    "chunkwise_linear_rnn_gla_amd/csrc/gla_api.hip",
    "chunkwise_linear_rnn_gla_amd/csrc/gla_fwd.hip",
    "chunkwise_linear_rnn_gla_amd/csrc/gla_bwd.hip",
    "chunkwise_linear_rnn_gla_amd/csrc/gla_bwd_recur.hip",
    "chunkwise_linear_rnn_gla_amd/csrc/gla_dma.h",
    "chunkwise_linear_rnn_gla_amd/csrc/gla_ggate.hip",
    "chunkwise_linear_rnn_gla_amd/build.py",
]
# rocprofv3 kernel names (mangled or demangled) -> the library's launch names
KERNEL_NAMES = {"chunk_prep": "chunk_prep", "chunk_recur": "chunk_recur",
                "segment_scan": "segment_scan", "cumsum": "chunk_cumsum",
                "chunk_state": "chunk_state", "chunk_attn": "chunk_attn",
                "chunk_dqdk": "chunk_dqdk", "chunk_dv": "chunk_dv",
                "rowsum_state": "rowsum_state", "dla_carry": "dla_carry",
                "bwd_inter": "bwd_inter", "seg_output": "seg_output", "decode": "decode",
                "gg_prep": "gg_prep", "gg_recur": "gg_recur", "gg_gate_scan": "gg_gate_scan",
                "gg_gate_carry": "gg_gate_carry", "gg_gate_add": "gg_gate_add",
                "gg_hsum": "gg_hsum", "chunk_da_cum": "chunk_da_cum"}


def launch_name(kname):
    """The launch name of a kernel as rocprofv3 reports it, or None.  The
    prep and recurrence kernels' last template argument is the time-reversed
    mode of the backward's dv pass (..., true> / ...Lb1EEEv); the
    recurrence's one before it is 1 for the output pass and 0 for the
    segments' local-state pass.  The general gate's fp32 passes (its
    backward) are named gg_prep_f32 and gg_recur_f32_r<state rows>."""
    import re
    m = re.search(r"k_([a-z_]+[a-z])", kname)
    if not m or m.group(1) not in KERNEL_NAMES:
        return None
    name = KERNEL_NAMES[m.group(1)]
    if name in ("gg_prep", "gg_recur"):
        if re.search(r"k_gg_(?:prep|recur)If", kname) or re.search(r"k_gg_(?:prep|recur)<float", kname):
            name += "_f32"
            if name == "gg_recur_f32":
                mt = (re.search(r"k_gg_recurI\w*?Li(\d+)ELi\d+E", kname)
                      or re.search(r"k_gg_recur<float,\s*[\w:]+,\s*(\d+),", kname))
                if mt:
                    name += f"_r{16 * int(mt.group(1))}"
        return name
    if name in ("chunk_prep", "chunk_recur"):
        tail = re.search(r"L[ib](\d)ELb([01])EEEv", kname)      # mangled
        dtail = re.search(r",\s*(\d+),\s*(true|false)\s*>", kname)  # demangled
        if name == "chunk_prep":
            rev = bool(re.search(r"Lb1EEEv", kname) or re.search(r",\s*true\s*>", kname))
        else:
            out, rev = True, False
            if tail:
                out, rev = tail.group(1) == "1", tail.group(2) == "1"
            elif dtail:
                out, rev = dtail.group(1) == "1", dtail.group(2) == "true"
            if not out:
                name = "recur_local"
        if rev:
            name += "_rev"
    return name


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------- byte and FLOP counts

CSRC = "chunkwise_linear_rnn_gla_amd/csrc"


def kernel_sources(launch):
    """The repository files a kernel's code comes from: the source that
    defines it, the headers it includes (transitively), the host-side
    planner and the build flags.  A traffic record stays valid until one of
    these changes."""
    import re
    inv = {v: k for k, v in KERNEL_NAMES.items()}
    base = launch
    while base not in inv and "_" in base:
        base = base.rsplit("_", 1)[0]
    if launch == "recur_local":
        base = "chunk_recur"
    if base not in inv:
        return list(KERNEL_SOURCES)
    pat = re.compile(r"void\s+k_" + re.escape(inv[base]) + r"\b")
    srcs = sorted(glob.glob(os.path.join(ROOT, CSRC, "*.hip")))
    found = [f for f in srcs if pat.search(open(f).read())]
    if not found:
        return list(KERNEL_SOURCES)
    deps, todo = set(), [found[0]]
    while todo:
        f = todo.pop()
        rel = os.path.relpath(f, ROOT)
        if rel in deps:
            continue
        deps.add(rel)
        for inc in re.findall(r'#include "([a-z_]+\.h)"', open(f).read()):
            todo.append(os.path.join(ROOT, CSRC, inc))
    deps |= {CSRC + "/gla_api.hip", "chunkwise_linear_rnn_gla_amd/build.py"}
    return sorted(deps)


def sources_digest(paths):
    """sha256 over the given repository files (the sources of the kernels)."""
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE record, or None when there is none or
    the kernels' sources changed after the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    for e in rec.get("entries", []):
        if e.get("kernel") == kernel and e.get("workload") == workload:
            if e.get("sources_sha256") != sources_digest(e.get("sources", [])):
                return None
            return e
    return None


def recur_plan(w, nc):
    """(waves per workgroup, sequence segments) of the two-pass forward's
    recurrence as the library plans them: 16 state columns per wave, the
    largest workgroup that still gives 256 workgroups, or, when even one-wave
    workgroups give fewer than 128, the largest workgroup and enough sequence
    segments to fill the chip."""
    bf16 = w.dtype == "bf16"
    wmin = 2 if (w.dk >= 256 if bf16 else w.dk >= 128) else 1
    wmax = 2 if (bf16 and w.dk >= 256) else 4
    bh = w.B * w.H
    starved = bh * (w.dv // (16 * wmin)) < 128
    nwv = wmin
    for cand in (4, 2, 1):
        if cand < wmin or cand > wmax or w.dv % (16 * cand):
            continue
        nwv = cand
        if starved or bh * (w.dv // (16 * cand)) >= 256:
            break
    units = bh * (w.dv // (16 * nwv))
    nseg = 1
    if nc > 1 and units < 128:
        want = min(-(-256 // units), nc)
        seg_chunks = -(-nc // want)
        nseg = -(-nc // seg_chunks)
    return nwv, nseg


def compulsory_fwd(w, esize):
    """The forward's compulsory HBM bytes, split by the kernel that moves them
    in the two-pass forward: chunk_prep reads q, k, log alpha and V (it
    brings V into the caches for the recurrence); the recurrence writes o;
    hT (and h0) belong to the launch that writes (reads) the states: the
    recurrence, or the segment scan when the sequence is segmented."""
    BH, L, dk, dv = w.B * w.H, w.L, w.dk, w.dv
    q = k = BH * L * dk * esize
    v = o = BH * L * dv * esize
    a = BH * L * dk * 4
    st = BH * dk * dv * 4
    h0 = st if w.h0_std else 0
    _, nseg = recur_plan(w, -(-L // w.chunk))
    per = {"chunk_prep": q + k + a + v}
    if nseg > 1:
        per.update({"recur_local": 0, "segment_scan": h0 + st, "chunk_recur": o})
    else:
        per["chunk_recur"] = o + st + h0
    return sum(per.values()), per


def overhead_fwd(w, esize):
    """Bytes of the records the two passes exchange (written by chunk_prep,
    read by each recurrence launch), and the segment states, per launch."""
    BH, L, dk, dv, C = w.B * w.H, w.L, w.dk, w.dv, w.chunk
    nc = -(-L // C)
    qg = kg = BH * nc * C * dk * esize
    jt = C // 16
    p_blocks = jt + ((jt - 1) >> 1) * (jt >> 1) if esize == 2 else jt * (jt + 1) // 2
    pm = BH * nc * p_blocks * 1024 + (BH * nc * C * 16 * esize if esize == 2 else 0)
    gl = BH * nc * 1024 * (-(-8 * dk // 1024))
    _, nseg = recur_plan(w, nc)
    seg = BH * nseg * dk * dv * 4 if nseg > 1 else 0
    return {"chunk_prep": qg + kg + pm + gl,
            "recur_local": kg + gl + seg,
            "segment_scan": 2 * seg,
            "chunk_recur": qg + kg + pm + gl + seg}


def compulsory_bwd(w, esize):
    """The backward's compulsory HBM bytes: read q, k, v, dout (I/O dtype),
    log alpha (fp32), h0 and dhT if given; write dq, dk, dv (I/O dtype),
    dlog alpha and dh0 (fp32)."""
    BH, L, dk, dv = w.B * w.H, w.L, w.dk, w.dv
    st = BH * dk * dv * 4
    rd = 2 * BH * L * dk * esize + 2 * BH * L * dv * esize + BH * L * dk * 4
    rd += st if w.h0_std else 0
    wr = 2 * BH * L * dk * esize + BH * L * dv * esize + BH * L * dk * 4 + st
    return rd + wr


def flops_bwd(w):
    """Backward FLOPs by the same convention as the stated forward count
    (full C x C square): per head, intra 2 L C (3 dk + 2 dv) for A, dA, dq,
    dk, dv's intra products and inter 10 L dk dv for the state recompute, the
    state-gradient scan and the three inter products (derived; the pages give
    no backward count)."""
    per_head = 2 * w.L * w.chunk * (3 * w.dk + 2 * w.dv) + 10 * w.L * w.dk * w.dv
    return w.B * w.H * per_head


# ----------------------------------------------------------------- measurement helpers

def events_by_kernel(_abi):
    per = {}
    for i in range(_abi.gla_profile_count()):
        try:
            name, ms = _abi.gla_profile_get(i)
        except Exception:  # a record whose events could not be taken
            continue
        per.setdefault(name, []).append(ms)
    return per


def timed(fn, steps, torch):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def step_percentiles(fn, steps, torch):
    """Per-step durations (us) of `steps` calls of fn(i), each bracketed by
    HIP events on the current stream (the stream the library launches on):
    10th percentile, median and 90th percentile.  A pass of its own, after
    the timed steps; the events between steps add a little to each."""
    import statistics
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    us = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps))
    pick = lambda f: us[min(len(us) - 1, int(round(f * (len(us) - 1))))]
    return {"p10": round(pick(0.1), 2), "median": round(statistics.median(us), 2),
            "p90": round(pick(0.9), 2), "steps": steps}


def copy_bandwidth(torch, dev, copies=60):
    """A plain device copy of 1 GiB, `copies` times: achievable HBM bandwidth
    for context (it also brings the GPU out of its idle clock state)."""
    nbytes = 1 << 30
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(copies):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbps = 2 * nbytes * copies / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbps


def forward_leg(w, args, torch, gla, _abi, dev, stream, primary):
    """Time the forward on workload w: K steps over rotating input sets (HBM),
    the same K steps with per-launch HIP events, and (primary only) a warm
    figure.  Returns the leg's dict."""
    from chunkwise_linear_rnn_gla_amd.inputs import workload_inputs
    esize = 2 if w.dtype == "bf16" else 4
    code = gla.GLA_BF16 if w.dtype == "bf16" else gla.GLA_FP32
    dims = gla.GlaDims(w.B, w.H, w.L, w.dk, w.dv, w.chunk, w.subchunk)
    x = workload_inputs(w).to(dev)
    set_bytes = sum(t.numel() * t.element_size() for t in (x.q, x.k, x.v, x.log_alpha))
    set_bytes += w.B * w.H * w.L * w.dv * esize  # o
    nsets = args.sets or max(2, -(-2 * INFINITY_CACHE_BYTES // set_bytes))
    sets = [dict(q=x.q.clone(), k=x.k.clone(), v=x.v.clone(), a=x.log_alpha.clone(),
                 o=torch.empty(w.B, w.H, w.L, w.dv, dtype=x.q.dtype, device=dev))
            for _ in range(nsets)]
    hT = torch.empty(w.B, w.H, w.dk, w.dv, dtype=torch.float32, device=dev)
    ws_bytes = gla.gla_fwd_workspace_size(dims, code)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    log(f"[bench] {w.name}: B={w.B} H={w.H} L={w.L} dk={w.dk} dv={w.dv} {w.dtype} C={w.chunk}; "
        f"{nsets} input sets of {set_bytes / 1e6:.1f} MB, workspace {ws_bytes / 1e6:.1f} MB")

    def step(i, rotate=True):
        s = sets[i % nsets] if rotate else sets[0]
        st = gla.gla_fwd(dims, code, s["q"], s["k"], s["v"], s["a"], x.h0, s["o"], hT, ws,
                         ws_bytes, stream)
        if st != 0:
            raise gla.GlaError(st, "gla_fwd")

    step(0)
    torch.cuda.synchronize()
    assert torch.isfinite(sets[0]["o"].float()).all().item()
    # the metric's own leg runs exactly the requested warm-up and timed steps;
    # the other legs at least 20 and 50, so that short runs stay steady
    nwarm = args.warmup if primary else max(20, args.warmup)
    ksteps = args.steps if primary else max(50, args.steps)
    for i in range(nwarm):
        step(i)
    ms = timed(step, ksteps, torch)
    log(f"[bench] {w.name}: timed {ksteps} steps, {ms * 1e3:.1f} us/step")
    _abi.gla_profile_begin(ksteps * 8)
    ms_prof = timed(step, ksteps, torch)
    _abi.gla_profile_end()
    per = events_by_kernel(_abi)
    warm = timed(lambda i: step(i, rotate=False), ksteps, torch) if primary else None
    pct = step_percentiles(step, ksteps, torch)

    tokens = w.B * w.L
    flops = w.stated_flops_fwd()
    comp, comp_per = compulsory_fwd(w, esize)
    over = overhead_fwd(w, esize)
    kernels = {}
    tot = sum(sum(v) for v in per.values()) or 1.0
    for name, lst in per.items():
        avg_s = sum(lst) / len(lst) * 1e-3
        cb = comp_per.get(name, 0)
        kernels[name] = {"launches": len(lst), "avg_us": round(avg_s * 1e6, 2),
                         "share": round(sum(lst) / tot, 4),
                         "compulsory_bytes": cb, "overhead_bytes": over.get(name),
                         "compulsory_gbps": round(cb / avg_s / 1e9, 1)}
    dom = max(per, key=lambda n: sum(per[n]))
    dom_s = kernels[dom]["avg_us"] * 1e-6
    tr = measured_traffic(dom, w.name)
    achieved = comp_per.get(dom, 0) / dom_s / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": tr["bytes_per_launch"] if tr else None,
                "traffic_read": tr["read_bytes_per_launch"] if tr else None,
                "traffic_write": tr["write_bytes_per_launch"] if tr else None,
                "compulsory_bytes_per_launch": comp_per.get(dom, 0),
                "overhead_bytes_per_launch": over.get(dom),
                "avg_launch_us": round(dom_s * 1e6, 2)}
    step_gbps = comp / (ms * 1e-3) / 1e9
    out = {"workload": w.name, "steps": ksteps, "ms_per_step": round(ms, 5),
           "ms_per_step_profiled": round(ms_prof, 5),
           "tokens_per_s": round(tokens / (ms * 1e-3), 1),
           "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
           "frac_bf16_mfma_peak": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
           "roofline": roofline,
           "step_roofline": {"bound": "hbm", "compulsory_bytes": comp,
                             "achieved": round(step_gbps, 1), "peak": HBM_PEAK_GBPS,
                             "unit": "GB/s", "frac": round(step_gbps / HBM_PEAK_GBPS, 4)},
           "kernels": kernels, "input_sets": nsets, "step_us_percentiles": pct}
    if warm is not None:
        out["warm"] = {"ms_per_step": round(warm, 5),
                       "tokens_per_s": round(tokens / (warm * 1e-3), 1)}
    del sets, ws
    return out


def backward_leg(w, args, torch, gla, _abi, dev, stream):
    """gla_bwd alone (K calls on the same inputs, which need no forward) and
    forward + backward, with per-launch HIP events of the backward."""
    from chunkwise_linear_rnn_gla_amd.inputs import workload_inputs
    esize = 2 if w.dtype == "bf16" else 4
    code = gla.GLA_BF16 if w.dtype == "bf16" else gla.GLA_FP32
    dims = gla.GlaDims(w.B, w.H, w.L, w.dk, w.dv, w.chunk, w.subchunk)
    xb = workload_inputs(w).to(dev)
    fws = torch.empty(gla.gla_fwd_workspace_size(dims, code), dtype=torch.uint8, device=dev)
    bws = torch.empty(gla.gla_bwd_workspace_size(dims, code), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(xb.q), torch.empty_like(xb.k), torch.empty_like(xb.v),
            torch.empty_like(xb.log_alpha),
            torch.empty(w.B, w.H, w.dk, w.dv, dtype=torch.float32, device=dev)]
    ob = torch.empty_like(xb.v)
    hT = torch.empty(w.B, w.H, w.dk, w.dv, dtype=torch.float32, device=dev)

    def bwd(i):
        st = gla.gla_bwd(dims, code, xb.q, xb.k, xb.v, xb.log_alpha, xb.h0, xb.do, None, *outs,
                         bws, bws.numel(), stream)
        if st:
            raise gla.GlaError(st, "gla_bwd")

    def fb(i):
        st = gla.gla_fwd(dims, code, xb.q, xb.k, xb.v, xb.log_alpha, xb.h0, ob, hT, fws,
                         fws.numel(), stream)
        if st:
            raise gla.GlaError(st, "gla_fwd")
        bwd(i)

    for i in range(max(20, args.warmup)):
        fb(i)
    kb = max(50, args.steps)
    bwd_ms = timed(bwd, kb, torch)
    fb_ms = timed(fb, kb, torch)
    bwd_pct = step_percentiles(bwd, kb, torch)
    # the materialised-state backward on the same inputs, for comparison
    mat_ms = None
    mcfg = gla.bwd_config("materialized")
    try:
        if args.no_materialized:
            raise gla.GlaError(0, "skipped")
        mws = torch.empty(gla.gla_bwd_ex_workspace_size(dims, code, mcfg), dtype=torch.uint8,
                          device=dev)

        def bwd_mat(i):
            st = gla.gla_bwd_ex(dims, code, mcfg, xb.q, xb.k, xb.v, xb.log_alpha, xb.h0, xb.do,
                                None, *outs, mws, mws.numel(), stream)
            if st:
                raise gla.GlaError(st, "gla_bwd_ex")

        for i in range(3):
            bwd_mat(i)
        mat_ms = timed(bwd_mat, max(5, kb // 5), torch)
        del mws
    except gla.GlaError:
        pass
    _abi.gla_profile_begin(kb * 16)
    timed(bwd, kb, torch)
    _abi.gla_profile_end()
    per = events_by_kernel(_abi)
    tokens = w.B * w.L
    comp = compulsory_bwd(w, esize)
    fl = flops_bwd(w)
    gbps = comp / (bwd_ms * 1e-3) / 1e9
    kernels = {}
    for n, l in per.items():
        kernels[n] = {"launches": len(l), "avg_us": round(sum(l) / len(l) * 1e3, 2)}
        tr = measured_traffic(n, w.name)
        if tr:
            kernels[n]["traffic"] = tr["bytes_per_launch"]
            kernels[n]["traffic_read"] = tr["read_bytes_per_launch"]
            kernels[n]["traffic_write"] = tr["write_bytes_per_launch"]
    log(f"[bench] {w.name}: bwd {bwd_ms * 1e3:.1f} us, fwd+bwd {fb_ms * 1e3:.1f} us; {kernels}")
    del fws, bws, outs
    return {"workload": w.name, "steps": kb,
            "ms_per_step": round(fb_ms, 5),
            "tokens_per_s": round(tokens / (fb_ms * 1e-3), 1),
            "bwd_ms": round(bwd_ms, 5), "bwd_step_us_percentiles": bwd_pct,
            "bwd_ms_materialized": round(mat_ms, 5) if mat_ms else None,
            "bwd_tokens_per_s": round(tokens / (bwd_ms * 1e-3), 1),
            "bwd_tflops": round(fl / (bwd_ms * 1e-3) / 1e12, 2),
            "bwd_flops": fl,
            "bwd_roofline": {"bound": "hbm", "compulsory_bytes": comp,
                             "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                             "frac": round(gbps / HBM_PEAK_GBPS, 4)},
            "kernels": kernels}


def decode_leg(w, torch, gla, _abi, dev, stream):
    """One-token decode steps (gla_decode) at the head shape of w: each reads
    and writes the fp32 state once.  The steps rotate over enough state
    buffers (more than the Infinity Cache holds) that each step's state comes
    from HBM."""
    esize = 2 if w.dtype == "bf16" else 4
    code = gla.GLA_BF16 if w.dtype == "bf16" else gla.GLA_FP32
    io = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(5)
    dq_ = (torch.randn(w.B, w.H, w.dk, generator=g) * w.dk ** -0.5).to(io).to(dev)
    dk_ = torch.randn(w.B, w.H, w.dk, generator=g).to(io).to(dev)
    dv_ = torch.randn(w.B, w.H, w.dv, generator=g).to(io).to(dev)
    da_ = (torch.nn.functional.logsigmoid(torch.randn(w.B, w.H, w.dk, generator=g)) / 16.0).to(dev)
    sbytes = w.B * w.H * w.dk * w.dv * 4
    nst = max(2, -(-INFINITY_CACHE_BYTES * 33 // 32 // sbytes))
    states = [torch.zeros(w.B, w.H, w.dk, w.dv, dtype=torch.float32, device=dev)
              for _ in range(nst)]
    do_ = torch.empty(w.B, w.H, w.dv, dtype=io, device=dev)
    dd = gla.GlaDims(w.B, w.H, 1, w.dk, w.dv, w.chunk, 16)

    def dec(i):
        st = gla.gla_decode(dd, code, dq_, dk_, dv_, da_, states[i % nst], do_, stream)
        if st != 0:
            raise gla.GlaError(st, "gla_decode")

    for i in range(200):
        dec(i)
    nd = 2000
    dec_us = timed(dec, nd, torch) * 1e3
    _abi.gla_profile_begin(nd)
    timed(dec, nd, torch)
    _abi.gla_profile_end()
    ev = [ms * 1e3 for lst in events_by_kernel(_abi).values() for ms in lst]
    ev_us = sum(ev) / max(1, len(ev))
    dbytes = (2 * w.B * w.H * w.dk * w.dv * 4
              + w.B * w.H * (2 * w.dk * esize + w.dk * 4 + 2 * w.dv * esize))
    del states
    log(f"[bench] decode {dec_us:.2f} us/step ({ev_us:.2f} us by event bracket)")
    return {"workload": f"decode B{w.B} H{w.H} dk{w.dk} dv{w.dv} one token, fp32 state",
            "state_buffers": nst, "us_per_step": round(dec_us, 2),
            "tokens_per_s": round(w.B / (dec_us * 1e-6), 1),
            "kernel_us_events": round(ev_us, 2), "bytes_per_step": dbytes,
            "achieved_gbps": round(dbytes / (dec_us * 1e-6) / 1e9, 1),
            "frac_hbm_peak": round(dbytes / (dec_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}


def general_leg(w, args, torch, gla, _abi, dev, stream):
    """The general gate G = alpha^T beta (ggla_fwd / ggla_bwd) at the head
    shape of w, with a column gate drawn like the row gate."""
    from chunkwise_linear_rnn_gla_amd.inputs import make_log_beta, workload_inputs
    esize = 2 if w.dtype == "bf16" else 4
    code = gla.GLA_BF16 if w.dtype == "bf16" else gla.GLA_FP32
    dims = gla.GlaDims(w.B, w.H, w.L, w.dk, w.dv, w.chunk, w.subchunk)
    x = workload_inputs(w).to(dev)
    lbg = make_log_beta(w.B, w.H, w.L, w.dv, seed=w.seed).to(dev)
    gws = torch.empty(gla.ggla_bwd_workspace_size(dims, code), dtype=torch.uint8, device=dev)
    og = torch.empty_like(x.v)
    hg = torch.empty(w.B, w.H, w.dk, w.dv, dtype=torch.float32, device=dev)
    gouts = [torch.empty_like(x.q), torch.empty_like(x.k), torch.empty_like(x.v),
             torch.empty_like(x.log_alpha), torch.empty_like(lbg)]
    dog = torch.randn(w.B, w.H, w.L, w.dv, generator=torch.Generator().manual_seed(6)
                      ).to(x.q.dtype).to(dev)

    def gf(i=0):
        st = gla.ggla_fwd(dims, code, x.q, x.k, x.v, x.log_alpha, lbg, None, og, hg, gws,
                          gws.numel(), stream)
        if st:
            raise gla.GlaError(st, "ggla_fwd")

    def gfb(i=0):
        gf()
        st = gla.ggla_bwd(dims, code, x.q, x.k, x.v, x.log_alpha, lbg, None, dog, None, *gouts,
                          None, gws, gws.numel(), stream)
        if st:
            raise gla.GlaError(st, "ggla_bwd")

    res = {}
    for name, fn, kk in (("fwd", gf, max(20, args.steps)), ("fwd_bwd", gfb, max(5, args.steps // 2))):
        for i in range(5):
            fn(i)
        res[name] = timed(fn, kk, torch)
    kf = max(20, args.steps)
    _abi.gla_profile_begin(2 * kf)
    timed(gf, kf, torch)
    _abi.gla_profile_end()
    per = events_by_kernel(_abi)
    nc16 = -(-w.L // 16)
    rb = 32 * w.dk * esize + 4 * 272 + 4 * w.dk   # one 16-token record
    BH = w.B * w.H
    gbytes = {"gg_prep": BH * w.L * (2 * w.dk * esize + 4 * w.dk) + BH * nc16 * rb,
              "gg_recur": BH * nc16 * rb + BH * w.L * w.dv * (2 * esize + 4) + BH * w.dk * w.dv * 4}
    gk = {}
    for nm, lst in per.items():
        avg = sum(lst) / len(lst) * 1e-3
        mt = measured_traffic(nm, "general_" + w.name)
        gk[nm] = {"avg_us": round(avg * 1e6, 2), "algorithmic_bytes": gbytes.get(nm),
                  "achieved_gbps": round(gbytes[nm] / avg / 1e9, 1) if nm in gbytes else None,
                  "traffic": mt["bytes_per_launch"] if mt else None}
    tokens = w.B * w.L
    del gws, og, hg, gouts, dog, lbg
    log(f"[bench] general gate fwd {res['fwd'] * 1e3:.1f} us, fwd+bwd {res['fwd_bwd'] * 1e3:.1f} us")
    return {"workload": f"general gate B{w.B} H{w.H} L{w.L} dk{w.dk} dv{w.dv} {w.dtype}",
            "fwd_ms": round(res["fwd"], 4),
            "fwd_tokens_per_s": round(tokens / (res["fwd"] * 1e-3), 1),
            "fwd_bwd_ms": round(res["fwd_bwd"], 4),
            "fwd_bwd_tokens_per_s": round(tokens / (res["fwd_bwd"] * 1e-3), 1),
            "kernels": gk}


def layer_leg(w, args, torch, dev, fwd_ms, fb_ms):
    """The op-level layer (projections, gate, norm and output gate in torch,
    the recurrence in the kernels) at d = H * dv, which gives w's head shape;
    seeded random weights."""
    from chunkwise_linear_rnn_gla_amd.layer import GlaLayer
    io = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    d_model = w.H * w.dv
    lay = GlaLayer(d_model, w.H, chunk=w.chunk, seed=9, dtype=io, device=dev)
    g = torch.Generator().manual_seed(10)
    xl = torch.randn(w.B, w.L, d_model, generator=g).to(io).to(dev)
    dyl = torch.randn(w.B, w.L, d_model, generator=g).to(io).to(dev)
    xg = xl.clone().requires_grad_(True)

    def lf(i=0):
        with torch.no_grad():
            lay(xl)

    def lfb(i=0):
        lay(xg).backward(dyl)

    res = {}
    for name, fn in (("fwd", lf), ("fwd_bwd", lfb)):
        for i in range(5):
            fn(i)
        res[name] = timed(fn, max(5, args.steps // 2), torch)
    tokens = w.B * w.L
    out = {"workload": f"GLA layer d{d_model} heads{w.H} B{w.B} L{w.L} {w.dtype}",
           "fwd_ms": round(res["fwd"], 4),
           "fwd_tokens_per_s": round(tokens / (res["fwd"] * 1e-3), 1),
           "fwd_bwd_ms": round(res["fwd_bwd"], 4),
           "fwd_bwd_tokens_per_s": round(tokens / (res["fwd_bwd"] * 1e-3), 1),
           "core_share_fwd": round(fwd_ms / res["fwd"], 4)}
    if fb_ms:
        out["core_share_fwd_bwd"] = round(fb_ms / res["fwd_bwd"], 4)
    log(f"[bench] layer fwd {res['fwd'] * 1e3:.1f} us, fwd+bwd {res['fwd_bwd'] * 1e3:.1f} us")
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(w):
    """The fp64 oracle (token recurrence, C) timed on the host cores over the
    whole workload: threads = the CPUs this process may use (at most 16, one
    (batch, head) pair per task), median of 3 runs, plus one run on 1 thread."""
    import oracle
    from chunkwise_linear_rnn_gla_amd.inputs import as_f64, workload_inputs
    x = workload_inputs(w)
    f64 = [as_f64(t) for t in (x.q, x.k, x.v, x.log_alpha, x.h0)]
    try:
        host = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        host = os.cpu_count() or 1
    threads = oracle.default_threads()
    times = []
    for r in range(3):
        tc = time.perf_counter()
        oracle.fwd(*f64, nthreads=threads)
        times.append(time.perf_counter() - tc)
        log(f"[bench] oracle run {r}: {times[-1]:.2f} s on {threads} threads")
    t1 = time.perf_counter()
    oracle.fwd(*f64, nthreads=1)
    t1 = time.perf_counter() - t1
    log(f"[bench] oracle run on 1 thread: {t1:.2f} s")
    tcpu = statistics.median(times)
    tokens = w.B * w.L
    # the oracle's own arithmetic: per head-token a decay multiply and an
    # outer-product multiply-add on every state entry (3 flops) and the output
    # row q S (2 flops per entry)
    own = 5.0 * w.B * w.H * w.L * w.dk * w.dv
    return {"value": round(tokens / tcpu, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the whole {w.name} forward (B{w.B} H{w.H} L{w.L} dk{w.dk} dv{w.dv}), "
                      f"fp64 token recurrence in C, one (batch, head) pair per task; median of 3 "
                      f"runs on {threads} threads, and one run on 1 thread",
            "seconds": round(tcpu, 3),
            "host_cpus": host, "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "gflops_oracle_work": round(own / tcpu / 1e9, 2),
            "gflops_stated_count": round(w.stated_flops_fwd() / tcpu / 1e9, 2),
            "one_thread": {"seconds": round(t1, 3), "tokens_per_s": round(tokens / t1, 1),
                           "gflops_oracle_work": round(own / t1 / 1e9, 2)}}


# ----------------------------------------------------------------- counter records

def _counter_sums(d):
    """{launch name: (dispatches, mean counter value)} from a rocprofv3 --pmc
    run's counter_collection.csv files under directory d."""
    acc = {}
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    for fn in files:
        with open(fn) as f:
            per_dispatch = {}
            for row in csv.DictReader(f):
                name = launch_name(row.get("Kernel_Name", ""))
                if name is None:
                    continue
                did = row.get("Dispatch_Id")
                per_dispatch[(name, did)] = per_dispatch.get((name, did), 0.0) + float(
                    row["Counter_Value"])
            for (name, _), val in per_dispatch.items():
                n, s = acc.get(name, (0, 0.0))
                acc[name] = (n + 1, s + val)
    return {k: (n, s / n) for k, (n, s) in acc.items()}


def ingest_counters(fetch_dir, write_dir, workload, cal_fetch, cal_write):
    """Write profiles/traffic.json entries for `workload` from FETCH_SIZE and
    WRITE_SIZE runs, scaled by what the same counters read for the 1 GiB
    calibration copy (--calibrate-copy)."""
    def cal(d):
        """Median per-dispatch counter value of the calibration run, which
        launches only torch's copy kernel."""
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        vals = {}
        for fn in files:
            with open(fn) as f:
                for row in csv.DictReader(f):
                    vals[row.get("Dispatch_Id")] = vals.get(row.get("Dispatch_Id"), 0.0) + float(
                        row["Counter_Value"])
        v = sorted(vals.values())
        return v[len(v) // 2]
    kib = CALIBRATE_BYTES / 1024
    fetch_scale = kib / cal(cal_fetch)     # bytes read per copy / FETCH_SIZE KiB
    write_scale = kib / cal(cal_write)
    fe, wr = _counter_sums(fetch_dir), _counter_sums(write_dir)
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec["note"] = ("HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per "
                   "dispatch), scaled by what the same counters read for a plain 1 GiB device "
                   "copy; bench.py reports them only while the listed sources hash to "
                   "sources_sha256.")
    entries = [e for e in rec.get("entries", []) if e.get("workload") != workload]
    for name in sorted(set(fe) & set(wr)):
        srcs = kernel_sources(name)
        rb = fe[name][1] * 1024 * fetch_scale
        wb = wr[name][1] * 1024 * write_scale
        entries.append({"kernel": name, "workload": workload, "dispatches": fe[name][0],
                        "fetch_size_kib": round(fe[name][1], 1),
                        "write_size_kib": round(wr[name][1], 1),
                        "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4),
                        "read_bytes_per_launch": int(rb), "write_bytes_per_launch": int(wb),
                        "bytes_per_launch": int(rb + wb),
                        "sources": srcs, "sources_sha256": sources_digest(srcs)})
    rec["entries"] = entries
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    for e in entries:
        if e["workload"] == workload:
            log(f"{e['kernel']}: read {e['read_bytes_per_launch'] / 1e6:.1f} MB, "
                f"write {e['write_bytes_per_launch'] / 1e6:.1f} MB per launch")


# ----------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gla340m_fwd")
    ap.add_argument("--sets", type=int, default=0, help="input copies to rotate over (0 = auto)")
    ap.add_argument("--only", choices=["fwd", "bwd", "general"], default=None,
                    help="run only the forward of --workload, only its backward, or only the "
                         "general gate at its head shape (for profiler runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the 1.3B-shape and long-sequence forward legs")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward leg")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step figure")
    ap.add_argument("--no-layer", action="store_true", help="skip the op-level layer figure")
    ap.add_argument("--no-general", action="store_true", help="skip the general-gate figure")
    ap.add_argument("--no-materialized", action="store_true",
                    help="skip timing the materialised-state backward beside the recurrent one")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (3 times), the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    ap.add_argument("--ingest-counters", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "WORKLOAD"))
    ap.add_argument("--calibration", nargs=2, metavar=("CAL_FETCH_DIR", "CAL_WRITE_DIR"))
    args = ap.parse_args()

    if args.ingest_counters:
        if not args.calibration:
            raise SystemExit("--ingest-counters needs --calibration CAL_FETCH_DIR CAL_WRITE_DIR")
        ingest_counters(*args.ingest_counters, *args.calibration)
        return

    if args.calibrate_copy:
        import torch
        dev = torch.device("cuda:0")
        src = torch.ones(CALIBRATE_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration: 3 copies of {CALIBRATE_BYTES} bytes")
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library has no "
              "multi-GPU path; see the sharding notes in the design document.", file=sys.stderr)
        sys.exit(2)

    import torch
    import chunkwise_linear_rnn_gla_amd as gla
    from chunkwise_linear_rnn_gla_amd import _abi
    from chunkwise_linear_rnn_gla_amd.inputs import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    w = WORKLOADS[args.workload]

    if args.only == "bwd":
        wb = w if w.backward else WORKLOADS["gla340m_fwdbwd"]
        print(json.dumps({"backward": backward_leg(wb, args, torch, gla, _abi, dev, stream)}))
        return
    if args.only == "general":
        print(json.dumps({"general": general_leg(w, args, torch, gla, _abi, dev, stream)}))
        return

    copy_gbps = copy_bandwidth(torch, dev)
    main_leg = forward_leg(w, args, torch, gla, _abi, dev, stream, primary=True)
    if args.only == "fwd":
        print(json.dumps(main_leg))
        return
    ms = main_leg["ms_per_step"]

    legs = {}
    if not args.no_legs:
        for name in ("gla1p3b_fwd", "long16k_fwd"):
            if name == w.name:
                continue
            try:
                legs[name] = forward_leg(WORKLOADS[name], args, torch, gla, _abi, dev, stream,
                                         primary=False)
            except Exception as e:  # reported, not hidden
                legs[name] = {"error": f"{type(e).__name__}: {e}"}
                log(f"[bench] {name} failed: {e}")

    backward = None
    if not args.no_bwd:
        try:
            backward = backward_leg(WORKLOADS["gla340m_fwdbwd"], args, torch, gla, _abi, dev,
                                    stream)
        except Exception as e:  # reported, not hidden
            backward = {"error": f"{type(e).__name__}: {e}"}
            log(f"[bench] backward failed: {e}")

    decode = None
    if not args.no_decode:
        try:
            decode = decode_leg(w, torch, gla, _abi, dev, stream)
        except Exception as e:  # reported, not hidden
            decode = {"error": f"{type(e).__name__}: {e}"}
            log(f"[bench] decode failed: {e}")

    general = None
    if not args.no_general:
        general = {}
        shapes = [w] if args.no_legs else [w, WORKLOADS["gla1p3b_fwd"]]
        for wg in shapes:
            try:
                general[wg.name] = general_leg(wg, args, torch, gla, _abi, dev, stream)
            except Exception as e:  # reported, not hidden
                general[wg.name] = {"error": f"{type(e).__name__}: {e}"}
                log(f"[bench] general gate failed: {e}")

    layer = None
    if not args.no_layer:
        try:
            fb = backward.get("ms_per_step") if backward else None
            layer = layer_leg(w, args, torch, dev, ms, fb)
        except Exception as e:  # reported, not hidden
            layer = {"error": f"{type(e).__name__}: {e}"}
            log(f"[bench] layer failed: {e}")

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w)

    out = {
        "metric": METRIC, "value": main_leg["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "ms_per_step_profiled": main_leg["ms_per_step_profiled"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "dk": w.dk, "dv": w.dv,
                   "chunk": w.chunk, "subchunk": w.subchunk,
                   "input_sets": main_leg["input_sets"]},
        "tflops": main_leg["tflops"], "frac_bf16_mfma_peak": main_leg["frac_bf16_mfma_peak"],
        "warm": main_leg.get("warm"),
        "step_us_percentiles": main_leg["step_us_percentiles"],
        "roofline": main_leg["roofline"], "step_roofline": main_leg["step_roofline"],
        "kernels": main_leg["kernels"], "copy_gbps": round(copy_gbps, 1),
        "legs": legs, "fwd_bwd": backward, "decode": decode, "general": general,
        "layer": layer, "cpu_baseline": cpu,
        # the build, identified by its kernel sources (GPU runs see no git
        # history)
        "build": {"sources_sha256": sources_digest(KERNEL_SOURCES)},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
