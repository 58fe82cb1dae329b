#!/usr/bin/env python3
"""Decode-step benchmark of the Fathom bit-plane key scan on one MI355X.

One step = plan (water-filling per KV-head group) + scan (scores of every
cached key from the t_j-plane prefixes) + top-k per query head + union per KV
head, over all layer x KV-head pairs of the workload, with the index already
resident in HBM (or in mapped pinned host memory for the host-resident
workload).  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload long1m]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "scan+top-k ms/decode step at 1M tokens; achieved GB/s vs HBM peak"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long1m")
    ap.add_argument("--budget", type=int, default=None, help="override the plane-bit budget")
    ap.add_argument("--mode", type=int, default=0, help="0 water-filling, 1 fixed top-r, 2 uniform")
    ap.add_argument("--cpu-baseline", type=int, default=1, help="time the CPU oracle beside it")
    ap.add_argument("--cpu-pairs", type=int, default=32)
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the all-cores leg (0: the CPUs this process may use, at most 16)")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def copy_probe(mib: int):
    """A plain copy of known size, for scaling the HBM byte counters."""
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)


def sample_fraction(n: int, k: int, run: int = 32) -> float:
    """Share of the index blocks in the fused threshold's sample: one run of
    `run` blocks (32, or 512 for an index read over the host link) in every
    s runs, s the largest power of two with (2s)^2 4k <= n and 2s <= the
    block count (the library's rule).  Over the host link the sample stage
    reads these blocks and the filter the rest."""
    nb = (n + 63) // 64
    s = 1
    while (2 * s) ** 2 * 4 * k <= n and 2 * s <= nb:
        s *= 2
    runs = (nb + run - 1) // run
    sampled = sum(min(run, nb - r * run) for r in range(0, runs, s))
    return sampled / nb


def src_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def scan_counters(workload: str) -> dict:
    """Committed rocprofv3 counters of the filtered scan (HBM bytes per launch,
    instruction mix), if they were taken on the current scan source; else {}."""
    f = os.path.join(ROOT, "profiles", f"scan_{workload}_pmc.json")
    if not os.path.exists(f):
        return {}
    d = json.load(open(f))
    if d.get("scan_src_sha256_16") != src_hash(os.path.join(ROOT, "sparse_attention_key_amd", "csrc", "scan.hip")):
        return {}
    return d


def build_index(F, w, device):
    import torch

    import workloads as wl

    nb = w.nb
    planes = torch.empty((w.P, w.D, 4, nb), dtype=torch.int64, device=device)
    scales = torch.empty((w.P, w.D, nb), dtype=torch.int16, device=device)
    chunk = 16
    t0 = time.time()
    for p0 in range(0, w.P, chunk):
        pairs = list(range(p0, min(w.P, p0 + chunk)))
        keys = wl.keys_device(w, pairs, device=device)
        F.pack_into(keys, planes[p0:p0 + len(pairs)], scales[p0:p0 + len(pairs)])
        del keys
        if (p0 // chunk) % 4 == 0:
            torch.cuda.synchronize()
            log(f"packed pairs {p0}..{pairs[-1]} ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()
    return planes, scales


def inputs(F, w, device):
    """Queries, and the calibration statistics computed on the device from
    each pair's calibration sample: per-channel variances, or for rotated
    storage the KLT basis and the variances of the rotated coordinates.
    Returns q (numpy), s2 and rot (device tensors) and the calibration time."""
    import torch

    import workloads as wl

    q = np.stack([wl.queries(w, p) for p in range(w.P)])
    keys = torch.from_numpy(np.stack([wl.calibration_sample(w, p) for p in range(w.P)])).to(device)
    cov, s2 = F.calib_covariance(keys, with_cov=w.rotated)
    rot = None
    if w.rotated:
        rot, s2 = F.calib_basis(cov)
    torch.cuda.synchronize()
    calib = calib_probe(F, keys, w.rotated)
    del keys, cov
    return q, s2, rot, calib


def calib_probe(F, keys, basis: bool, reps: int = 3):
    """Device time of the calibration statistics for these keys [P][m][D]
    (covariance, and the eigenbasis when the storage is rotated), and of the
    per-KV-head statistics from a session's own prefill: one layer's 8 KV
    heads x 102,400 keys, covariance alone and with the eigenbasis."""
    import torch

    def timed(k, with_basis):
        F.calib_covariance(k, with_cov=with_basis)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            cov, _ = F.calib_covariance(k, with_cov=with_basis)
            if with_basis:
                F.calib_basis(cov)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = {"pairs": int(keys.shape[0]), "keys_per_pair": int(keys.shape[1]), "basis": bool(basis),
           "ms": round(timed(keys, basis), 3)}
    g = torch.Generator(device=keys.device).manual_seed(20260915)
    pre = (torch.randn((8, 102400, keys.shape[2]), device=keys.device, generator=g)).to(torch.bfloat16)
    out["prefill_8x102400_cov_ms"] = round(timed(pre, False), 3)
    out["prefill_8x102400_cov_basis_ms"] = round(timed(pre, True), 3)
    del pre
    return out


def build_host_index(F, w, rot, device):
    """Keys drawn on the GPU, rotated into the calibration basis (a float32
    GEMM of the input generator side), packed on the GPU chunk by chunk and
    copied into mapped pinned host memory."""
    import torch

    import workloads as wl

    nb = w.nb
    pbytes = w.D * 4 * nb * 8
    sbytes = w.D * nb * 2
    from sparse_attention_key_amd.hostmem import PinnedHost

    planes_h = PinnedHost(w.P * pbytes)
    scales_h = PinnedHost(w.P * sbytes)
    chunk = 8
    stream = torch.cuda.current_stream()
    planes = torch.empty((chunk, w.D, 4, nb), dtype=torch.int64, device=device)
    scales = torch.empty((chunk, w.D, nb), dtype=torch.int16, device=device)
    t0 = time.time()
    for p0 in range(0, w.P, chunk):
        pairs = list(range(p0, min(w.P, p0 + chunk)))
        keys = wl.keys_device(w, pairs, device=device)
        y = torch.empty((len(pairs), w.n, w.D), dtype=torch.float32, device=device)
        for i, p in enumerate(pairs):
            y[i] = keys[i].float() @ rot[p]
        del keys
        F.pack_into(y, planes[: len(pairs)], scales[: len(pairs)])
        del y
        planes_h.copy_from_device(p0 * pbytes, planes.data_ptr(), len(pairs) * pbytes, stream)
        scales_h.copy_from_device(p0 * sbytes, scales.data_ptr(), len(pairs) * sbytes, stream)
        torch.cuda.synchronize()
        if (p0 // chunk) % 8 == 0:
            log(f"packed pairs {p0}..{pairs[-1]} into pinned host memory ({time.time() - t0:.1f}s)")
    del planes, scales
    torch.cuda.empty_cache()
    return planes_h, scales_h


def link_probes(F, planes_h, device):
    """Host-link read bandwidth: zero-copy streaming reads of the mapped
    index, and pinned host-to-device hipMemcpy, over the same 4 GiB."""
    import torch

    nbytes = min(4 << 30, planes_h.nbytes)
    sink = torch.zeros(1024, dtype=torch.int32, device=device)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=device)
    stream = torch.cuda.current_stream()
    res = {}
    for name, fn in (("zero_copy_read", lambda: F.read_probe(planes_h.dev, nbytes, sink)),
                     ("pinned_h2d_memcpy", lambda: planes_h.copy_to_device(dst.data_ptr(), 0, nbytes, stream))):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(3 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9, 2)
    del dst
    torch.cuda.empty_cache()
    return res


def hbm_probe(F, planes, device):
    """Streaming read bandwidth of the HBM-resident index itself."""
    import torch

    nbytes = planes.numel() * 8
    sink = torch.zeros(1024, dtype=torch.int32, device=device)
    F.read_probe(planes, nbytes, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        F.read_probe(planes, nbytes, sink)
    e1.record()
    torch.cuda.synchronize()
    return round(5 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)


def fetch_probe(F, w, out, device):
    """Winner-row fetch after the step: the union rows of every pair (K and V
    of one token side by side, bf16, D=128 each: 512 B) gathered from a
    row table in mapped pinned host memory into HBM.  One table of n rows is
    shared by all pairs (the link carries the same bytes as per-pair tables,
    without 151 GB of pinned memory)."""
    import torch

    from sparse_attention_key_amd.hostmem import PinnedHost

    row_bytes = 2 * w.D * 2
    nbytes = w.n * row_bytes
    src = torch.randint(-32768, 32767, (nbytes // 2,), dtype=torch.int16, device=device)
    table = PinnedHost(nbytes)
    table.copy_from_device(0, src.data_ptr(), nbytes, torch.cuda.current_stream())
    torch.cuda.synchronize()
    del src
    cap = out.union.shape[1]
    dst = torch.empty((w.P, cap, row_bytes // 2), dtype=torch.int16, device=device)
    F.gather_rows(table.dev, w.n, row_bytes, 0, out.union, out.union_len, dst)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        F.gather_rows(table.dev, w.n, row_bytes, 0, out.union, out.union_len, dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    rows = int(out.union_len.to(torch.int64).sum().item())
    table.free()
    del dst
    torch.cuda.empty_cache()
    return {"rows": rows, "bytes": rows * row_bytes, "ms": round(ms, 4),
            "GBps": round(rows * row_bytes / (ms * 1e-3) / 1e9, 2),
            "source": "mapped pinned host memory, K|V rows of 512 B (bf16, D=128)"}


def per_layer_probe(F, w, planes, scales, q, s2, rot, budget, mode, device, reps=3):
    """The same decode step as 36 sequential calls, one per layer with its
    8 KV heads (P = 8), the way a model's layers run one after another:
    plan and fused scan + top-k per call.  Timed eagerly and as one captured
    HIP graph of all layers replayed (the calls are launch-bound at P = 8);
    every replay's winners are checked against the eager ones."""
    import torch

    per = w.kv_heads
    layers = w.P // per
    plans = [F.Plan(per, w.G, w.D, device) for _ in range(layers)]
    outs = [F.TopkOut(per, w.G, w.n, w.k, device, fused=True) for _ in range(layers)]
    sl = lambda L: slice(L * per, (L + 1) * per)
    rot_l = (lambda L: None) if rot is None else (lambda L: rot[sl(L)])

    if isinstance(planes, int):  # mapped host memory: device addresses of each layer's pairs
        pb, sb = w.D * 4 * w.nb * 8, w.D * w.nb * 2
        idx_of = lambda L: (planes + L * per * pb, scales + L * per * sb)
    else:
        idx_of = lambda L: (planes[sl(L)], scales[sl(L)])

    def all_layers():
        for L in range(layers):
            F.plan_into(plans[L], q[sl(L)], s2[sl(L)], budget, mode, rot=rot_l(L))
            pl_, sc_ = idx_of(L)
            F.scan_topk_into(pl_, sc_, w.n, plans[L], outs[L])

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    eager_ms = timed(all_layers)
    ref = [(o.idx.clone(), o.union.clone(), o.union_len.clone()) for o in outs]
    res = {"layers": layers, "pairs_per_call": per, "eager_ms_total": round(eager_ms, 4),
           "eager_ms_per_layer": round(eager_ms / layers, 4)}
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            all_layers()  # warm up on the capture stream
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            all_layers()
        same = True
        for _ in range(3):  # eager work and a sync between replays, each replay checked
            for o in outs:
                o.idx.fill_(-7)
            graph.replay()
            torch.cuda.synchronize()
            same &= all(torch.equal(o.idx, r[0]) and torch.equal(o.union, r[1]) and torch.equal(o.union_len, r[2])
                        for o, r in zip(outs, ref))
        graph_ms = timed(graph.replay)
        res.update({"graph_ms_total": round(graph_ms, 4), "graph_ms_per_layer": round(graph_ms / layers, 4),
                    "graph_same_result": bool(same)})
        del graph
    except Exception as e:  # capture unsupported here: report the eager numbers only
        res["graph_error"] = str(e)[:200]
    del plans, outs
    torch.cuda.empty_cache()
    return res


def append_probe(F, w, planes, scales, device):
    """Cost of ingesting one new key per pair: the block of the last token is
    repacked from its raw keys (its scale is recomputed from all of them), for
    every pair in one call.  The bench index is dense, so the last block is
    repacked in place; it runs after every timed step."""
    import torch

    tok0 = (w.nb - 1) * 64
    m = w.n - tok0
    keys = (torch.randn((w.P, m, w.D), device=device) * 2).to(torch.bfloat16)
    F.pack_range(keys, tok0, planes, scales)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        F.pack_range(keys, tok0, planes, scales)
    e1.record()
    torch.cuda.synchronize()
    return {"pairs": w.P, "tokens_in_block": m, "us_per_call": round(e0.elapsed_time(e1) / reps * 1e3, 2)}


def cpu_info() -> dict:
    """Host CPU facts for the baseline line: model string, online CPUs, and
    the CPUs this process may run on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity_cpus": affinity}


def cpu_baseline(w, q, budget, mode, pairs, threads, single_pairs=2):
    """Time the CPU oracle (as it stands) on a bounded sample of pairs: the
    same plan + scores + top-k + union per pair.  Two legs: one pair after
    another on one thread, and the sample spread over `threads` host threads
    (one pair per thread at a time).  Both are scaled to a whole step of all
    pairs.  The oracle's calibration statistics come from the oracle, on the
    same calibration samples."""
    import oracle
    import workloads as wl

    import torch

    pairs = min(pairs, w.P)
    sel = [int(p) for p in np.linspace(0, w.P - 1, pairs).round()]
    s2, rot = {}, None
    if w.rotated:
        rot = {}
        for p in sel:
            rot[p], s2[p] = oracle.calib.klt_basis(wl.calibration_sample(w, p))
    else:
        for p in sel:
            s2[p] = oracle.calib.channel_variance(wl.calibration_sample(w, p))
    packed = {}
    t0 = time.time()

    def prep(p, x):
        if rot is not None:
            x = (x.astype(np.float64) @ rot[p].astype(np.float64)).astype(np.float32)
        packed[p] = oracle.pack(x)

    # keys drawn by the input generator a few pairs at a time (host memory stays bounded)
    with cf.ThreadPoolExecutor(max_workers=min(threads, pairs)) as ex:
        for c0 in range(0, pairs, 8):
            chunk = sel[c0:c0 + 8]
            keys = [wl.keys_device(w, [p])[0].float().cpu().numpy() for p in chunk]
            list(ex.map(prep, chunk, keys))
            del keys
    torch.cuda.empty_cache()
    log(f"cpu baseline: oracle packed {pairs} pairs on the host in {time.time() - t0:.1f}s")

    def run(p):
        pl, sc = packed[p]
        oracle.step(pl, sc, w.n, q[p], s2[p], budget, w.k, mode=mode,
                    rot=None if rot is None else rot[p])

    single = sel[:single_pairs]
    t0 = time.perf_counter()
    for p in single:
        run(p)
    wall1 = time.perf_counter() - t0
    ms1 = wall1 * 1e3 * w.P / len(single)
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(run, sel))
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 * w.P / pairs
    used = min(threads, pairs)
    info = cpu_info()
    log(f"cpu baseline: {ms1:.0f} ms/step on one thread, {ms_step:.0f} ms/step on {used} threads; {info}")
    return {"value": round(ms_step, 3), "unit": "ms/step", "cores": used, "kind": "oracle",
            "sample": f"{pairs} of {w.P} pairs at n={w.n} (plan+fixed-point scores+top-k+union per pair), "
                      f"{used} pairs at a time on {used} host threads ({wall:.1f}s wall), scaled x{w.P / pairs:.1f}",
            "single_thread": {"value": round(ms1, 3), "unit": "ms/step", "cores": 1,
                              "sample": f"{len(single)} pairs one after another ({wall1:.1f}s), "
                                        f"scaled x{w.P / len(single):.1f}"},
            **info}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}); the scan shards by "
              f"(layer, KV head) pair with no exchange, so run one process per GPU.", file=sys.stderr)
        sys.exit(2)
    if a.copy_probe:
        copy_probe(a.copy_probe)
        return
    import torch

    import workloads as wl
    from sparse_attention_key_amd import fathom as F

    w = wl.WORKLOADS[a.workload]
    budget = w.budget if a.budget is None else a.budget
    dev = torch.device("cuda:0")
    F.lib()
    log(f"workload {w.name}: P={w.P} n={w.n} G={w.G} D={w.D} B={budget} k={w.k} mode={a.mode}")
    q_np, s2, rot, calib = inputs(F, w, dev)
    log(f"calibration on the device: {calib}")
    host = None
    link = {}
    if w.host_resident:
        host = build_host_index(F, w, rot, dev)
        planes, scales = host[0].dev, host[1].dev  # device addresses of mapped host memory
        link = link_probes(F, host[0], dev)
        log(f"host link: {link}")
    else:
        planes, scales = build_index(F, w, dev)
        link = {"hbm_read_probe": hbm_probe(F, planes, dev)}
        log(f"HBM streaming read of the index: {link['hbm_read_probe']} GB/s")
    q = torch.from_numpy(q_np).to(dev)
    pl = F.Plan(w.P, w.G, w.D, dev)
    npad = w.nb * 64
    out = F.TopkOut(w.P, w.G, w.n, w.k, dev, fused=True)

    ev = lambda: torch.cuda.Event(enable_timing=True)

    def step(rec=None):
        """plan, then the three stages of the fused scan + top-k."""
        if rec is not None:
            rec[0].record()
        F.plan_into(pl, q, s2, budget, a.mode, rot=rot)
        for s_ in (1, 2, 3):
            if rec is not None:
                rec[s_].record()
            F.scan_topk_stage(s_, planes, scales, w.n, pl, out)
        if rec is not None:
            rec[4].record()

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    recs = [[ev() for _ in range(5)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in recs:
        step(r)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / a.steps
    span = lambda i, j: float(np.mean([r[i].elapsed_time(r[j]) for r in recs]))
    plan_ms, thr_ms, scan_ms, sel_ms, gpu_ms = span(0, 1), span(1, 2), span(2, 3), span(3, 4), span(0, 4)

    # the same step with materialised scores (fathom_scan + fathom_topk), for reference
    scores = torch.empty((w.P, w.G, npad), dtype=torch.float32, device=dev)
    mout = F.TopkOut(w.P, w.G, w.n, w.k, dev)
    mrec = [[ev() for _ in range(3)] for _ in range(3)]
    for r in [None] + mrec:
        if r is not None:
            r[0].record()
        F.plan_into(pl, q, s2, budget, a.mode, rot=rot)
        F.scan_into(planes, scales, w.n, pl, scores)
        if r is not None:
            r[1].record()
        F.topk_into(scores, w.n, mout)
        if r is not None:
            r[2].record()
    torch.cuda.synchronize()
    mat_scan = float(np.mean([r[0].elapsed_time(r[1]) for r in mrec]))
    mat_total = float(np.mean([r[0].elapsed_time(r[2]) for r in mrec]))
    same = bool(torch.equal(mout.idx, out.idx) and torch.equal(mout.union, out.union))
    del scores, mout
    torch.cuda.empty_cache()

    depth = pl.depth.to(torch.int64)
    bits = depth.sum(1)  # plane bits per token, per pair
    act = (depth > 0).sum(1)
    alg_bytes = int(((bits * 8 + act * 2) * w.nb).sum().item())  # plane words + fp16 scales
    bits_tok = float((bits.double() + 16.0 * act.double() / 64.0).mean().item())
    achieved = alg_bytes / (scan_ms * 1e-3) / 1e9
    log(f"step {ms_step:.3f} ms wall, gpu {gpu_ms:.3f} ms (plan {plan_ms:.3f}, threshold {thr_ms:.3f}, "
        f"scan {scan_ms:.3f}, select {sel_ms:.3f}); scan {achieved:.0f} GB/s algorithmic; "
        f"bits/token {bits_tok:.2f}; materialised path {mat_total:.3f} ms (scan {mat_scan:.3f}), same={same}")

    if host is None:
        # The filtered scan streams the index once: its roofline is HBM.  The
        # algorithmic bytes are the plane words of the planned depths and the
        # fp16 scales of the active channels, over every block of every pair.
        prof = scan_counters(w.name)
        roof = {"bound": "hbm", "kernel": "scan_kernel (filter)", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": prof.get("hbm_bytes_per_launch"), "alg_bytes_per_launch": alg_bytes,
                "measured_read_probe_GBs": link["hbm_read_probe"],
                # issue profile of the same kernel source (rocprofv3 SQ counters):
                # wavefront instructions per 64-token block and stall share
                "issue": {k: v for k, v in (prof.get("issue") or {}).items()
                          if k not in ("counters_mean_of_dispatches", "commands")} or None}
    else:
        # Over the host link every plane word and scale the plan reads must
        # cross the link once per step, so these bytes over the whole step's
        # GPU time (plan, sample, filtered scan, select) cannot exceed the
        # link's rate; the peak is the faster of two measured ways of moving
        # the same index over the link.  (The sample stage reads the sampled
        # runs and the filter every other block, each once; their own rates
        # are reported beside the fraction.)
        peak = max(link["zero_copy_read"], link["pinned_h2d_memcpy"])
        fs = sample_fraction(w.n, w.k, run=512)
        step_gbs = alg_bytes / (gpu_ms * 1e-3) / 1e9
        roof = {"bound": "host_link", "kernel": "whole step (plan, sample, filtered scan, select)",
                "achieved": round(step_gbs, 2), "peak": peak,
                "peak_kind": "max of measured zero-copy streaming read of the mapped index and pinned "
                             "host-to-device hipMemcpy",
                "unit": "GB/s", "frac": round(step_gbs / peak, 4), "traffic": None,
                "alg_bytes_per_step": alg_bytes,
                # each stage's link rate on the bytes it reads: the sample
                # stage its runs, the filter every other block
                "sample_stage_GBs": round(alg_bytes * fs / (thr_ms * 1e-3) / 1e9, 2),
                "filtered_scan_GBs": round(alg_bytes * (1 - fs) / (scan_ms * 1e-3) / 1e9, 2),
                "link_probes_GBs": link}
    res = {
        "metric": METRIC, "value": round(ms_step, 4), "unit": "ms/step", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": w.name, "pairs": w.P, "n": w.n, "G": w.G, "D": w.D, "budget": budget,
                   "mode": ["waterfill", "topr", "uniform"][a.mode], "k": w.k, "keys": w.key_dtype,
                   "index": "host-mapped pinned" if host else "hbm",
                   "basis": "klt" if w.rotated else "raw",
                   "scan": "int8-mfma fixed-point: int8 coefficient digits x int8 codes, exact int32/int64 "
                           "sums, one float32 rounding per score"},
        "gpu_ms_per_step": round(gpu_ms, 4), "plan_ms": round(plan_ms, 4),
        "threshold_ms": round(thr_ms, 4), "scan_ms": round(scan_ms, 4), "select_ms": round(sel_ms, 4),
        "materialised_ms": round(mat_total, 4), "materialised_scan_ms": round(mat_scan, 4),
        "materialised_same_result": same,
        "keys_per_s": round(w.P * w.n / (ms_step * 1e-3), 1),
        "bits_per_token": round(bits_tok, 2), "active_channels_mean": round(float(act.double().mean()), 2),
        "roofline": roof,
        "calibration": calib,
    }
    if w.P > w.kv_heads:
        res["per_layer"] = per_layer_probe(F, w, planes, scales, q, s2, rot, budget, a.mode, dev)
        log(f"per-layer calls: {res['per_layer']}")
    if host is not None:
        for h in host:
            h.free()
    if w.n >= (1 << 17):
        res["fetch"] = fetch_probe(F, w, out, dev)
        log(f"winner-row fetch: {res['fetch']}")
    if host is None:
        res["append"] = append_probe(F, w, planes, scales, dev)
        log(f"append (repack the last block of every pair): {res['append']}")
    if a.cpu_baseline:
        threads = a.cpu_threads or min(16, cpu_info()["affinity_cpus"])
        res["cpu_baseline"] = cpu_baseline(w, q_np, budget, a.mode, a.cpu_pairs, threads)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
