"""Benchmark: paged decode KV GB/s (and prefill TFLOP/s) on one MI355X.

A step is one decode pass over the batch of 8 streams x 65,536 positions
(24 q / 4 kv heads, head_dim 256, bf16 KV, 4,096-key splits): write_kv of
each stream's newest row, the split-K partial kernel, and the merge.
`value` is KV bytes read per step / step time.  Prefill (4,096 causal rows
after a 28,672 prefix), the fp8 mixed paged/slab batch and the 16-stream fp8
verify batch are measured too and reported under "secondary".

Kernel durations come from HIP events recorded on the stream the kernels
are launched on.  HBM traffic per launch is read from the committed
rocprofv3 counter summary when it was taken on the current kernel source,
else reported as null.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--no-secondary] [--profile decode|prefill|copy|verify]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SOURCES = ["paged_kv_cache_addressing_amd/csrc/decode.hip",
                  "paged_kv_cache_addressing_amd/csrc/prefill.hip",
                  "paged_kv_cache_addressing_amd/csrc/verify.hip",
                  "paged_kv_cache_addressing_amd/csrc/pa_device.hpp",
                  "paged_kv_cache_addressing_amd/csrc/pa_kargs.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest(paths=KERNEL_SOURCES) -> str:
    """Digest of the kernel sources' code: comments and blank space are
    dropped, so documentation edits do not retire the committed counters."""
    import re
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def kv_bytes(wl) -> int:
    """Algorithmic KV bytes a decode pass reads: every visible key's K and V
    row for every kv head (2 * Hkv * D * element size per position)."""
    esz = 2 if wl.kv_dtype == "bf16" else 1
    per_pos = 2 * wl.n_kv_heads * wl.head_dim * esz
    return sum(st.first_pos + st.n_rows for st in wl.streams) * per_pos


def kv_bytes_stream(wl, s) -> int:
    """KV bytes one decode pass reads for stream s."""
    esz = 2 if wl.kv_dtype == "bf16" else 1
    st = wl.streams[s]
    return (st.first_pos + st.n_rows) * 2 * wl.n_kv_heads * wl.head_dim * esz


def attn_flops(wl) -> int:
    """4 * D * Hq flop per visible (row, key) pair (QK^T and PV)."""
    pairs = 0
    for st in wl.streams:
        # rows at positions p = first_pos .. first_pos+n_rows-1 see p + 1 keys
        pairs += st.n_rows * (st.first_pos + 1) + st.n_rows * (st.n_rows - 1) // 2
    return 4 * wl.head_dim * wl.n_q_heads * pairs


_HIP = None


def _hip():
    """The HIP runtime torch loaded (the library's kernels run on it too),
    with the event calls the timers use."""
    global _HIP
    if _HIP is None:
        import ctypes as C

        import torch
        torch.cuda.init()
        path = next(line.split()[-1] for line in open("/proc/self/maps")
                    if "libamdhip64" in line)
        h = C.CDLL(path)
        h.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        h.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        h.hipEventDestroy.argtypes = [C.c_void_p]
        _HIP = h
    return _HIP


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class EventTimer:
    """Accumulates HIP-event durations of work enqueued on the current stream.

    The events are created with hipEventDisableSystemFence, HIP's flag for
    events used only for timing: recording one then skips the system-scope
    cache write-back and invalidate, which would otherwise add ~3 us to every
    timed decode step (measured: 0.3303 ms per config-2 step with no events,
    0.3326 with these around each partial launch, 0.3359 with torch's)."""

    def __init__(self, n: int = 0):
        """n: event pairs to create now, so that creating them (a host call
        that is slow next to a record) stays out of the timed steps."""
        self.pairs = []
        self.pool = [self._new() for _ in range(2 * n)]

    @staticmethod
    def _new():
        import ctypes as C
        e = C.c_void_p()
        if _hip().hipEventCreateWithFlags(C.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e

    def _event(self):
        return self.pool.pop() if self.pool else self._new()

    def _record(self, e):
        import ctypes as C

        import torch
        st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
        if _hip().hipEventRecord(e, st) != 0:
            raise RuntimeError("hipEventRecord failed")

    def __enter__(self):
        self.s, self.e = self._event(), self._event()
        self._record(self.s)
        return self

    def __exit__(self, *exc):
        self._record(self.e)
        self.pairs.append((self.s, self.e))

    def times_ms(self) -> list:
        import ctypes as C

        import torch
        torch.cuda.synchronize()
        if not hasattr(self, "_ms"):
            self._ms = []
        for s, e in self.pairs:
            ms = C.c_float()
            if _hip().hipEventElapsedTime(C.byref(ms), s, e) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            self._ms.append(ms.value)
            _hip().hipEventDestroy(s)
            _hip().hipEventDestroy(e)
        self.pairs = []
        return list(self._ms)

    def __del__(self):
        if _HIP is not None:
            for e in getattr(self, "pool", []):
                _HIP.hipEventDestroy(e)

    def mean_ms(self) -> float:
        ts = self.times_ms()
        return sum(ts) / len(ts)

    def stats(self) -> dict:
        """Mean, median and min of the recorded durations (ms)."""
        ts = sorted(self.times_ms())
        n = len(ts)
        med = ts[n // 2] if n % 2 else 0.5 * (ts[n // 2 - 1] + ts[n // 2])
        return {"mean": round(sum(ts) / n, 5), "median": round(med, 5), "min": round(ts[0], 5),
                "n": n}


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None if the
    summary is missing or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except OSError:
        return None
    if t.get("kernel_source_digest") != source_digest():
        return None
    ent = t.get("kernels", {}).get(kernel)
    if not ent or ent.get("workload") != workload:
        return None
    return ent.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------- decode

def setup_decode(wl):
    import torch

    import paged_kv_cache_addressing_amd as pa
    from paged_kv_cache_addressing_amd.resident import upload
    res = upload(wl)
    ws = pa.decode_workspace(res.cache, res.streams, wl.n_q_heads, wl.split_keys)
    out = torch.empty_like(res.q)
    # the step's store: each stream's newest row (position ctx-1)
    new_k = torch.stack([wl.k_rows[s][-1] for s in range(len(wl.streams))]).cuda()
    new_v = torch.stack([wl.v_rows[s][-1] for s in range(len(wl.streams))]).cuda()
    store = []
    for s, st in enumerate(res.streams):
        store.append(pa.Stream(st.ctx_len, 1, s, st.ctx_len - 1, page_table=st.page_table,
                               k_slab=st.k_slab, v_slab=st.v_slab, slab_cap=st.slab_cap,
                               layout=st.layout))
    return res, ws, out, new_k, new_v, store


EVENT_EVERY = 4  # timed steps per event-bracketed partial launch


def run_decode(wl, steps, warmup, with_store=True, aa=False):
    """Time `steps` decode steps (store, partials, merge).  Inside the timed
    region the partial kernel (the roofline kernel) is bracketed by events on
    every EVENT_EVERY-th step, and its average duration is taken over those
    launches: even fence-free event records cost ~2.3 us of a 330 us step,
    and the sample keeps most of that out of the timed steps.  The store and
    merge durations come from a short pass after the timed region."""
    import torch

    import paged_kv_cache_addressing_amd as pa
    res, ws, out, nk, nv, store = setup_decode(wl)
    n_after = max(3, min(steps, 10))
    n_ev = (steps + EVENT_EVERY - 1) // EVENT_EVERY
    t_store, t_part, t_merge = EventTimer(n_after), EventTimer(n_ev), EventTimer(n_after)

    def partials():
        pa.paged_attn_decode_partials(res.cache, res.streams, res.q, ws,
                                      sm_scale=res.sm_scale, split_keys=res.split_keys)

    def merge():
        pa.paged_attn_decode_merge(res.cache, res.streams, out, ws, split_keys=res.split_keys)

    def step(timer=None, i=0):
        if with_store:
            pa.write_kv(res.cache, store, nk, nv)
        if timer is not None:
            if i % EVENT_EVERY == 0:
                with timer:
                    partials()
            else:
                partials()
            merge()
        else:
            pa.paged_attn_decode(res.cache, res.streams, res.q, out=out, sm_scale=res.sm_scale,
                                 split_keys=res.split_keys, workspace=ws)

    def timed_steps(timer):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(timer, i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    for _ in range(warmup):
        step()
    wall_ms = timed_steps(t_part)
    # per-kernel breakdown, outside the timed region
    for _ in range(max(3, min(steps, 10))):
        if with_store:
            with t_store:
                pa.write_kv(res.cache, store, nk, nv)
        partials()
        with t_merge:
            merge()
    # A/A: a second arm of the same timed steps, to show the run-to-run spread
    t_arm2 = EventTimer(n_ev if aa else 0)
    wall2_ms = timed_steps(t_arm2) if aa else None
    r = {"ms_per_step": wall_ms, "partial_ms": t_part.mean_ms(), "merge_ms": t_merge.mean_ms(),
         "partial_stats": t_part.stats()}
    if aa:
        r["hbm_probe"] = probe_abba(partials, kv_bytes(wl))
    if aa:
        a1, a2 = r["partial_ms"], t_arm2.mean_ms()
        r["aa"] = {"arm1_partial_ms": round(a1, 5), "arm2_partial_ms": round(a2, 5),
                   "spread": round(abs(a1 - a2) / a1, 5),
                   "arm1_ms_per_step": round(wall_ms, 5), "arm2_ms_per_step": round(wall2_ms, 5),
                   "step_spread": round(abs(wall_ms - wall2_ms) / wall_ms, 5)}
    if with_store:
        r["store_ms"] = t_store.mean_ms()
    return r, res, out


SETTLE_WARMUP = 100  # untimed steps before the secondary decode workloads are timed
PROBE_BYTES = 8 << 30  # larger runs read faster: 6.25 / 6.21 / 6.44 / 6.63 TB/s at 1 / 2 / 4 / 8 GiB


def probe_abba(arm_a, a_bytes: int, launches: int = 10, rounds: int = 3) -> dict:
    """ABBA rounds of arm A (the decode partial kernel) against arm B, the
    library's plain streaming read of an 8 GiB buffer (pa_hbm_read_probe):
    the device's achievable read rate, measured between the same launches."""
    import torch

    import paged_kv_cache_addressing_amd as pa
    buf = torch.zeros(PROBE_BYTES, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ta, tb = EventTimer(2 * rounds * launches), EventTimer(2 * rounds * launches)

    def arm(t, f):
        for _ in range(launches):
            with t:
                f()

    def probe():
        pa.hbm_read_probe(buf, sink)
    for _ in range(3):
        probe()
    for _ in range(rounds):
        arm(ta, arm_a)
        arm(tb, probe)
        arm(tb, probe)
        arm(ta, arm_a)
    sa, sb = ta.stats(), tb.stats()
    del buf
    probe_gbs = PROBE_BYTES / (sb["median"] * 1e-3) / 1e9
    a_gbs = a_bytes / (sa["median"] * 1e-3) / 1e9
    return {"probe": "pa_hbm_read_probe over 8 GiB (one contiguous run per workgroup, "
                     "1,024 x 512 threads, 32 KiB steps, 4 steps of nontemporal loads in "
                     "flight)", "rounds": f"ABBA x{rounds}, {launches} launches an arm",
            "probe_gbs_median": round(probe_gbs, 1),
            "probe_gbs_max": round(PROBE_BYTES / (sb["min"] * 1e-3) / 1e9, 1),
            "partial_gbs_median": round(a_gbs, 1),
            "partial_over_probe": round(a_gbs / probe_gbs, 4)}


# ----------------------------------------------------------------------------- prefill

def run_prefill(wl, steps, warmup):
    import torch

    import paged_kv_cache_addressing_amd as pa
    from paged_kv_cache_addressing_amd.resident import upload
    res = upload(wl)
    out = torch.empty_like(res.q)
    t = EventTimer(steps)
    for _ in range(warmup):
        pa.paged_attn_prefill(res.cache, res.streams, res.q, out=out, sm_scale=res.sm_scale)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        with t:
            pa.paged_attn_prefill(res.cache, res.streams, res.q, out=out, sm_scale=res.sm_scale)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    return {"ms_per_step": wall_ms, "prefill_ms": t.mean_ms(), "prefill_stats": t.stats()}


def run_latency(wl, calls=200, warmup=20):
    """Latency of one decode call (partials + merge) on a small workload: HIP
    events around each call, median and min over `calls` calls."""
    import torch

    import paged_kv_cache_addressing_amd as pa
    from paged_kv_cache_addressing_amd.resident import upload
    res = upload(wl)
    ws = pa.decode_workspace(res.cache, res.streams, wl.n_q_heads, wl.split_keys)
    out = torch.empty_like(res.q)

    def call():
        pa.paged_attn_decode(res.cache, res.streams, res.q, out=out, sm_scale=res.sm_scale,
                             split_keys=res.split_keys, workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t = EventTimer(calls)
    for _ in range(calls):
        with t:
            call()
    st = t.stats()
    return {"workload": wl.name, "call": "paged_attn_decode (partials + merge)",
            "median_us": round(st["median"] * 1e3, 2), "min_us": round(st["min"] * 1e3, 2),
            "mean_us": round(st["mean"] * 1e3, 2), "calls": calls}


# ----------------------------------------------------------------------------- oracle baseline

def cpu_baseline(wl, min_s: float = 10.0):
    """Time the float64 oracle on the host over whole streams of the same
    workload, cycling over the batch until at least min_s seconds of work;
    returns KV GB/s."""
    import numpy as np

    import torch

    import oracle

    def bits16(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    threads = oracle_threads()
    hkv, d = wl.n_kv_heads, wl.head_dim
    ps = hkv * 256 * d
    kp = np.zeros((wl.n_pages, hkv, 256, d), np.uint16)
    vp = np.zeros_like(kp)
    for s, st in enumerate(wl.streams):
        oracle.store(kp, vp, oracle.DTYPE_BF16, bits16(wl.k_rows[s]), bits16(wl.v_rows[s]), 0,
                     page_table=st.pages, page_stride=ps)
    done_bytes, spent, n_calls = 0, 0.0, 0
    while spent < min_s:
        for s, st in enumerate(wl.streams):
            q = bits16(wl.q[st.row_offset:st.row_offset + st.n_rows])
            t0 = time.perf_counter()
            oracle.attention(kp, vp, oracle.DTYPE_BF16, q, st.first_pos, hkv, st.ctx_len,
                             page_table=st.pages, page_stride=ps, sm_scale=wl.sm_scale,
                             n_threads=threads)
            spent += time.perf_counter() - t0
            done_bytes += (st.first_pos + st.n_rows) * 2 * hkv * d * 2
            n_calls += 1
        log(f"oracle: {n_calls} stream passes, {spent:.1f}s so far")
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n_calls} stream passes over the decode batch's 8 streams (whole "
                      f"65,536-position context, all 24 q heads, float64 gather+softmax, "
                      f"{threads} threads over (row, q head)), {spent:.1f} s",
            "host": host_cpus()}


def oracle_threads() -> int:
    """Threads the oracle runs on: the process's CPUs, at most 16 (one GPU's
    share of an eight-GPU host)."""
    return min(16, len(os.sched_getaffinity(0)))


def host_cpus() -> dict:
    """The host's processor counts, apart from the threads the oracle uses:
    logical CPUs (what nproc and std::thread::hardware_concurrency report)
    and the CPUs this process may run on."""
    return {"logical_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "oracle_threads": oracle_threads(),
            "cap": "the oracle uses at most 16 threads, one GPU's share of the host"}


def oracle_stream_time(wl, s, rows, threads, min_s):
    """Seconds per oracle call over rows `rows` of stream s (a contiguous copy of
    the stream's cache, built once), repeated until min_s seconds are spent."""
    import numpy as np

    import torch

    import oracle

    def bits16(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    st = wl.streams[s]
    dt = oracle.DTYPE_BF16 if wl.kv_dtype == "bf16" else oracle.DTYPE_E4M3
    npd = np.uint16 if wl.kv_dtype == "bf16" else np.uint8
    k = np.zeros((st.ctx_len, wl.n_kv_heads, wl.head_dim), npd)
    v = np.zeros_like(k)
    oracle.store(k, v, dt, bits16(wl.k_rows[s]), bits16(wl.v_rows[s]), 0, k_scale=wl.k_scale,
                 v_scale=wl.v_scale, n_threads=threads)
    q = bits16(wl.q[st.row_offset:st.row_offset + st.n_rows])
    sel = np.array(rows, np.int32)
    n, spent = 0, 0.0
    while n == 0 or spent < min_s:
        t0 = time.perf_counter()
        oracle.attention(k, v, dt, q, st.first_pos, wl.n_kv_heads, st.ctx_len, rows=sel,
                         sm_scale=wl.sm_scale, k_scale=wl.k_scale, v_scale=wl.v_scale,
                         n_threads=threads)
        spent += time.perf_counter() - t0
        n += 1
    return spent / n, n, spent


def cpu_baseline_others(wls: dict, min_s: float = 2.0):
    """Oracle timings on the other workloads (`wls`: config name -> workload,
    built by the GPU legs), each a bounded sample."""
    import workloads
    out = {}
    thr = oracle_threads()
    for name in ("config1", "config2"):
        wl = wls.get(name) or getattr(workloads, name)()
        st = wl.streams[0]
        t, n, spent = oracle_stream_time(wl, 0, [0], 1, min_s)
        nb = kv_bytes_stream(wl, 0)
        out[f"{name}_1thread"] = {
            "value": round(nb / t / 1e9, 4), "unit": "GB/s", "cores": 1,
            "latency_ms": round(t * 1e3, 3),
            "sample": f"stream 0 of {wl.name} (1 row, {st.ctx_len} keys, all {wl.n_q_heads} q "
                      f"heads), {n} calls in {spent:.1f} s on 1 thread"}
        log(f"oracle {name} 1 thread: {out[name + '_1thread']['value']} GB/s")
    wl = wls.get("config4") or workloads.config4()
    st = wl.streams[0]
    rows = [0, 1365, 2730, 4095]
    t, n, spent = oracle_stream_time(wl, 0, rows, thr, min_s)
    pairs = sum(st.first_pos + r + 1 for r in rows)
    fl = 4 * wl.head_dim * wl.n_q_heads * pairs
    out["config4_sampled"] = {
        "value": round(fl / t / 1e12, 6), "unit": "TFLOP/s", "cores": thr,
        "projected_full_s": round(t * attn_flops(wl) / fl, 1),
        "sample": f"rows {rows} of the 4,096-row prefill ({pairs} row-key pairs, all 24 q heads), "
                  f"{n} calls in {spent:.1f} s; projected_full_s scales by the workload's flop"}
    log(f"oracle config4 sampled: {out['config4_sampled']['value']} TFLOP/s")
    wl = wls.get("config5") or workloads.config5()
    st = wl.streams[0]
    rows = [0, 15]
    t, n, spent = oracle_stream_time(wl, 0, rows, thr, min_s)
    total_rows = sum(x.n_rows for x in wl.streams)
    per_row = t / len(rows)
    # every row re-reads its stream's keys in the oracle: a row of stream 0
    # stands for a row of average context
    mean_ctx = sum(x.ctx_len for x in wl.streams) / len(wl.streams)
    proj = per_row * total_rows * mean_ctx / st.ctx_len
    out["config5_sampled"] = {
        "value": round(kv_bytes(wl) / proj / 1e9, 4), "unit": "GB/s", "cores": thr,
        "projected_full_s": round(proj, 1),
        "sample": f"rows {rows} of stream 0 ({st.ctx_len} keys, fp8, all 24 q heads), {n} calls "
                  f"in {spent:.1f} s; scaled to all {total_rows} rows at the batch's mean context"}
    log(f"oracle config5 sampled: {out['config5_sampled']['value']} GB/s")
    return out


# ----------------------------------------------------------------------------- main

def copy_calibration():
    """A plain 1 GiB device copy: reads and writes exactly 2^30 bytes."""
    import torch
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--profile", choices=["decode", "prefill", "copy", "verify", "fp8"])
    ap.add_argument("--only", choices=["prefill", "verify", "fp8"],
                    help="time one secondary workload only and print its record")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads
    torch.cuda.set_device(0)

    if args.only == "prefill":
        wl4 = workloads.config4()
        p = run_prefill(wl4, args.steps, args.warmup)
        fl = attn_flops(wl4)
        tf = fl / (p["prefill_ms"] * 1e-3) / 1e12
        print(json.dumps({"prefill_ms": round(p["prefill_ms"], 4), "tflops": round(tf, 2),
                          "frac": round(tf / BF16_PEAK_TFLOPS, 4)}), flush=True)
        return

    if args.only in ("verify", "fp8"):
        w = workloads.config5() if args.only == "verify" else workloads.config3()
        rr, _, _ = run_decode(w, args.steps, args.warmup, with_store=args.only == "fp8")
        nb, fl = kv_bytes(w), attn_flops(w)
        print(json.dumps({"workload": w.name, "partial_ms": round(rr["partial_ms"], 5),
                          "merge_ms": round(rr["merge_ms"], 5),
                          "frac_hbm_partial": round(nb / (rr["partial_ms"] * 1e-3) / 1e9 /
                                                    HBM_PEAK_GBS, 4),
                          "tflops_partial": round(fl / (rr["partial_ms"] * 1e-3) / 1e12, 2)}),
              flush=True)
        return

    if args.profile:  # a short run for rocprofv3: the named kernels only
        if args.profile == "copy":
            copy_calibration()
        elif args.profile == "decode":
            run_decode(workloads.config2(), args.steps, args.warmup)
        elif args.profile == "fp8":
            run_decode(workloads.config3(), args.steps, args.warmup)
        elif args.profile == "verify":
            run_decode(workloads.config5(), args.steps, args.warmup, with_store=False)
        else:
            run_prefill(workloads.config4(), args.steps, args.warmup)
        log(f"profile run {args.profile} done")
        return

    wl = workloads.config2()
    log(f"decode {wl.name}: uploading")
    r, res, out = run_decode(wl, args.steps, args.warmup, aa=True)
    nbytes = kv_bytes(wl)
    value = nbytes / (r["ms_per_step"] * 1e-3) / 1e9
    achieved = nbytes / (r["partial_ms"] * 1e-3) / 1e9
    log(f"decode: {r}")
    line = {
        "metric": "paged decode KV GB/s (% HBM peak); prefill attention TFLOP/s (% MFMA peak)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, shuffled 256-position pages)",
        "config": {"workload": "decode batch: 8 streams x 1 row at context 65,536, 24 q / 4 kv "
                               "heads, head_dim 256, bf16 KV in 256-position pages shuffled in "
                               "one 2,048-page pool, 4,096-key splits + LSE merge",
                   "streams": 8, "context": 65536, "q_heads": 24, "kv_heads": 4,
                   "head_dim": 256, "kv_dtype": "bf16", "split_keys": 4096,
                   "kv_bytes_per_step": nbytes,
                   "step": "write_kv (1 row/stream) + decode partials + merge"},
        "roofline": {"bound": "hbm", "kernel": "decode_partial_kernel<bf16,256>",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for("decode_partial_kernel<bf16,256>", "config2"),
                     "kernel_ms": round(r["partial_ms"], 5),
                     "algorithmic_bytes": nbytes},
        "kernel_ms": {k: round(v, 5) for k, v in r.items() if isinstance(v, float)},
        "partial_ms_stats": r["partial_stats"],
        "aa": r["aa"],
        "hbm_probe": r["hbm_probe"],
    }
    del res, out
    torch.cuda.empty_cache()

    kept = {"config2": wl}  # host-side workloads reused by the oracle timings
    if not args.no_secondary:
        sec = {}
        wl4 = workloads.config4()
        kept["config4"] = wl4
        log(f"prefill {wl4.name}")
        # the GPU idles while the workload is generated on the host; ten
        # untimed launches (~30 ms) let the clock settle before timing
        p = run_prefill(wl4, max(10, args.steps // 2), 10)
        fl = attn_flops(wl4)
        tf = fl / (p["prefill_ms"] * 1e-3) / 1e12
        sec["prefill"] = {"workload": "1 stream, 4,096 causal rows after a 28,672-position "
                                      "paged prefix, 24/4 heads, D 256, bf16",
                          "kernel": "prefill_kernel<bf16,256>", "kernel_ms": round(p["prefill_ms"], 4),
                          "flop": fl, "tflops": round(tf, 2), "peak_tflops": BF16_PEAK_TFLOPS,
                          "frac": round(tf / BF16_PEAK_TFLOPS, 4), "bound": "mfma",
                          "kernel_ms_stats": p["prefill_stats"],
                          "traffic": traffic_for("prefill_kernel<bf16,256>", "config4")}
        for name, fn, store in (("decode_fp8_mixed", workloads.config3, True),
                                ("verify_fp8", workloads.config5, False)):
            w = fn()
            log(f"{name} {w.name}")
            # The clock needs tens of launches to settle after the host-side
            # workload generation: launch by launch, the verify batch ran
            # 0.51 ms cold, 0.64-0.70 ms at launches 4-10 and 0.50-0.51 ms
            # from about the 50th on.  The timed launches follow SETTLE_WARMUP
            # untimed steps.
            rr, res, out = run_decode(w, args.steps, max(args.warmup, SETTLE_WARMUP),
                                      with_store=store)
            nb = kv_bytes(w)
            fl = attn_flops(w)
            sec[name] = {"workload": w.name, "kv_bytes": nb,
                         "partial_ms": round(rr["partial_ms"], 5),
                         "merge_ms": round(rr["merge_ms"], 5),
                         "kv_gbs_partial": round(nb / (rr["partial_ms"] * 1e-3) / 1e9, 2),
                         "kv_gbs_step": round(nb / (rr["ms_per_step"] * 1e-3) / 1e9, 2),
                         "frac_hbm_partial": round(nb / (rr["partial_ms"] * 1e-3) / 1e9 /
                                                   HBM_PEAK_GBS, 4),
                         "frac_hbm_partial_merge": round(nb / ((rr["partial_ms"] + rr["merge_ms"])
                                                               * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "tflops_partial": round(fl / (rr["partial_ms"] * 1e-3) / 1e12, 2),
                         "partial_ms_stats": rr["partial_stats"]}
            if name == "verify_fp8":
                sec[name]["kernel"] = "verify_kernel<256>"
                sec[name]["traffic"] = traffic_for("verify_kernel<256>", "config5")
            else:
                sec[name]["kernel"] = "decode_partial_kernel<fp8,256>"
                sec[name]["traffic"] = traffic_for("decode_partial_kernel<fp8,256>", "config3")
            if name == "verify_fp8":
                kept["config5"] = w
            del w, res, out
            torch.cuda.empty_cache()
        w1 = workloads.config1()
        log(f"latency {w1.name}")
        sec["config1_latency"] = run_latency(w1)
        kept["config1"] = w1
        line["secondary"] = sec

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(wl)
        line["cpu_baseline"]["others"] = cpu_baseline_others(kept)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
