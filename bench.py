#!/usr/bin/env python3
"""SGMV benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode7b]
    python bench.py --sweep decode|prefill     (time per call against batch size or
                                                 prompt length, one JSON line)
    python bench.py --layer                    (backbone GEMM alone vs the LoRA layer)
    python bench.py --load                     (adapter uploads, host to HBM)

One step is one batch through the whole SGMV path, with every input resident in HBM:
  * batches of <= 64 tokens (the decode workloads) take the one-launch path,
    sgmv_lora_add_pool: the segment metadata (stable sort of the batch's adapter ids),
    the shrink and the expand all run in one kernel; the K timed steps are captured in
    one HIP graph and replayed once, as a serving loop runs its decode steps;
  * larger batches (prefill, mixed) build the segment metadata with libsgmv's host
    builder, upload it with one host-to-device copy from pinned memory and call
    sgmv_lora_add (MFMA tiles for segments of 16+ rows).
Every step uses a different slot of x / y buffers, adapter ids and adapters, the slots
together spanning more than 1 GiB, so each step reads its operands from HBM and not from
the 256 MB Infinity Cache (cache-cold by construction).

Printed: one JSON line with the whole-step throughput (algorithmic bytes per step over
the wall time of K steps), the average duration of the SGMV kernel(s) of one call from
HIP events on their stream (the roofline figure: over the timed graph replay on the
one-launch path, over a graph of the same calls on the table path), and the fp64 CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from workloads import synth  # noqa: E402

METRIC = "SGMV shrink+expand us/call and HBM GB/s, h=4096 r=16 bs=32 distinct adapters"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16/fp16 MFMA, AMD published figure
ROTATION_BYTES = 1 << 30       # operand slots cycled per pass (> 2x the 256 MB MALL)
FLUSH_BYTES = 1 << 30          # read before every timed replay (4x the 256 MB MALL)
_CSRC = os.path.join(ROOT, "adapter_gemv_amd", "csrc")
KERNEL_SRCS = [os.path.join(_CSRC, f)
               for f in ("sgmv_checks.h", "sgmv_device.h", "sgmv_kernels.hip", "sgmv_decode.hip")]
# the sources each kernel's code comes from (a counter summary stays valid while they do)
KERNEL_SRCS_OF = {
    "lora_add_pool_kernel": ("sgmv_checks.h", "sgmv_device.h", "sgmv_decode.hip"),
    "lora_add_ids_kernel": ("sgmv_checks.h", "sgmv_device.h", "sgmv_decode.hip"),
    "sgmv_lora_add": ("sgmv_checks.h", "sgmv_device.h", "sgmv_kernels.hip"),
}


def workload_problem(name: str):
    """The named workload; also decode7b_bs<N> (N = 1..64 tokens) and
    prefill13b_<proj>_len<L> (4 requests of L tokens) for the batch sweeps."""
    table = dict(synth.all_workloads())
    if name in table:
        return table[name]()
    if name.startswith("decode7b_bs") and name[11:].isdigit():
        return synth.decode7b_bs(int(name[11:]))
    for proj in synth.PREFILL13B_SHAPES:
        pre = f"prefill13b_{proj}_len"
        if name.startswith(pre) and name[len(pre):].isdigit():
            return synth.prefill13b_len(int(name[len(pre):]), proj)
    raise SystemExit(f"unknown workload {name!r}; choose from {sorted(table)}, "
                     "decode7b_bs<N>, prefill13b_<proj>_len<L>")


def algorithmic_bytes(p) -> int:
    """x read once, y read and written once, each distinct adapter's A and B read once."""
    e = 2
    D = p.distinct_adapters()
    return e * (p.n * p.h_in + 2 * p.n * p.h_out + D * p.r * (p.h_in + p.h_out))


def algorithmic_flops(p) -> int:
    return 2 * p.n * p.r * (p.h_in + p.h_out)


def kernel_source_hash(kernel: str = "") -> str:
    """First 16 hex digits of the SHA-256 of the kernel sources: all of them, or those that
    `kernel` (a key of KERNEL_SRCS_OF) is built from."""
    paths = [os.path.join(_CSRC, f) for f in KERNEL_SRCS_OF[kernel]] if kernel else KERNEL_SRCS
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# --------------------------------------------------------------------------------------
# CPU oracle baseline
# --------------------------------------------------------------------------------------
def cpu_baseline_1thread(p, budget_s: float) -> dict:
    """The same oracle timing with the BLAS pool limited to one thread."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"):
        out = cpu_baseline(p, budget_s)
    return out


def cpu_baseline(p, budget_s: float = 12.0, runs: int = 5):
    """The fp64 oracle on the same workload, its inputs decoded to float64 before the timed
    region (x, y and every adapter the batch uses), so that what is timed is the oracle's
    per-adapter products (x[rows] @ A) @ B and the y update: `runs` runs of repeated full
    calls for budget_s / runs seconds each, the median of the runs' per-call times."""
    import oracle
    from threadpoolctl import threadpool_info
    X, Y = oracle.decode(p.x, p.dtype), oracle.decode(p.y, p.dtype)
    A64, B64 = oracle.DecodedPool(p.A, p.dtype), oracle.DecodedPool(p.B, p.dtype)
    for a in np.unique(p.ids):
        A64[int(a)], B64[int(a)]
    oracle.lora_add_f64(Y, X, p.ids, A64, B64, p.scale)      # untimed first call
    per_run, calls = [], 0
    for _ in range(runs):
        reps = 0
        t0 = time.perf_counter()
        while True:
            oracle.lora_add_f64(Y, X, p.ids, A64, B64, p.scale)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s / runs:
                break
        per_run.append(el / reps)
        calls += reps
    per_call = float(np.median(per_run))
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    cores = int(blas[0].get("num_threads", 1)) if blas else 1
    lib = (f"{blas[0].get('internal_api')} {blas[0].get('version')}" if blas else "none")
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {
        "value": round(algorithmic_bytes(p) / per_call / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{p.name}, full calls, inputs decoded to fp64 before timing; median of "
                  f"{runs} runs ({calls} calls in {budget_s:.0f} s): {per_call * 1e3:.3f} ms/call, "
                  f"{algorithmic_flops(p) / per_call / 1e9:.2f} GFLOP/s; numpy fp64 on {lib}, "
                  f"BLAS threads {cores}, os.cpu_count() {os.cpu_count()}, affinity {affinity}",
        "us_per_call": round(per_call * 1e6, 2),
        "runs_us": [round(t * 1e6, 2) for t in per_run],
    }


# --------------------------------------------------------------------------------------
# GPU setup
# --------------------------------------------------------------------------------------
class Rig:
    """Rotation slots of x, y, adapter ids and adapters on the device."""

    def __init__(self, p, device, seed=1234):
        import torch
        from adapter_gemv_amd import sgmv
        self.p = p
        self.device = device
        per_slot = algorithmic_bytes(p)
        self.slots = max(2, min(256, -(-ROTATION_BYTES // per_slot)))
        S_, P = self.slots, p.n_adapters
        tdt = torch.float16 if p.dtype == "f16" else torch.bfloat16
        g = torch.Generator(device=device)
        g.manual_seed(seed)

        def randn(shape, std):
            t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
            return (t * std).to(tdt)

        self.x = randn((S_, p.n, p.h_in), 1.0)
        self.y = randn((S_, p.n, p.h_out), 1.0)
        self.A = randn((S_ * P, p.r, p.h_in), 1.0 / np.sqrt(p.h_in))
        self.B = randn((S_ * P, p.h_out, p.r), 1.0 / np.sqrt(p.r))
        # slot 0 holds the seeded problem itself (checked against the oracle)
        self.x[0].copy_(sgmv.as_tensor(p.x, p.dtype, device))
        self.y[0].copy_(sgmv.as_tensor(p.y, p.dtype, device))
        self.A[:P].copy_(sgmv.as_tensor(p.A, p.dtype, device))
        self.B[:P].copy_(sgmv.as_tensor(p.B, p.dtype, device))
        self.y0 = self.y[0].clone()
        self.n_pool = S_ * P
        # slot k's batch uses adapters [k*P, (k+1)*P) of the big pool
        self.ids = [np.ascontiguousarray(p.ids + k * P, dtype=np.int32) for k in range(S_)]
        self.ids_dev = torch.as_tensor(np.stack(self.ids), device=device)
        self.ws = sgmv.make_workspace(p.n, p.h_in, p.r, device)
        self.dtype_code = sgmv.dtype_code(self.x)
        self.ld_x, self.ld_y = p.h_in, p.h_out
        self.pool_path = p.n <= sgmv.DECODE_MAX_TOKENS
        self.host_ids = False
        # table path: metadata staging ring (pinned host -> device)
        self.A_bases = sgmv.adapter_bases(self.A)
        self.B_bases = sgmv.adapter_bases(self.B)
        self.ring = 64
        S_max = min(p.n, self.n_pool)
        self.meta_bytes = 16 * S_max + 4 * (S_max + 1) + 4 * p.n + 64
        self.pinned = torch.empty((self.ring, self.meta_bytes), dtype=torch.uint8, pin_memory=True)
        self.pinned_np = self.pinned.numpy()
        self.dev_meta = torch.empty((self.ring, self.meta_bytes), dtype=torch.uint8, device=device)
        self.ring_evt = [None] * self.ring

    def step(self, k: int, ev=None):
        """One step on slot k.  ``ev`` = (start, end) events bracket the SGMV call."""
        if self.host_ids:
            return self.step_host_ids(k, ev)
        return self.step_pool(k, ev) if self.pool_path else self.step_table(k, ev)

    def step_host_ids(self, k: int, ev=None):
        """Shrink and expand in one launch, the batch's adapter ids (host memory) carried
        in the kernel arguments."""
        import torch
        from adapter_gemv_amd import sgmv
        p = self.p
        slot = k % self.slots
        stream = torch.cuda.current_stream()
        if ev is not None:
            ev[0].record(stream)
        st = sgmv.sgmv_lora_add_host_ids(
            stream.cuda_stream, self.dtype_code, self.y[slot].data_ptr(), self.ld_y,
            self.x[slot].data_ptr(), self.ld_x, self.ids[slot].ctypes.data, p.n,
            self.A.data_ptr(), self.A.stride(0), self.B.data_ptr(), self.B.stride(0),
            self.n_pool, p.h_in, p.h_out, p.r, p.scale, self.ws.data_ptr(), self.ws.numel())
        if ev is not None:
            ev[1].record(stream)
        if st != 0:
            raise RuntimeError(f"sgmv_lora_add_host_ids failed: {sgmv.sgmv_status_string(st)}")

    def step_pool(self, k: int, ev=None):
        """Segment metadata, shrink and expand in one launch (device-resident ids)."""
        import torch
        from adapter_gemv_amd import sgmv
        p = self.p
        slot = k % self.slots
        stream = torch.cuda.current_stream()
        if ev is not None:
            ev[0].record(stream)
        st = sgmv.sgmv_lora_add_pool(
            stream.cuda_stream, self.dtype_code, self.y[slot].data_ptr(), self.ld_y,
            self.x[slot].data_ptr(), self.ld_x, self.ids_dev[slot].data_ptr(), p.n,
            self.A.data_ptr(), self.A.stride(0), self.B.data_ptr(), self.B.stride(0),
            self.n_pool, p.h_in, p.h_out, p.r, p.scale, self.ws.data_ptr(), self.ws.numel())
        if ev is not None:
            ev[1].record(stream)
        if st != 0:
            raise RuntimeError(f"sgmv_lora_add_pool failed: {sgmv.sgmv_status_string(st)}")

    def step_table(self, k: int, ev=None):
        """Segment metadata for slot k's batch (host build + one pinned H2D copy) and the
        fused LoRA add-on through the table interface."""
        import torch
        from adapter_gemv_amd import sgmv
        p = self.p
        slot = k % self.slots
        i = k % self.ring
        if self.ring_evt[i] is not None:
            self.ring_evt[i].synchronize()
        tab = sgmv.sgmv_build_segments(self.ids[slot], self.n_pool)
        a_ptr = sgmv.sgmv_build_ptr_table(self.A_bases, tab.seg_adapter)
        b_ptr = sgmv.sgmv_build_ptr_table(self.B_bases, tab.seg_adapter)
        S, n = tab.n_segments, tab.n
        buf = self.pinned_np[i]
        buf[: 8 * S] = a_ptr.view(np.uint8)
        buf[8 * S: 16 * S] = b_ptr.view(np.uint8)
        o_s = 16 * S
        buf[o_s: o_s + 4 * (S + 1)] = tab.seg_starts.view(np.uint8)
        o_p = o_s + 4 * (S + 1)
        buf[o_p: o_p + 4 * n] = tab.perm.view(np.uint8)
        dev = self.dev_meta[i]
        dev[: o_p + 4 * n].copy_(self.pinned[i, : o_p + 4 * n], non_blocking=True)
        base = dev.data_ptr()
        stream = torch.cuda.current_stream()
        if ev is not None:
            ev[0].record(stream)
        st = sgmv.sgmv_lora_add(
            stream.cuda_stream, self.dtype_code, self.y[slot].data_ptr(), self.ld_y,
            self.x[slot].data_ptr(), self.ld_x, base, base + 8 * S, base + o_s, base + o_p,
            n, S, tab.min_seg_len, tab.max_seg_len, p.h_in, p.h_out, p.r, p.scale,
            self.ws.data_ptr(), self.ws.numel())
        if ev is not None:
            ev[1].record(stream)
        if st != 0:
            raise RuntimeError(f"sgmv_lora_add failed: {sgmv.sgmv_status_string(st)}")
        e = torch.cuda.Event()
        e.record(stream)
        self.ring_evt[i] = e


def kernel_pass(rig, k0: int, count: int, fixed_slot=None) -> float:
    """Average duration of sgmv_lora_add alone on the table path: the segment tables of
    `count` steps are built and uploaded first, the calls are captured in one HIP graph
    and the replay is bracketed by HIP events.  ``fixed_slot``: every call on that slot
    (warm caches) instead of rotating."""
    import torch
    from adapter_gemv_amd import sgmv
    p = rig.p
    calls = []
    keep = []
    for k in range(count):
        slot = (k0 + k) % rig.slots if fixed_slot is None else fixed_slot
        b = sgmv.Batch.build(rig.ids[slot], rig.A, rig.B)
        keep.append(b)
        calls.append((slot, b))
    torch.cuda.synchronize()

    def run():
        st = torch.cuda.current_stream()
        for slot, b in calls:
            t = b.table
            rc = sgmv.sgmv_lora_add(st.cuda_stream, rig.dtype_code, rig.y[slot].data_ptr(),
                                    rig.ld_y, rig.x[slot].data_ptr(), rig.ld_x, b.A_ptrs_addr,
                                    b.B_ptrs_addr, b.seg_starts_addr, b.perm_addr, t.n,
                                    t.n_segments, t.min_seg_len, t.max_seg_len, p.h_in, p.h_out,
                                    p.r, p.scale, rig.ws.data_ptr(), rig.ws.numel())
            if rc != 0:
                raise RuntimeError(sgmv.sgmv_status_string(rc))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    g.replay()
    torch.cuda.synchronize()
    # the untimed replay's operands out of the caches; the timed replay is queued behind
    # the flush (warm calls: behind a spin kernel), so that its submission is not timed
    if fixed_slot is None:
        flush_caches(rig.device, wait=False)
    else:
        gpu_hold()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / count


_FLUSH = {}


def flush_caches(device, wait: bool = True) -> int:
    """Read FLUSH_BYTES of a buffer used for nothing else (a reduction: the lines it leaves
    in the caches are clean), so that whatever an untimed replay brought into the L2s and
    the Infinity Cache is evicted before the timed one.  With wait=False the read is only
    enqueued: a timed region whose start event follows it on the stream then begins with
    the launches already queued behind the flush, so their submission is not timed.
    Returns the bytes read."""
    import torch
    buf = _FLUSH.get(device)
    if buf is None:
        buf = _FLUSH[device] = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=device)
    torch.cuda.synchronize()
    buf.sum()
    if wait:
        torch.cuda.synchronize()
    return FLUSH_BYTES


def gpu_hold(us: float = 200.0, sync: bool = True) -> None:
    """Enqueue a spin kernel of about `us` microseconds (no memory traffic), so that the
    launches that follow are queued before the GPU reaches them and their submission is
    not timed (for warm-cache timings, where a flush would evict what they reuse)."""
    import torch
    if sync:
        torch.cuda.synchronize()
    torch.cuda._sleep(int(us * 2400))   # cycles at about 2.4 GHz


def queued_time(body, count: int, flush=None) -> float:
    """Average time of one `body(k)` call, k = 0 .. count-1 launched one after another on
    the current stream, queued behind a spin kernel long enough for the host to enqueue
    them all (and, with `flush`, behind a cache flush), bracketed by HIP events: the
    GPU runs them back to back with no launch gap.  body(0) runs once untimed first."""
    import torch
    stream = torch.cuda.current_stream()
    body(0)
    torch.cuda.synchronize()
    if flush is not None:
        flush_caches(flush, wait=False)
    gpu_hold(100.0 + 40.0 * count, sync=flush is None)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for k in range(count):
        body(k)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / count


def captured_call_time(rig) -> bool:
    """Whether the call's duration is taken from a graph replay: the device-table path
    (device ids, n > 64), whose captured calls overlap their two chains."""
    from adapter_gemv_amd import sgmv
    return rig.pool_path and not rig.host_ids and rig.p.n > sgmv.DECODE_MAX_TOKENS


def graph_call_time(rig, slot: int, count: int) -> float:
    """Average duration of `count` captured calls on one slot (warm caches), from HIP
    events around a replay queued behind a spin kernel."""
    import torch
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        rig.step(slot)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(count):
            rig.step(slot)
    g.replay()
    gpu_hold()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e-3 / count


def warm_call_time(rig, steps: int, use_graph: bool) -> float:
    """The SGMV call with warm caches: every call on the same slot (slot 1, not the
    parity slot), so its operands stay in the L2s and the Infinity Cache."""
    if use_graph and captured_call_time(rig):
        return graph_call_time(rig, 1, min(steps, 500))
    if use_graph:
        return queued_time(lambda k: rig.step(1), steps)
    return kernel_pass(rig, 1, min(steps, 500), fixed_slot=1)


def floors(nbytes: int, device, count: int) -> dict:
    """Reference floors on this GPU: a plain device copy moving the call's algorithmic
    bytes (half read, half written), cache-cold over > 1 GiB of rotating buffers, and
    one launch of a one-element kernel, both replayed from a HIP graph."""
    import torch
    half = max(1, nbytes // 4)                      # fp16 elements per copy side
    slots = max(2, min(256, -(-ROTATION_BYTES // (4 * half))))
    src = torch.ones((slots, half), dtype=torch.float16, device=device)
    dst = torch.empty_like(src)
    # slot 0 is copied untimed first; the timed copies start at slot 1
    t_copy = queued_time(lambda k: dst[(k + 1) % slots].copy_(src[(k + 1) % slots]), count,
                         flush=device)
    one = torch.zeros(1, dtype=torch.float32, device=device)
    t_launch = queued_time(lambda k: one.add_(1.0), count)
    del src, dst
    torch.cuda.empty_cache()
    moved = 4 * half
    return {"copy_same_bytes": {"bytes": moved, "us": round(t_copy * 1e6, 3),
                                "gbs": round(moved / t_copy / 1e9, 1),
                                "how": "torch device copy, rotating slots over > 1 GiB, "
                                       "after a 1 GiB cache flush, timed like us_per_call"},
            "launch_us": round(t_launch * 1e6, 3),
            "launch_how": "one-element torch add, timed like us_per_call"}


def parity_check(rig):
    """Run slot 0 (the seeded problem) once from its initial y and compare to the oracle."""
    import torch
    import oracle
    from adapter_gemv_amd.device_problem import to_numpy_storage
    p = rig.p
    rig.y[0].copy_(rig.y0)
    rig.step(0)
    torch.cuda.synchronize()
    got = oracle.decode(to_numpy_storage(rig.y[0], p.dtype), p.dtype)
    ref = oracle.lora_add_problem(p)
    err = np.abs(got - ref)
    tol = 1e-2 + 1e-2 * np.abs(ref)
    rig.y[0].copy_(rig.y0)
    flag = int(rig.ws[:4].view(torch.int32).item())
    return {"max_abs_err": float(err.max()), "worst_err_over_tol": float((err / tol).max()),
            "ok": bool(np.all(err <= tol)) and flag == 0, "workspace_flag": flag}


def load_traffic(workload: str, kernel: str):
    """HBM bytes per call from the committed rocprofv3 counter summary (FETCH_SIZE and
    WRITE_SIZE scaled by a plain copy of known size) of `kernel` on `workload`, if it was
    taken on the current kernel source; otherwise None.  Returns (bytes or None, where the
    figure comes from)."""
    rel = os.path.join("profiles", f"{kernel}_{workload}_counters.txt")
    path = os.path.join(ROOT, rel)
    if not os.path.exists(path):
        return None, f"no counter summary {rel} for this workload"
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("#", "rocprofv3", "`")):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.split()[0] if v.split() else ""
    src = rec.get("kernel_source_sha256_16")
    if src != kernel_source_hash(kernel):
        return None, (f"{rel} was taken on kernel source {src}, not the current sources' "
                      f"{kernel_source_hash(kernel)} ({', '.join(KERNEL_SRCS_OF[kernel])})")
    return int(float(rec["hbm_bytes_per_call"])), (
        f"from {rel}: FETCH_SIZE + WRITE_SIZE per call from two rocprofv3 --pmc runs, scaled "
        f"by a plain copy of known size; taken on kernel source {src}, the same as the "
        f"current sources; not measured in this run")


def measure(p, device, steps: int, warmup: int, eager: bool = False, force_table: bool = False,
            force_device: bool = False, host_ids: bool = False, warm: bool = True):
    """Check slot 0 against the oracle, then time `steps` steps after `warmup` untimed
    ones: wall time per step, GPU time per step, and the SGMV call's average duration."""
    import torch
    from adapter_gemv_amd import sgmv
    rig = Rig(p, device)
    if force_table:
        rig.pool_path = False
    if force_device:
        if p.n > sgmv.POOL_MAX_TOKENS:
            raise SystemExit(f"--path device takes at most {sgmv.POOL_MAX_TOKENS} tokens")
        rig.pool_path = True
    if host_ids:
        if p.n > sgmv.DECODE_MAX_TOKENS:
            raise SystemExit(f"--path host takes at most {sgmv.DECODE_MAX_TOKENS} tokens")
        rig.host_ids = True
    parity = parity_check(rig)
    print(f"# {p.name}: slots={rig.slots} pool_path={rig.pool_path} parity={parity}",
          file=sys.stderr, flush=True)
    use_graph = rig.pool_path and not eager
    for k in range(warmup):
        rig.step(1 + k)
    torch.cuda.synchronize()
    base = 1 + warmup
    stream = torch.cuda.current_stream()
    t_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    if use_graph:
        # capture the K timed steps (each on its own slot) into one graph
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            rig.step(base)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for k in range(steps):
                rig.step(base + k)
        graph.replay()                     # untimed: uploads the graph
        torch.cuda.synchronize()
        k_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        if captured_call_time(rig):
            # Device tables (n > 64): a captured call runs its short- and long-segment
            # chains side by side, an eager one runs them one after the other, so the
            # call's duration is taken from the graph: HIP events around a replay queued
            # behind a cache flush (the replay's fixed cost, about 12 us on this GPU, is
            # spread over the K calls).
            flush_caches(device, wait=False)
            k_ev[0].record(stream)
            graph.replay()
            k_ev[1].record(stream)
        else:
            # One launch per call: the K calls launched one after another on the stream,
            # queued behind a cache flush and a spin kernel long enough for the host to
            # enqueue them all, so that the GPU runs them back to back and the HIP events
            # around them see no launch gap (a graph launch adds about 12 us of its own
            # per replay on this GPU, whatever it holds).
            flush_caches(device, wait=False)
            gpu_hold(100.0 + 40.0 * steps, sync=False)
            k_ev[0].record(stream)
            for k in range(steps):
                rig.step(base + k)
            k_ev[1].record(stream)
        torch.cuda.synchronize()
        kernel_s = k_ev[0].elapsed_time(k_ev[1]) * 1e-3 / steps
        # the K steps' wall time: host clock around a replay of the graph after a cache
        # flush; the GPU time of the replay (HIP events) from a second replay after another
        # flush, so that recording the events is not in the wall time.  Two untimed
        # replays first (warm-up: the first replays of a graph launch more slowly; the
        # flush then evicts what they cached)
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        flush_caches(device)
        gc.disable()    # no collector pass inside the timed region
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        gc.enable()
        flush_caches(device)
        t_ev[0].record(stream)
        graph.replay()
        t_ev[1].record(stream)
        torch.cuda.synchronize()
        del graph
    else:
        torch.cuda.synchronize()
        flush_caches(device)
        gc.disable()
        t0 = time.perf_counter()
        t_ev[0].record(stream)
        for k in range(steps):
            rig.step(base + k)
        t_ev[1].record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        gc.enable()
    wall = (t1 - t0) / steps
    gpu_step = t_ev[0].elapsed_time(t_ev[1]) * 1e-3 / steps
    if use_graph:
        call_s = kernel_s
        call_how = ("HIP events around one replay of the K captured calls (short and long "
                    "chains side by side), queued behind a cache flush, / K"
                    if captured_call_time(rig) else
                    "HIP events around the K calls launched one after another, queued behind "
                    "a cache flush and a spin kernel (no launch gap), / K")
    else:
        call_s = kernel_pass(rig, base + steps, min(steps, 500))
        call_how = "HIP events over a graph of the same calls (tables pre-uploaded) / count"
    flag = int(rig.ws[:4].view(torch.int32).item())
    warm_s = None
    if warm:
        warm_s = warm_call_time(rig, steps, use_graph)
        flag = max(flag, int(rig.ws[:4].view(torch.int32).item()))
    return dict(rig=rig, parity=parity, use_graph=use_graph, wall=wall, gpu_step=gpu_step,
                call_s=call_s, call_how=call_how, flag=flag, warm_s=warm_s)


def layer_measure(p, device, steps: int) -> dict:
    """The LoRA linear layer end to end: the backbone y = x @ W (one torch matrix product,
    hipBLASLt, shared by every request) and then the SGMV add-on on the same stream.
    Times K steps of the backbone alone and K steps of the whole layer, each captured in
    one HIP graph (table-path segment tables are uploaded before capture).  Parity: the
    layer output of slot 0 against the oracle applied to the GPU backbone's output."""
    import torch
    import oracle
    from adapter_gemv_amd import sgmv
    from adapter_gemv_amd.device_problem import to_numpy_storage
    rig = Rig(p, device)
    tdt = rig.x.dtype
    g = torch.Generator(device=device)
    g.manual_seed(4321)
    # W stored as [h_in, h_out] so the product needs no transposed view
    Wt = (torch.randn((p.h_in, p.h_out), generator=g, device=device) / np.sqrt(p.h_in)).to(tdt)
    st = torch.cuda.current_stream()
    tables = {}

    def sgmv_call(k):
        slot = k % rig.slots
        if rig.pool_path:
            rig.step_pool(k)
            return
        b = tables[slot]
        t = b.table
        rc = sgmv.sgmv_lora_add(torch.cuda.current_stream().cuda_stream, rig.dtype_code,
                                rig.y[slot].data_ptr(), rig.ld_y,
                                rig.x[slot].data_ptr(), rig.ld_x, b.A_ptrs_addr, b.B_ptrs_addr,
                                b.seg_starts_addr, b.perm_addr, t.n, t.n_segments,
                                t.min_seg_len, t.max_seg_len, p.h_in, p.h_out, p.r, p.scale,
                                rig.ws.data_ptr(), rig.ws.numel())
        if rc != 0:
            raise RuntimeError(sgmv.sgmv_status_string(rc))

    def gemm(k):
        slot = k % rig.slots
        torch.mm(rig.x[slot], Wt, out=rig.y[slot])

    count = min(steps, rig.slots * 4)
    if not rig.pool_path:
        for k in range(count + 1):
            slot = k % rig.slots
            if slot not in tables:
                tables[slot] = sgmv.Batch.build(rig.ids[slot], rig.A, rig.B)
    # parity on slot 0
    gemm(0)
    torch.cuda.synchronize()
    y_bb = to_numpy_storage(rig.y[0], p.dtype).copy()
    sgmv_call(0)
    torch.cuda.synchronize()
    got = oracle.decode(to_numpy_storage(rig.y[0], p.dtype), p.dtype)
    ref = oracle.lora_add(y_bb, p.x, p.ids, p.A, p.B, p.scale, p.dtype)
    err = np.abs(got - ref)
    tol = 1e-2 + 1e-2 * np.abs(ref)
    parity = {"max_abs_err": float(err.max()), "worst_err_over_tol": float((err / tol).max()),
              "ok": bool(np.all(err <= tol))}

    def timed(body):
        side = torch.cuda.Stream()
        side.wait_stream(st)
        with torch.cuda.stream(side):
            for k in range(3):
                body(1 + k)
        st.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for k in range(count):
                body(1 + k)
        graph.replay()
        torch.cuda.synchronize()
        flush_caches(device, wait=False)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        graph.replay()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / count

    def layer(k):
        gemm(k)
        sgmv_call(k)

    t_gemm = timed(gemm)
    t_layer = timed(layer)
    return {"workload": p.name, "n_tokens": p.n, "h_in": p.h_in, "h_out": p.h_out, "r": p.r,
            "path": "one launch (sgmv_lora_add_pool)" if rig.pool_path else "table (sgmv_lora_add)",
            "steps": count, "backbone_us": round(t_gemm * 1e6, 3), "layer_us": round(t_layer * 1e6, 3),
            "sgmv_added_us": round((t_layer - t_gemm) * 1e6, 3),
            "sgmv_overhead_frac": round((t_layer - t_gemm) / t_gemm, 4), "parity": parity}


LAYER_WORKLOADS = ["decode7b", "sweep_b", "prefill13b_qo", "prefill13b_gateup", "prefill13b_down",
                   "mixed70b_r16_gate", "mixed70b_r64_gate"]


def run_layer(device, args) -> int:
    """One JSON line: backbone GEMM vs the whole LoRA layer for each layer workload."""
    import torch
    rows = []
    for name in LAYER_WORKLOADS:
        rows.append(layer_measure(workload_problem(name), device, args.steps))
        print(f"# {json.dumps(rows[-1])}", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "LoRA linear layer: backbone GEMM alone vs GEMM + SGMV, us per call",
                      "unit": "us", "higher_is_better": False, "n_gpus": 1, "data": "synthetic",
                      "cache": "cold (rotating slots, 1 GiB read before each timed run)", "points": rows}), flush=True)
    return 0 if all(r["parity"]["ok"] for r in rows) else 1


def run_load(device, args) -> int:
    """Adapter loading: host-to-HBM copies of LoRA adapters into a device adapter pool,
    from pinned and from pageable host memory, timed with HIP events; every copy is
    read back and compared bit for bit.  Sizes are Llama2-7B LoRA adapters at r = 16
    (fp16): one projection pair, q/k/v/o over 32 layers, and all seven projections."""
    import torch
    r, h, f, layers = 16, 4096, 11008, 32
    pair = 2 * r * h
    qkvo = layers * 4 * pair
    full = layers * (4 * pair + 2 * r * (h + f) + r * (f + h))
    rows = []
    ok = True
    st = torch.cuda.current_stream()
    for label, elems in [("one projection (A and B, 4096 x 16)", pair),
                         ("q/k/v/o, 32 layers", qkvo), ("all 7 projections, 32 layers", full)]:
        for pinned in (True, False):
            src = torch.randn(elems, dtype=torch.float32).to(torch.float16)
            if pinned:
                src = src.pin_memory()
            dst = torch.empty(elems, dtype=torch.float16, device=device)
            for _ in range(3):
                dst.copy_(src, non_blocking=pinned)
            torch.cuda.synchronize()
            reps = 20
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for _ in range(reps):
                dst.copy_(src, non_blocking=pinned)
            e1.record(st)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / reps
            same = bool(torch.equal(dst.cpu().view(torch.int16), src.view(torch.int16)))
            ok = ok and same
            rows.append({"adapter": label, "bytes": 2 * elems, "host_memory": "pinned" if pinned else "pageable",
                         "ms_per_upload": round(t * 1e3, 4), "GB_per_s": round(2 * elems / t / 1e9, 2),
                         "bit_exact": same})
            del src, dst
    first = upload_and_first_call(device)
    ok = ok and all(f.get("parity_ok", True) for f in first)
    print(json.dumps({"metric": "LoRA adapter upload, host to HBM", "unit": "ms", "higher_is_better": False,
                      "n_gpus": 1, "data": "synthetic", "points": rows,
                      "upload_plus_first_call": first}), flush=True)
    return 0 if ok else 1


def upload_and_first_call(device) -> list:
    """On-demand loading end to end (AdapterPool): a 7B-shaped decode batch (32 tokens,
    h = 4096, r = 16, fp16) whose 32 adapters are registered in pinned host memory, against
    a device pool of 64 slots.  Host wall time from the slot mapping to the end of the SGMV
    call: every adapter missing (32 uploads of A and B), one adapter missing, none missing.
    Each result is checked against the oracle."""
    import torch
    import oracle
    from adapter_gemv_amd import sgmv
    from adapter_gemv_amd.adapter_pool import AdapterPool
    from adapter_gemv_amd.device_problem import to_numpy_storage
    p = synth.decode7b()
    pool = AdapterPool(64, p.r, p.h_in, p.h_out, dtype=torch.float16, device=device)
    keys = list(range(100, 100 + p.n_adapters + 1))
    for i in range(p.n_adapters):
        pool.register(keys[i], sgmv.as_tensor(p.A[i], p.dtype), sgmv.as_tensor(p.B[i], p.dtype))
    pool.register(keys[-1], sgmv.as_tensor(p.A[0], p.dtype), sgmv.as_tensor(p.B[0], p.dtype))
    x = sgmv.as_tensor(p.x, p.dtype, device)
    ws = sgmv.make_workspace(p.n, p.h_in, p.r, device)
    ref = oracle.lora_add_problem(p)
    # one untimed round first (first copies and launch), then the pool is emptied again
    y = sgmv.as_tensor(p.y, p.dtype, device)
    pool.lora_add(y, x, pool.prepare([keys[i] for i in p.ids]), p.scale, workspace=ws)
    torch.cuda.synchronize()
    for k in keys[:-1]:
        pool.cache.evict(k)
    out = []
    # all 32 missing; then the same batch (all resident); then one row on a new key (whose
    # adapter equals adapter 0), the other 31 resident
    batches = [("all 32 adapters missing", [keys[i] for i in p.ids]),
               ("all resident", [keys[i] for i in p.ids]),
               ("one adapter missing", [keys[-1] if i == 0 else keys[i] for i in p.ids])]
    for label, bkeys in batches:
        y = sgmv.as_tensor(p.y, p.dtype, device)
        torch.cuda.synchronize()
        m0 = pool.stats["misses"]
        t0 = time.perf_counter()
        slots = pool.prepare(bkeys)
        pool.lora_add(y, x, slots, p.scale, workspace=ws)
        torch.cuda.synchronize()
        t = time.perf_counter() - t0
        got = oracle.decode(to_numpy_storage(y, p.dtype), p.dtype)
        err = np.abs(got - ref)
        out.append({"case": label, "uploads": pool.stats["misses"] - m0,
                    "ms_map_upload_and_call": round(t * 1e3, 4),
                    "parity_ok": bool(np.all(err <= 1e-2 + 1e-2 * np.abs(ref)))})
    out.append({"bytes_per_adapter": 2 * p.r * (p.h_in + p.h_out),
                "how": "host wall clock around AdapterPool.prepare (native slot cache + "
                       "sgmv_upload_adapter from pinned memory) and the one-launch SGMV call, "
                       "then a synchronisation; parity_ok false on a missing row"})
    pool.close()
    return out


def use_host_ids(path: str, p) -> bool:
    """The default path of a decode batch (<= 64 tokens) is the one-launch kernel with the
    ids in its arguments (the scheduler that forms the batch has them on the host)."""
    from adapter_gemv_amd import sgmv
    return path == "host" or (path == "auto" and p.n <= sgmv.DECODE_MAX_TOKENS)


def run_phases(device, args) -> int:
    """Per-phase timeline of the one-launch decode kernel, from the profiling variant of the
    library (libsgmv_phases.so: lane 0 of every wave stamps the 100 MHz real-time counter at
    fixed points of its item).  K cache-cold calls queued behind a flush and a spin kernel,
    as for us_per_call; each call's stamps are taken relative to its first wave's start.
    One JSON line: per phase, the median and p90 over every wave of every call."""
    import torch
    from adapter_gemv_amd import _lib, sgmv
    _lib.use_phase_stamps()
    p = workload_problem(args.workload)
    if p.n > sgmv.DECODE_MAX_TOKENS:
        raise SystemExit("--phases times the one-launch decode kernel (<= 64 tokens)")
    rig = Rig(p, device)
    rig.host_ids = use_host_ids(args.path, p)
    parity = parity_check(rig)
    K = args.steps
    kc, cols = 8192 // p.r, 64 * (128 // p.r)   # shrink K chunk, expand columns per item
    KS, NS = -(-p.h_in // kc), -(-p.h_out // cols)
    grid = p.n * (KS + NS)
    if grid > 8192:
        raise SystemExit("grid too large for the stamp buffer")
    buf = torch.zeros(K * 8192 * 8, dtype=torch.int64, device=device)
    for k in range(args.warmup):
        rig.step(1 + k)
    base = 1 + args.warmup
    stream = torch.cuda.current_stream()
    flush_caches(device, wait=False)
    gpu_hold(100.0 + 40.0 * K, sync=False)
    L = _lib.lib()
    L.sgmv_phase_stamps_attach(buf.data_ptr(), K)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for k in range(K):
        rig.step(base + k)
    e1.record(stream)
    torch.cuda.synchronize()
    stamped = int(L.sgmv_phase_stamps_attach(None, 0))
    call_us = e0.elapsed_time(e1) * 1e3 / K
    st = buf.view(K, 8192, 8)[:stamped, :grid].cpu().numpy().astype(np.float64)
    t0 = np.where(st[:, :, 0] > 0, st[:, :, 0], np.inf).min(axis=1)[:, None]
    rel = (st - t0[:, :, None]) * 0.01                      # 100 MHz ticks -> us
    shrink, expand = rel[:, : p.n * KS], rel[:, p.n * KS:]
    active = st[:, : p.n * KS, 2] > 0                        # shrink items that had work

    def stat(a):
        a = a[np.isfinite(a)]
        return {"median_us": round(float(np.median(a)), 3), "p90_us": round(float(np.percentile(a, 90)), 3)} \
            if a.size else None

    names_s = ["wave start", "ids in registers", "A and x loaded", "partial sums issued",
               "partial sums acknowledged"]
    names_e = ["wave start", "ids in registers", "B and y loaded", "every partial sum present",
               "y stored (issued)", "y store acknowledged", "item done"]
    span = np.nanmax(np.where(st > 0, rel, np.nan).reshape(stamped, -1), axis=1)
    out = {
        "metric": "one-launch decode kernel: phase timeline (us after the call's first wave started)",
        "workload": p.name, "path": "host ids" if rig.host_ids else "device ids",
        "calls": stamped, "grid": grid, "shrink_items": p.n * KS, "expand_items": p.n * NS,
        "active_shrink_items_per_call": round(float(active.sum(axis=1).mean()), 1),
        "us_per_call_stamped_build": round(call_us, 3),
        "first_to_last_wave_start_us": stat(np.nanmax(np.where(st[:, :, 0] > 0, rel[:, :, 0], np.nan), axis=1)),
        "last_stamp_us": stat(span),
        "shrink": {n: stat(np.where(active, shrink[:, :, i], np.nan)) for i, n in enumerate(names_s)},
        "expand": {n: stat(expand[:, :, i]) for i, n in enumerate(names_e)},
        "parity": parity,
        "how": "libsgmv_phases.so (-DSGMV_PHASE_STAMPS): s_memrealtime after waiting for the "
               "wave's memory operations at each point; the waits themselves change timing a "
               "little (compare us_per_call_stamped_build with bench.py's us_per_call)",
    }
    print(json.dumps(out), flush=True)
    return 0 if parity["ok"] else 1


SWEEPS = {
    # the pages' idea I5: latency against batch size, per stage
    "decode": [f"decode7b_bs{n}" for n in (1, 2, 4, 8, 16, 24, 32, 48, 64)],
    "prefill": [f"prefill13b_gateup_len{L}" for L in (16, 32, 64, 128, 256, 512, 1024)],
}


def run_sweep(kind: str, device, args) -> int:
    """SGMV time per call against batch size (decode shape) or prompt length (prefill
    shape); one JSON line with one entry per point."""
    import torch
    points = []
    ok = True
    for name in SWEEPS[kind]:
        p = workload_problem(name)
        steps = args.steps if kind == "decode" else max(20, args.steps // 20)
        m = measure(p, device, steps, min(args.warmup, steps), eager=args.eager, warm=False,
                    host_ids=use_host_ids(args.path, p))
        nbytes = algorithmic_bytes(p)
        points.append({
            "workload": p.name, "n_tokens": p.n, "distinct_adapters": p.distinct_adapters(),
            "path": ("one launch, host ids (sgmv_lora_add_host_ids)" if m["rig"].host_ids else
                     "one launch (sgmv_lora_add_pool)") if m["rig"].pool_path else
                    "table (sgmv_lora_add)",
            "us_per_call": round(m["call_s"] * 1e6, 3),
            "us_per_step": round(m["wall"] * 1e6, 3),
            "algorithmic_bytes_per_call": nbytes,
            "GB_per_s": round(nbytes / m["call_s"] / 1e9, 2),
            "frac_of_hbm_peak": round(nbytes / m["call_s"] / 1e9 / HBM_PEAK_GBS, 4),
            "parity_ok": m["parity"]["ok"] and m["flag"] == 0,
        })
        ok = ok and points[-1]["parity_ok"]
        del m
        torch.cuda.empty_cache()
    print(json.dumps({
        "metric": f"SGMV us/call against {'batch size' if kind == 'decode' else 'prompt length'}",
        "sweep": kind, "unit": "us", "higher_is_better": False, "n_gpus": 1,
        "data": "synthetic", "cache": "cold (rotating slots, 1 GiB read before each timed run)", "points": points,
    }), flush=True)
    return 0 if ok else 1


# --------------------------------------------------------------------------------------
# mixed ranks in one call
# --------------------------------------------------------------------------------------
def ranked_bytes(q) -> int:
    """x read once, y read and written once, each distinct adapter's A and B once at its
    own rank."""
    ranks = q.ranks()
    ad = sum(int(ranks[a]) * (q.h_in + q.h_out) for a in np.unique(q.ids))
    return 2 * (q.n * q.h_in + 2 * q.n * q.h_out + ad)


def ranked_flops(q) -> int:
    return 2 * int(q.ranks()[q.ids].sum()) * (q.h_in + q.h_out)


def run_ranked(device, args) -> int:
    """One mixed-rank workload through sgmv_lora_add_ranked: rank-16 and rank-64 adapters
    in one call.  Tables of every rotation slot are built and uploaded first; the K timed
    calls are replayed from one HIP graph bracketed by HIP events."""
    import torch
    import oracle
    from adapter_gemv_amd import sgmv
    from adapter_gemv_amd.device_problem import to_numpy_storage
    proj = args.workload[len("mixed70b_rmix_"):]
    if proj not in synth.MIXED70B_SHAPES:
        raise SystemExit(f"unknown projection {proj!r}")
    q = synth.mixed70b_ranked(proj)
    nbytes, flops = ranked_bytes(q), ranked_flops(q)
    slots = max(2, min(64, -(-ROTATION_BYTES // nbytes)))
    tdt = torch.bfloat16
    g = torch.Generator(device=device)
    g.manual_seed(4321)

    def randn(shape, std):
        return (torch.randn(shape, generator=g, device=device) * std).to(tdt)

    x = randn((slots, q.n, q.h_in), 1.0)
    y = randn((slots, q.n, q.h_out), 1.0)
    x[0].copy_(sgmv.as_tensor(q.x, q.dtype, device))
    y[0].copy_(sgmv.as_tensor(q.y, q.dtype, device))
    y0 = y[0].clone()
    pools, offs, big_off = [], [], 0
    for A_h, B_h in q.pools:
        P, r = A_h.shape[0], A_h.shape[1]
        A = randn((slots * P, r, q.h_in), 1.0 / np.sqrt(q.h_in))
        B = randn((slots * P, q.h_out, r), 1.0 / np.sqrt(r))
        A[:P].copy_(sgmv.as_tensor(A_h, q.dtype, device))
        B[:P].copy_(sgmv.as_tensor(B_h, q.dtype, device))
        pools.append((A, B))
        offs.append((big_off, P))
        big_off += slots * P
    starts = np.cumsum([0] + [A.shape[0] for A, _ in q.pools])
    batches = []
    for s in range(slots):
        ids = np.empty_like(q.ids)
        for k, (bo, P) in enumerate(offs):
            m = (q.ids >= starts[k]) & (q.ids < starts[k + 1])
            ids[m] = bo + s * P + (q.ids[m] - starts[k])
        batches.append(sgmv.RankedBatch.build(ids, pools))
    ws = sgmv.make_workspace(q.n, q.h_in, 64, device)
    torch.cuda.synchronize()

    def call(k):
        sgmv.lora_add_ranked(y[k % slots], x[k % slots], batches[k % slots], q.scales, ws)

    call(0)
    torch.cuda.synchronize()
    got = oracle.decode(to_numpy_storage(y[0], q.dtype), q.dtype)
    ref = oracle.lora_add_ranked(q.y, q.x, q.ids, q.pools, q.scales, q.dtype)
    err = np.abs(got - ref)
    tol = 1e-2 + 1e-2 * np.abs(ref)
    parity = {"max_abs_err": float(err.max()), "worst_err_over_tol": float((err / tol).max()),
              "ok": bool(np.all(err <= tol))}
    y[0].copy_(y0)
    print(f"# {q.name}: slots={slots} parity={parity}", file=sys.stderr, flush=True)
    for k in range(args.warmup):
        call(1 + k)
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        call(1)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(args.steps):
            call(1 + k)
    graph.replay()
    torch.cuda.synchronize()
    flush_caches(device, wait=False)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    call_s = e0.elapsed_time(e1) * 1e-3 / args.steps
    flush_caches(device)
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    ranks = q.ranks()
    out = {
        "metric": METRIC,
        "value": round(nbytes / wall / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": q.dtype,
        "data": "synthetic",
        "config": {
            "workload": q.name, "n_tokens": q.n, "h_in": q.h_in, "h_out": q.h_out,
            "rows_per_rank": {int(r): int((ranks[q.ids] == r).sum()) for r in q.scales},
            "scales": {int(r): v for r, v in q.scales.items()},
            "distinct_adapters": int(np.unique(q.ids).size), "rotation_slots": slots,
            "cache": "cold: every timed call on its own slot, "
                     f"{FLUSH_BYTES >> 20} MiB read between the untimed and the timed run",
            "step": "sgmv_lora_add_ranked (one call, both rank groups), tables pre-uploaded, "
                    "K calls replayed from one HIP graph",
        },
        "us_per_call": round(call_s * 1e6, 3),
        "us_per_call_wall": round(wall * 1e6, 3),
        "algorithmic_bytes_per_call": nbytes,
        "gflops_per_s": round(flops / call_s / 1e9, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(nbytes / call_s / 1e9, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(nbytes / call_s / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": None,
            "kernel": "sgmv_lora_add_ranked: table kernels of every rank group",
            "mfma_frac": round(flops / call_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5),
        },
        "parity": parity,
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    print(json.dumps(out), flush=True)
    return 0 if parity["ok"] else 1


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="decode7b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", choices=["auto", "table", "device", "host"], default="auto",
                    help="auto: one launch with the host ids in its kernel arguments for "
                         "batches of <= 64 tokens, host-built tables above; device: device ids "
                         "for any batch up to 4096 tokens (one launch up to 64, device "
                         "grouping + table kernels above, graph-captured); table: host "
                         "tables; host: the one-launch host-id kernel (<= 64)")
    ap.add_argument("--eager", action="store_true", help="no HIP graph on the one-launch path")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--cold-only", action="store_true",
                    help="skip the warm-cache timing and the floors (profiled runs: only the "
                         "cold calls reach the profiler)")
    ap.add_argument("--sweep", choices=sorted(SWEEPS),
                    help="time a batch-size (decode) or prompt-length (prefill) sweep instead")
    ap.add_argument("--layer", action="store_true",
                    help="time the LoRA linear layer (backbone GEMM + SGMV) on several workloads")
    ap.add_argument("--load", action="store_true",
                    help="time LoRA adapter uploads from host memory into HBM")
    ap.add_argument("--phases", action="store_true",
                    help="per-phase timeline of the one-launch decode kernel (profiling build)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter scaling)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only; multi-GPU runs are not supported "
              "(--gpus 1)", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 2
        a = torch.ones(n, dtype=torch.float16, device=device)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": 2 * n}))
        return 0

    if args.phases:
        return run_phases(device, args)
    if args.sweep:
        return run_sweep(args.sweep, device, args)
    if args.layer:
        return run_layer(device, args)
    if args.load:
        return run_load(device, args)
    if args.workload.startswith("mixed70b_rmix_"):
        return run_ranked(device, args)

    p = workload_problem(args.workload)
    m = measure(p, device, args.steps, args.warmup, eager=args.eager,
                force_table=args.path == "table", force_device=args.path == "device",
                host_ids=use_host_ids(args.path, p), warm=not args.cold_only)
    rig, parity, use_graph = m["rig"], m["parity"], m["use_graph"]
    wall, gpu_step, call_s, call_how, flag = (m["wall"], m["gpu_step"], m["call_s"],
                                              m["call_how"], m["flag"])

    nbytes = algorithmic_bytes(p)
    flops = algorithmic_flops(p)
    if rig.host_ids:
        traffic, traffic_src = load_traffic(args.workload, "lora_add_ids_kernel")
    elif rig.pool_path and p.n <= 64:
        traffic, traffic_src = load_traffic(args.workload, "lora_add_pool_kernel")
    elif not rig.pool_path:
        traffic, traffic_src = load_traffic(args.workload, "sgmv_lora_add")
    else:
        traffic, traffic_src = None, "no counter summary for the device-id table path"
    if rig.host_ids:
        kernel = "lora_add_ids_kernel (one launch per call, ids in the kernel arguments)"
    elif rig.pool_path and p.n <= 64:
        kernel = "lora_add_pool_kernel (one launch per call)"
    elif rig.pool_path:
        kernel = "sgmv_lora_add_pool: device segment sort + table kernels (all launches of one call)"
    else:
        kernel = "sgmv_lora_add table path (all kernels of one call)"
    out = {
        "metric": METRIC,
        "value": round(nbytes / wall / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic",
        "config": {
            "workload": p.name, "n_tokens": p.n, "h_in": p.h_in, "h_out": p.h_out, "r": p.r,
            "distinct_adapters": p.distinct_adapters(), "adapter_pool": p.n_adapters,
            "scale": p.scale, "rotation_slots": rig.slots,
            "rotation_bytes": rig.slots * nbytes,
            "cache": "cold: every timed step on its own slot of x, y, ids and adapters, and "
                     f"{FLUSH_BYTES >> 20} MiB read between the untimed and the timed run",
            "min_bytes_between_slot_reuse": min(FLUSH_BYTES, rig.slots * nbytes)
                                            if args.steps > rig.slots else FLUSH_BYTES,
            "step": ("sgmv_lora_add_host_ids: host ids in the kernel arguments, grouping + "
                     "shrink + expand in one launch" +
                     (", K steps replayed from one HIP graph" if use_graph else ", eager"))
                    if rig.host_ids else
                    (("sgmv_lora_add_pool: device segment sort + shrink + expand, one launch"
                      if p.n <= 64 else
                      "sgmv_lora_add_pool: device segment sort, then the table kernels") +
                     (", K steps replayed from one HIP graph" if use_graph else ", eager"))
                    if rig.pool_path else
                    "host segment build + pinned H2D tables + sgmv_lora_add, eager",
        },
        "us_per_step_gpu": round(gpu_step * 1e6, 3),
        "us_per_call": round(call_s * 1e6, 3),
        "us_per_call_how": call_how,
        "algorithmic_bytes_per_call": nbytes,
        "gflops_per_s": round(flops / call_s / 1e9, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(nbytes / call_s / 1e9, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(nbytes / call_s / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_source": traffic_src,
            "kernel": kernel,
            "mfma_frac": round(flops / call_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5),
        },
        "parity": parity,
        "workspace_flag_after": flag,
        "kernel_source_sha256_16": kernel_source_hash(),
        "kernel_source_sha256_16_by_path": {k: kernel_source_hash(k) for k in
                                            ("lora_add_ids_kernel", "sgmv_lora_add")},
    }
    if m["warm_s"] is not None:
        out["warm"] = {"us_per_call": round(m["warm_s"] * 1e6, 3),
                       "gbs": round(nbytes / m["warm_s"] / 1e9, 1),
                       "how": "every call on one slot (operands cached), same timing as "
                              "us_per_call"}
        out["floors"] = floors(nbytes, device, min(args.steps, 500))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p, args.cpu_budget)
        out["cpu_baseline_1thread"] = cpu_baseline_1thread(p, args.cpu_budget / 2)
    print(json.dumps(out), flush=True)
    return 0 if parity["ok"] else 1


if __name__ == "__main__":
    sys.exit(main())
