"""Benchmark: q8 decode-attention decode steps on one MI355X.

One step = for every layer of the workload: append one new token per sequence
and run the decode attention over every sequence's whole history.  By default
(--append fused) that is q8_decode_step: the append inside the decode's
partial kernel, then the merge kernel; --append separate runs q8_kv_append,
then q8_decode_attn (partial + merge).  Inputs (cache history, the step's q and new
K/V, block tables) are resident in HBM before timing starts.

Prints ONE JSON line (rank 0): achieved algorithmic HBM GB/s of the whole step
as `value`, plus a `roofline` object for the dominant kernel (the decode
partial kernel, timed with HIP events on its own stream) and a `cpu_baseline`
object (the CPU oracle on one layer-step of the same workload).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix-core peak, vendor figure (no sparsity)
POOL_TOKENS = 65536            # N(0,1) source rows the history is appended from
FILL_CHUNK = 32768


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen2b_b64_ragged", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--nparts", type=int, default=0, help="decode partitions (0 = automatic)")
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (0 = the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", choices=("q8", "f32", "sparse", "prefill"), default="q8",
                    help="q8: the q8 cache (default); f32: the fp32 mirror and its exact decode "
                         "(the append then writes the mirror too); sparse: block-sparse decode (top-k "
                         "32-token blocks per query head by probe); prefill: batched causal prefill of "
                         "the workload's new tokens (a qwen2b_prefill_* workload)")
    ap.add_argument("--topk", type=int, default=32, help="blocks kept per query head (--path sparse)")
    ap.add_argument("--append", choices=("fused", "separate"), default="fused",
                    help="--path q8: the new tokens appended inside the decode's partial kernel "
                         "(q8_decode_step) or by q8_kv_append before it")
    ap.add_argument("--invariant", action="store_true",
                    help="decode with the batch-invariant cut (Q8_BATCH_INVARIANT: a sequence's bits independent "
                         "of the rest of the batch; no step plan)")
    ap.add_argument("--no-plan", action="store_true",
                    help="decode without a step plan: every layer's partial kernel makes the cut itself "
                         "(default: q8_decode_plan once per step, read by every layer, when a step has "
                         "more than one layer)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the other batch x context configurations (reported under config.sweep)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--read-probe", type=int, default=0, metavar="MIB",
                    help="only measure the read ceiling: stream a buffer of this many MiB once per launch "
                         "(q8_stream_read), plain and non-temporal, over 256 / 512 / 1024 workgroups")
    ap.add_argument("--issue-probe", action="store_true",
                    help="only measure instruction issue (q8_issue_probe): VALU waves alone, matrix-core waves "
                         "alone, both on the same SIMDs, and two or four VALU waves per SIMD")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of replaying the step as one HIP graph")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "q8_attn_partial_kernel_hbm_traffic.json"),
                    help="measured HBM bytes per launch (from rocprofv3 counters), if present")
    ap.add_argument("--traffic-from", default=None, metavar="DIR",
                    help="no GPU work: read rocprofv3 counter CSVs under DIR/{copyf,copyw,fetch,write} "
                         "and record the workload's bytes per partial launch in --traffic")
    return ap.parse_args()


def algorithmic_bytes(w: workloads.Workload, lens: np.ndarray, kv_bs: int, path: str = "q8", topk: int = 32):
    """Bytes one layer-step must move at least once.
    q8 attention: K and V codes and scales of every visible token, read once
    per KV head (n * nkv * (2*128 + 8)); f32 attention: the fp32 mirror rows
    instead (n * nkv * 2*128*4); sparse attention: the probe rows' K codes
    and scales per KV head plus the kept blocks' K and V codes and scales per
    query head (a kept block counted as 32 tokens).  Both: q in and out (B*nq*128*4*2), block-
    table entries and lengths.  append: fp32 K and V in (T*nkv*128*4*2),
    codes and scales out (T*nkv*(2*128 + 8)), with the mirror also the fp32
    rows out (T*nkv*128*4*2), token indices (T*8)."""
    n = lens.astype(np.int64)
    per_tok = 2 * w.head_dim * 4 if path == "f32" else 2 * w.head_dim + 8
    kv = int(n.sum()) * w.nkv * per_tok
    if path == "sparse":
        # probe: K codes and scale of rows 0, 4, ..., 28 of every block of a
        # probed sequence, once per KV head; attention: every token of the kept
        # blocks, K and V codes and scales, once per query head
        nb = (n + 31) // 32
        probed = nb > topk
        probe_rows = int(np.minimum((n - 32 * (nb - 1) + 3) // 4, 8)[probed].sum() + (8 * (nb[probed] - 1)).sum())
        kept = np.where(probed, 32 * topk, n)
        kv = probe_rows * w.nkv * (w.head_dim + 4) + int(kept.sum()) * w.nq * (2 * w.head_dim + 8)
    qo = w.batch * w.nq * w.head_dim * 4 * 2
    meta = int(((n + kv_bs - 1) // kv_bs).sum()) * 4 + w.batch * 4
    t = w.batch * w.append_per_step
    app = t * w.nkv * w.head_dim * 4 * 2 + t * w.nkv * (2 * w.head_dim + 8) + t * 8
    if path == "f32":
        app += t * w.nkv * w.head_dim * 4 * 2
    return kv + qo + meta, app


def _counter_values(path: str, counter: str, kernel_substr: str) -> list:
    import csv
    import glob
    vals = []
    for f in sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)):
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] == counter and kernel_substr in row["Kernel_Name"]:
                    vals.append(float(row["Counter_Value"]))
    return vals


def traffic_from(args):
    """Copy-calibrated HBM bytes per decode partial launch.  FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) are read for a plain copy of a known size
    (bench.py --copy-probe) and for the partial kernel of the workload; each
    counter is scaled by (copy bytes / counter reading of the copy)."""
    d = args.traffic_from
    probe = None
    for name in ("copyf", "copyw"):
        log = os.path.join(d, name + ".log")
        if os.path.exists(log):
            for line in open(log):
                if line.startswith("{") and "copy_probe_bytes" in line:
                    probe = json.loads(line)["copy_probe_bytes"]
    if probe is None:
        raise SystemExit("no copy-probe size found in copyf.log / copyw.log")
    kib = probe / 1024.0

    def factor(sub, counter):
        v = sorted(_counter_values(os.path.join(d, sub), counter, "copyBuffer"))
        v = [x for x in v if x > 0.5 * kib / 4]   # the probe's copies, not small blits
        if not v:
            raise SystemExit(f"no copy dispatches with {counter} under {sub}")
        return kib / float(np.median(v)), float(np.median(v))

    ff, fcopy = factor("copyf", "FETCH_SIZE")
    fw, wcopy = factor("copyw", "WRITE_SIZE")
    fetch = _counter_values(os.path.join(d, "fetch"), "FETCH_SIZE", "q8_attn_partial_kernel")
    write = _counter_values(os.path.join(d, "write"), "WRITE_SIZE", "q8_attn_partial_kernel")
    if not fetch or not write:
        raise SystemExit("no q8_attn_partial_kernel dispatches in fetch/ or write/")
    fk, wk = float(np.median(fetch)), float(np.median(write))
    total = (fk * ff + wk * fw) * 1024.0
    rec = {}
    if os.path.exists(args.traffic):
        with open(args.traffic) as f:
            rec = json.load(f)
    rec[args.workload] = {
        "kernel": "q8_attn_partial_kernel", "kernel_hash": kernel_hash(),
        "bytes_per_launch": int(round(total)),
        "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
        "dispatches": [len(fetch), len(write)],
        "copy_probe_bytes": probe, "copy_fetch_kib": round(fcopy, 1), "copy_write_kib": round(wcopy, 1),
        "fetch_factor": round(ff, 4), "write_factor": round(fw, 4),
    }
    with open(args.traffic, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(rec[args.workload]))


# Configurations measured beside the headline workload, each with the
# workload's own layer count and a distinct cache pool per layer (so every
# layer's cache is cold in the 256 MB last-level cache whenever a layer
# exceeds it).
SWEEP = ("single_head_256", "qwen2b_b1_n506", "qwen2b_b1_n2046", "qwen2b_b1_n4059",
         "qwen8b_b32_n32k", "qwen8b_b1_n128k", "qwen8b_b128_stress")


def measure(torch, q8, dev, w, layers, steps, warmup, nparts_arg=0, eager=False, path="q8", topk=32,
            fused=True, planned=True, invariant=False):
    """One workload: fill `layers` cache pools, then time whole decode steps
    (graph replay unless eager) and, in an eager pass with HIP events on the
    library's stream, each kernel.  With `planned` (the q8 and f32 paths), a
    step starts with q8_decode_plan and every layer's decode reads the plan;
    the plan kernel is inside the timed step.  Returns a dict of figures."""
    lens = workloads.seq_lens(w)
    kv_bs = w.kv_bs
    B, nq, nkv, hd = w.batch, w.nq, w.nkv, w.head_dim
    scale = float(workloads.softmax_scale(hd))
    t_setup = time.perf_counter()

    # ---- cache: one pool per layer, blocks of every sequence scattered at random
    table, nblocks = workloads.block_table(lens, kv_bs, w.seed)
    table_t = torch.from_numpy(table).to(dev)
    lens_t = torch.from_numpy(lens).to(dev)
    invariant = invariant and path in ("q8", "f32")
    batch = q8.make_batch(table_t, lens_t, int(max(1, lens.max())), invariant=invariant)
    pools = [q8.alloc_layer(nblocks, kv_bs, nkv, dev, mirror=(path == "f32")) for _ in range(layers)]
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    partial = q8.decode_attn_f32_partial if path == "f32" else q8.decode_attn_partial
    merge = q8.decode_attn_merge
    fused = fused and path == "q8"
    if path == "sparse":
        # the whole sparse decode (probe + attend kernels) in the partial slot; no merge
        def partial(pool, batch_, nq_, q_, scale_, out_, ws_, nparts=0, dev_status=None):
            q8.decode_attn_sparse(pool, batch_, nq_, q_, scale_, out_, ws_, topk=topk, dev_status=dev_status)

        def merge(*a, **k):
            pass

    # history: every position but the last, appended from a source pool drawn
    # with the workload's value distribution
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    src_k = workloads.kv_pool_torch(w, POOL_TOKENS + FILL_CHUNK, gen, dev)
    src_v = workloads.kv_pool_torch(w, POOL_TOKENS + FILL_CHUNK, gen, dev)
    hist_seq = np.concatenate([np.full(max(n - 1, 0), b, np.int32) for b, n in enumerate(lens)])
    hist_pos = np.concatenate([np.arange(max(n - 1, 0), dtype=np.int32) for n in lens])
    hist_seq_t = torch.from_numpy(hist_seq).to(dev)
    hist_pos_t = torch.from_numpy(hist_pos).to(dev)
    rng = np.random.default_rng(w.seed)
    for li, pool in enumerate(pools):
        for c0 in range(0, hist_seq.size, FILL_CHUNK):
            c1 = min(hist_seq.size, c0 + FILL_CHUNK)
            off = int(rng.integers(0, POOL_TOKENS))
            q8.kv_append(pool, batch, hist_seq_t[c0:c1], hist_pos_t[c0:c1],
                         src_k[off:off + c1 - c0], src_v[off:off + c1 - c0], dev_status=status)
    del src_k, src_v

    # the step's inputs: one new token per sequence (position n_b - 1) and q, per layer
    step_seq = torch.arange(B, dtype=torch.int32, device=dev)
    step_pos = (lens_t - 1).clamp(min=0).to(torch.int32)
    new_k = torch.randn((layers, B, nkv, hd), generator=gen, device=dev)
    new_v = torch.randn((layers, B, nkv, hd), generator=gen, device=dev)
    qs = torch.randn((layers, B, nq, hd), generator=gen, device=dev)
    outs = torch.empty((layers, B, nq, hd), dtype=torch.float32, device=dev)
    # the calls get the requested count (0: the library's automatic cut, which
    # may also choose the workgroup shape); the JSON reports the resolved count
    nparts = nparts_arg or q8.decode_attn_auto_parts(pools[0], batch, nq)
    call_parts = nparts_arg
    ws_bytes = q8.decode_attn_workspace_bytes(pools[0], batch, nq, call_parts)
    if path == "sparse":
        ws_bytes = max(ws_bytes, q8.decode_attn_sparse_workspace_bytes(pools[0], batch, nq, topk))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    # a plan is made once per step and pays for itself over the step's layers;
    # a one-layer step does not plan
    planned = planned and path in ("q8", "f32") and layers > 1 and not invariant
    plan = None
    if planned:
        plan = torch.empty(q8.decode_plan_bytes(pools[0], batch, nq, call_parts), dtype=torch.uint8, device=dev)
    batch_p = batch.with_plan(plan)   # the decode calls' batch (the appends and the plan itself ignore it)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "device status set during fill"
    setup_s = time.perf_counter() - t_setup

    def make_plan():
        if planned:
            q8.decode_plan(pools[0], batch, nq, plan, nparts=call_parts, dev_status=status)

    def append(li):
        if not fused:
            q8.kv_append(pools[li], batch, step_seq, step_pos, new_k[li], new_v[li], dev_status=status)

    def attend(li):
        if fused:
            q8.decode_step_partial(pools[li], batch_p, nq, new_k[li], new_v[li], qs[li], scale, outs[li], ws,
                                   nparts=call_parts, dev_status=status)
        else:
            partial(pools[li], batch_p, nq, qs[li], scale, outs[li], ws, nparts=call_parts, dev_status=status)

    def step_plain():
        make_plan()
        for li in range(layers):
            append(li)
            attend(li)
            merge(pools[li], batch_p, nq, qs[li], scale, outs[li], ws, nparts=call_parts, dev_status=status)

    # ---- timed region 1: whole steps (HIP graph replays unless eager).  A
    # graph holds graph_steps consecutive steps: a step of one small layer
    # takes less GPU time than the host needs to launch a replay, and one
    # step per replay would time the host instead of the GPU.
    graph = None
    copies = 1
    if not eager:
        copies = graph_steps(layers)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step_plain()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(copies):
                step_plain()
    run = graph.replay if graph is not None else step_plain
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    steps_timed = steps * copies
    assert int(status.item()) == 0, "device status set during timing"

    # ---- timed region 2: eager launches with HIP events around each kernel on
    # the stream the library launches on (the roofline's per-kernel durations)
    stream = torch.cuda.current_stream()
    ev_steps = max(2, min(steps, 5))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(ev_steps * layers)]
    ahead = HostAhead(torch)
    for s_ in range(ev_steps + 1):
        ahead.start(s_ > 0)
        make_plan()
        for li in range(layers):
            e = ev[(s_ - 1) * layers + li] if s_ > 0 else None   # first pass is a warm-up
            if e: e[0].record(stream)
            append(li)
            if e: e[1].record(stream)
            attend(li)
            if e: e[2].record(stream)
            merge(pools[li], batch_p, nq, qs[li], scale, outs[li], ws, nparts=call_parts, dev_status=status)
            if e: e[3].record(stream)
        ahead.stop()
    torch.cuda.synchronize()
    t_append = np.array([e[0].elapsed_time(e[1]) for e in ev]) * 1e3     # us
    t_partial = np.array([e[1].elapsed_time(e[2]) for e in ev]) * 1e3
    t_merge = np.array([e[2].elapsed_time(e[3]) for e in ev]) * 1e3
    t_layer = np.array([e[0].elapsed_time(e[3]) for e in ev]) * 1e3

    attn_b, app_b = algorithmic_bytes(w, lens, kv_bs, path, topk)
    ms_per_step = wall * 1e3 / steps_timed
    del pools, outs, qs, new_k, new_v, ws, plan
    return {
        "lens": lens, "table": table, "nblocks": nblocks, "nparts": nparts, "layers": layers,
        "ms_per_step": ms_per_step, "attn_bytes": attn_b, "append_bytes": app_b,
        "t_append": t_append, "t_partial": t_partial, "t_merge": t_merge, "t_layer": t_layer,
        "graph": graph is not None, "graph_steps": copies, "setup_s": setup_s, "fused": fused, "planned": planned,
        "invariant": invariant,
    }


class HostAhead:
    """Keeps the GPU on a bounded spin kernel (torch.cuda._sleep) while the
    host enqueues one event-timed step, so the events around each kernel
    bracket GPU time only: for a small kernel the host's per-call argument
    checks and launch take longer than the kernel itself, and without a head
    start the GPU would wait for the host between two events.  The spin is
    sized from the host's enqueue time of the untimed first pass."""

    def __init__(self, torch):
        self.torch = torch
        torch.cuda._sleep(1000)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 2_000_000
        e0.record()
        torch.cuda._sleep(n)
        e1.record()
        torch.cuda.synchronize()
        self.cycles_per_us = n / max(1e-3, e0.elapsed_time(e1) * 1e3)
        self.host_us = 0.0
        self.t = 0.0

    def start(self, timed: bool):
        if timed and self.host_us > 0:
            self.torch.cuda._sleep(int(min(1.5 * self.host_us + 50.0, 200_000.0) * self.cycles_per_us))
        self.t = time.perf_counter()

    def stop(self):
        self.host_us = max(self.host_us, (time.perf_counter() - self.t) * 1e6)


def graph_steps(layers: int) -> int:
    """Decode steps per captured graph: 32 layer-steps or more per replay."""
    return max(1, 32 // max(1, layers))


def prefill_flops(w: workloads.Workload, lens: np.ndarray) -> int:
    """Algorithmic flops of one layer's prefill attention: for every query row
    at position p and query head, p + 1 keys, each 128 multiply-adds for the
    score and 128 for the weighted V (2 flops per multiply-add)."""
    nb = w.append_per_step
    n = lens.astype(np.int64)
    keys = nb * (n - nb) + nb * (nb + 1) // 2   # sum over the new rows of (p + 1)
    return int(keys.sum()) * w.nq * 4 * w.head_dim


def measure_prefill(torch, q8, dev, w, layers, steps, warmup, eager=False):
    """A prefill step: per layer, append the workload's new tokens (the last
    append_per_step positions of every sequence) and run q8_prefill_attn over
    them.  Same structure as measure(): whole steps as one HIP graph, then an
    eager pass with HIP events around each kernel."""
    lens = workloads.seq_lens(w)
    nb = w.append_per_step
    assert nb > 1 and np.all(lens >= nb), "not a prefill workload"
    kv_bs = w.kv_bs
    B, nq, nkv, hd = w.batch, w.nq, w.nkv, w.head_dim
    scale = float(workloads.softmax_scale(hd))
    t_setup = time.perf_counter()
    table, nblocks = workloads.block_table(lens, kv_bs, w.seed)
    table_t = torch.from_numpy(table).to(dev)
    lens_t = torch.from_numpy(lens).to(dev)
    batch = q8.make_batch(table_t, lens_t, int(lens.max()))
    pools = [q8.alloc_layer(nblocks, kv_bs, nkv, dev) for _ in range(layers)]
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    # history (positions below n_b - nb) from a source pool, as in measure()
    hist = [(b, n - nb) for b, n in enumerate(lens) if n > nb]
    if hist:
        src_k = workloads.kv_pool_torch(w, POOL_TOKENS + FILL_CHUNK, gen, dev)
        src_v = workloads.kv_pool_torch(w, POOL_TOKENS + FILL_CHUNK, gen, dev)
        hist_seq = torch.from_numpy(np.concatenate([np.full(h, b, np.int32) for b, h in hist])).to(dev)
        hist_pos = torch.from_numpy(np.concatenate([np.arange(h, dtype=np.int32) for _, h in hist])).to(dev)
        rng = np.random.default_rng(w.seed)
        for pool in pools:
            for c0 in range(0, hist_seq.numel(), FILL_CHUNK):
                c1 = min(hist_seq.numel(), c0 + FILL_CHUNK)
                off = int(rng.integers(0, POOL_TOKENS))
                q8.kv_append(pool, batch, hist_seq[c0:c1], hist_pos[c0:c1], src_k[off:off + c1 - c0],
                             src_v[off:off + c1 - c0], dev_status=status)
        del src_k, src_v
    T = B * nb
    new_seq = torch.from_numpy(np.repeat(np.arange(B, dtype=np.int32), nb)).to(dev)
    new_pos = torch.from_numpy(np.concatenate([np.arange(n - nb, n, dtype=np.int32) for n in lens])).to(dev)
    q_start = torch.from_numpy((np.arange(B + 1) * nb).astype(np.int32)).to(dev)
    new_k = torch.randn((layers, T, nkv, hd), generator=gen, device=dev)
    new_v = torch.randn((layers, T, nkv, hd), generator=gen, device=dev)
    qs = torch.randn((layers, T, nq, hd), generator=gen, device=dev)
    outs = torch.empty((layers, T, nq, hd), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "device status set during fill"
    setup_s = time.perf_counter() - t_setup

    def step_plain():
        for li in range(layers):
            q8.kv_append(pools[li], batch, new_seq, new_pos, new_k[li], new_v[li], dev_status=status)
            q8.prefill_attn(pools[li], batch, nq, q_start, nb, qs[li], scale, outs[li], dev_status=status)

    graph = None
    if not eager:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step_plain()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step_plain()
    run = graph.replay if graph is not None else step_plain
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert int(status.item()) == 0, "device status set during timing"

    stream = torch.cuda.current_stream()
    ev_steps = max(2, min(steps, 5))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(ev_steps * layers)]
    ahead = HostAhead(torch)
    for s_ in range(ev_steps + 1):
        ahead.start(s_ > 0)
        for li in range(layers):
            e = ev[(s_ - 1) * layers + li] if s_ > 0 else None
            if e: e[0].record(stream)
            q8.kv_append(pools[li], batch, new_seq, new_pos, new_k[li], new_v[li], dev_status=status)
            if e: e[1].record(stream)
            q8.prefill_attn(pools[li], batch, nq, q_start, nb, qs[li], scale, outs[li], dev_status=status)
            if e: e[2].record(stream)
        ahead.stop()
    torch.cuda.synchronize()
    t_append = np.array([e[0].elapsed_time(e[1]) for e in ev]) * 1e3
    t_prefill = np.array([e[1].elapsed_time(e[2]) for e in ev]) * 1e3
    del pools, outs, qs, new_k, new_v
    return {"lens": lens, "table": table, "nblocks": nblocks, "layers": layers, "ms_per_step": wall * 1e3 / steps,
            "t_append": t_append, "t_prefill": t_prefill, "graph": graph is not None, "setup_s": setup_s}


def prefill_cpu_baseline(w, lens):
    """The oracle's prefill on a bounded sample: the first sequence's first
    rows (positions from n - nb on) of one layer, all query heads, repeated
    for ~10 s; in algorithmic TFLOP/s."""
    import oracle
    nb = w.append_per_step
    n = int(lens[0])
    rows = min(nb, 256)
    sample_len = n - nb + rows   # a cache holding the history and the sampled rows
    rng = np.random.default_rng(w.seed)
    k = rng.standard_normal((1, sample_len, w.nkv, w.head_dim), dtype=np.float32)
    v = rng.standard_normal((1, sample_len, w.nkv, w.head_dim), dtype=np.float32)
    q = rng.standard_normal((rows, w.nq, w.head_dim), dtype=np.float32)
    tab, nbl = workloads.block_table(np.array([sample_len], np.int32), w.kv_bs, w.seed)
    cache = oracle.build_cache(k, v, np.array([sample_len], np.int32), tab, nbl, w.kv_bs)
    threads, host = oracle_threads(oracle)
    keys = rows * (sample_len - rows) + rows * (rows + 1) // 2
    flops = keys * w.nq * 4 * w.head_dim
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.prefill_attn(cache, q, [0, rows], w.nq, float(workloads.softmax_scale(w.head_dim)), nthreads=threads)
        reps += 1
        if time.perf_counter() - t0 > 10.0:
            break
    dt = time.perf_counter() - t0
    return {"value": round(flops * reps / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} query rows at positions {n - nb}..{n - nb + rows - 1} of one sequence, all "
                      f"{w.nq} query heads, one layer, oracle prefill_attn repeated {reps}x in {dt:.1f} s", **host}


def prefill_main(args, torch, q8, dev):
    w = workloads.WORKLOADS[args.workload]
    layers = args.layers or w.layers
    m = measure_prefill(torch, q8, dev, w, layers, args.steps, args.warmup, args.eager)
    lens = m["lens"]
    flops = prefill_flops(w, lens)
    ms = m["ms_per_step"]
    value = layers * flops / (ms * 1e-3) / 1e12
    pre_us = float(m["t_prefill"].mean())
    achieved = flops / (pre_us * 1e-6) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": "q8_prefill_kernel", "kernel_us": round(pre_us, 2), "algorithmic_flops_per_launch": flops}
    cpu = None if args.no_cpu_baseline else prefill_cpu_baseline(w, lens)
    line = {
        "metric": "q8 prefill-attn achieved TFLOP/s (algorithmic: 4 * 128 flops per query head and visible key)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8/bf16x3/fp32", "data": "synthetic",
        "config": {
            "workload": w.name, "path": "prefill", "batch": w.batch, "nq_heads": w.nq, "nkv_heads": w.nkv,
            "head_dim": w.head_dim, "kv_bs": w.kv_bs, "layers": layers, "ctx": list(w.lens),
            "new_tokens_per_seq": w.append_per_step,
            "us_per_layer_step": round(ms * 1e3 / layers, 2),
            "us_append": round(float(np.median(m["t_append"])), 2),
            "us_prefill": round(float(np.median(m["t_prefill"])), 2),
            "flops_per_layer": flops, "graph": m["graph"], "setup_s": round(m["setup_s"], 1),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def sweep_entry(w, m):
    step_bytes = m["layers"] * (m["attn_bytes"] + m["append_bytes"])
    gbs = step_bytes / (m["ms_per_step"] * 1e-3) / 1e9
    part_us = float(m["t_partial"].mean())
    part_b = m["attn_bytes"] + (m["append_bytes"] if m["fused"] else 0)
    return {
        "workload": w.name, "batch": w.batch, "nq_heads": w.nq, "nkv_heads": w.nkv, "ctx": list(w.lens),
        "layers": m["layers"], "nparts": m["nparts"],
        "us_per_layer_step": round(m["ms_per_step"] * 1e3 / m["layers"], 2),
        "GBps": round(gbs, 1), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "us_decode_partial": round(float(np.median(m["t_partial"])), 2),
        "partial_GBps": round(part_b / (part_us * 1e-6) / 1e9, 1),
        "us_decode_merge": round(float(np.median(m["t_merge"])), 2),
        "us_append": None if m["fused"] else round(float(np.median(m["t_append"])), 2),
    }


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(each GPU would run the same kernels on its own share of sequences or KV heads). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import decode_attention_int8_kv_amd as q8

    q8.lib()   # raises if the HIP library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        copy_probe(torch, dev, args.copy_probe, args.steps)
        return
    if args.read_probe:
        read_probe(torch, q8, dev, args.read_probe, args.steps, args.warmup)
        return
    if args.issue_probe:
        issue_probe(torch, q8, dev, args.steps, args.warmup)
        return
    w = workloads.WORKLOADS[args.workload]
    if args.path == "prefill":
        if w.append_per_step <= 1:
            raise SystemExit("--path prefill needs a prefill workload (qwen2b_prefill_*)")
        prefill_main(args, torch, q8, dev)
        return
    if w.append_per_step > 1:
        raise SystemExit(f"{w.name} is a prefill workload: use --path prefill")
    layers = args.layers or w.layers
    fused = args.append == "fused" and args.path == "q8"
    m = measure(torch, q8, dev, w, layers, args.steps, args.warmup, args.nparts, args.eager, args.path, args.topk,
                fused, not args.no_plan, args.invariant)
    lens = m["lens"]
    B, nq, nkv, hd, kv_bs = w.batch, w.nq, w.nkv, w.head_dim, w.kv_bs
    attn_b, app_b = m["attn_bytes"], m["append_bytes"]
    step_bytes = layers * (attn_b + app_b)
    ms_per_step = m["ms_per_step"]
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    t_partial, t_merge, t_append, t_layer = m["t_partial"], m["t_merge"], m["t_append"], m["t_layer"]

    # dominant kernel: the decode partial kernel; its algorithmic bytes are the
    # attention bytes, plus the append's when it appends too (the merge traffic
    # is overhead and not counted)
    part_us = float(t_partial.mean())
    part_b = attn_b + (app_b if fused else 0)
    achieved = part_b / (part_us * 1e-6) / 1e9
    traffic = None
    if os.path.exists(args.traffic) and args.path == "q8":
        with open(args.traffic) as f:
            tr = json.load(f).get(args.workload)
        if tr and tr.get("kernel_hash") == kernel_hash():
            traffic = tr.get("bytes_per_launch")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": {"f32": "q8_attn_f32_partial_kernel", "sparse": "q8_sparse_probe_kernel + q8_sparse_attend_kernel"}.get(
                    args.path, "q8_attn_partial_kernel"),
                "kernel_us": round(part_us, 2),
                "algorithmic_bytes_per_launch": int(part_b)}

    sweep = None
    if not args.no_sweep and args.path == "q8":
        sweep = []
        for name in SWEEP:
            if name == args.workload:
                continue
            ws_ = workloads.WORKLOADS[name]
            sweep.append(sweep_entry(ws_, measure(torch, q8, dev, ws_, ws_.layers, 10, 2, 0, args.eager,
                                                  fused=fused, planned=not args.no_plan, invariant=args.invariant)))
            torch.cuda.empty_cache()
            print(f"[sweep] {name} done", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline and args.path == "q8":
        cpu = cpu_baseline(w, lens, m["table"], m["nblocks"], attn_b)

    line = {
        "metric": "q8 decode-attn achieved HBM GB/s (% of peak) + us/layer-step, batch x ctx sweep",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp32" if args.path == "f32" else "int8/fp32", "data": "synthetic",
        "config": {
            "workload": w.name, "path": args.path, "topk": args.topk if args.path == "sparse" else None,
            "append": "fused" if fused else "separate", "step_plan": m["planned"], "batch_invariant": m["invariant"],
            "batch": B, "nq_heads": nq, "nkv_heads": nkv, "head_dim": hd, "kv_bs": kv_bs,
            "layers": layers, "ctx": list(w.lens), "ctx_mean": float(lens.mean()), "nparts": m["nparts"],
            "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
            "us_per_layer_step": round(ms_per_step * 1e3 / layers, 2),
            "us_per_layer_step_eager_p10_p50_p90": [round(float(np.percentile(t_layer, q)), 2) for q in (10, 50, 90)],
            "us_append": None if fused else round(float(np.median(t_append)), 2),
            "us_decode_partial": round(float(np.median(t_partial)), 2),
            "us_decode_merge": round(float(np.median(t_merge)), 2),
            "graph": m["graph"], "graph_steps": m["graph_steps"],
            "bytes_per_layer_step": int(attn_b + app_b), "setup_s": round(m["setup_s"], 1),
            "sweep": sweep,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def copy_probe(torch, dev, mib, reps):
    """A plain device-to-device copy of a known size, so hardware byte counters
    can be scaled: FETCH_SIZE and WRITE_SIZE of one copy should read mib MiB."""
    src = torch.ones(mib * 2 ** 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": mib * 2 ** 20, "reps": reps}), flush=True)


def read_probe(torch, q8, dev, mib, reps, warmup):
    """The read ceiling: q8_stream_read over a buffer of `mib` MiB (larger
    than the 256 MB last-level cache, so every launch reads HBM), plain and
    non-temporal loads, over 256 / 512 / 1024 workgroups; `reps` launches per
    setting timed with HIP events on the library's stream (mean)."""
    buf = torch.ones(mib * 2 ** 20, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    reps = max(reps, 3)
    res = {}
    for nt in (0, 1):
        for wg in (256, 512, 1024):
            for _ in range(max(warmup, 1)):
                q8.stream_read(buf, wg, nt, sink)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            ev[0].record(stream)
            for i in range(reps):
                q8.stream_read(buf, wg, nt, sink)
                ev[i + 1].record(stream)
            torch.cuda.synchronize()
            us = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]) * 1e3
            res[f"{'nt' if nt else 'plain'}_wg{wg}"] = {"us_mean": round(float(us.mean()), 2),
                                                         "GBps": round(buf.numel() / (us.mean() * 1e-6) / 1e9, 1)}
    best = max(res.values(), key=lambda r: r["GBps"])
    print(json.dumps({"read_probe_bytes": buf.numel(), "reps": reps, "results": res,
                      "best_GBps": best["GBps"], "best_pct_of_hbm_peak": round(100 * best["GBps"] / HBM_PEAK_GBS, 2)}),
          flush=True)


def issue_probe(torch, q8, dev, reps, warmup):
    """Instruction issue on the CUs (q8_issue_probe, one workgroup per CU):
    cycles at 2.4 GHz per launch for each mode, and the cycles per VALU FMA
    and per matrix-core product of one wave that they imply."""
    wg, vit, mit = 256, 4096, 512
    out = torch.empty(wg * 1024, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    reps = max(reps, 3)
    names = ["1 VALU wave per SIMD", "1 matrix-core wave per SIMD", "1 VALU + 1 matrix-core wave per SIMD",
             "2 VALU waves per SIMD", "4 VALU waves per SIMD"]
    res = {}
    for mode in range(5):
        for _ in range(max(warmup, 1)):
            q8.issue_probe(out, mode, vit, mit, wg)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for i in range(reps):
            q8.issue_probe(out, mode, vit, mit, wg)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        us = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])) * 1e3
        res[names[mode]] = {"us": round(us, 2), "cycles": round(us * 2400.0)}
    fma = vit * 8   # FMAs per VALU wave
    mm = mit * 4    # products per matrix-core wave
    c = [res[n]["cycles"] for n in names]
    print(json.dumps({"issue_probe": res, "valu_fmas_per_wave": fma, "mfma_products_per_wave": mm,
                      "cycles_per_fma_one_wave": round(c[0] / fma, 2),
                      "cycles_per_fma_per_simd_two_waves": round(c[3] / (2 * fma), 2),
                      "cycles_per_fma_per_simd_four_waves": round(c[4] / (4 * fma), 2),
                      "cycles_per_product_one_wave": round(c[1] / mm, 2),
                      "both_over_valu_alone": round(c[2] / c[0], 3)}), flush=True)


# the sources that define the q8 decode partial kernel and its launch plan
KERNEL_SOURCES = ("q8kv_decode.hip", "q8kv_device.hpp", "q8kv_plan.hpp", "q8kv_ranges.hpp", "q8kv_tile.hpp")


def _code_only(text: str) -> str:
    """Source text with comments removed and white space collapsed."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_hash() -> str:
    """Hash of the code (comments and layout ignored) of the q8 decode
    kernel's sources: counter figures taken on other code are stale."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_attention_int8_kv_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def cpu_baseline(w, lens, table, nblocks, attn_bytes):
    """The CPU oracle, as it stands, on a bounded sample of one layer-step of
    the workload: the first sequences up to ~96K tokens, every query head.
    Their K/V are N(0,1) rows drawn on the host and quantized by the oracle's
    own quantizer.  The oracle decode is repeated until ~10 s have passed;
    returns GB/s of the same algorithmic attention bytes."""
    import oracle
    threads, host = oracle_threads(oracle)
    keep = np.cumsum(lens) <= 98304
    keep[0] = True
    sl = lens[keep]
    sub = workloads.Workload(w.name, w.nq, w.nkv, int(keep.sum()), 1, ("fixed", int(sl.max())), w.dist, w.seed)
    t0 = time.perf_counter()
    k, v = workloads.kv_host(sub, sl)
    tab, nb = workloads.block_table(sl, w.kv_bs, w.seed)
    cache = oracle.build_cache(k, v, sl, tab, nb, w.kv_bs)
    del k, v
    q = workloads.query(sub)
    print(f"[cpu_baseline] sample ready in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.decode_attn(cache, q, w.nq, float(workloads.softmax_scale(w.head_dim)), nthreads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or reps >= 20000:
            break
    n = sl.astype(np.int64)
    b = int(n.sum()) * w.nkv * (2 * w.head_dim + 8) + sub.batch * w.nq * w.head_dim * 8
    return {"value": round(b * reps / dt / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{sub.batch} of {w.batch} sequences ({int(n.sum())} tokens, all {w.nq} query heads) "
                      f"of one layer-step, oracle decode_attn repeated {reps}x in {dt:.1f} s", **host}


def oracle_threads(oracle):
    """Threads for the CPU baseline: every thread this job may use -- the
    OpenMP thread count (OMP_NUM_THREADS, which the GPU host sets to the CPU
    share it gives a one-GPU job), else the CPUs in this process's affinity
    mask -- and a record of what the host reports."""
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    omp = os.environ.get("OMP_NUM_THREADS")
    threads = oracle.threads_available() if omp else aff
    return threads, {"nproc": os.cpu_count(), "affinity_cpus": aff, "omp_num_threads": omp}


if __name__ == "__main__":
    main()
