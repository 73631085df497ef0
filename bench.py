"""Decode throughput of the DeltaLog path on one MI355X.

One step = one dl_decode_step over every (sequence, head) tile of the
workload: base + log reads, output, append, and the fold on steps that fill
the log.  Default workload: GDN, batch 64, 32 heads, dk = dv = 128, L = 16,
all logs starting empty, inputs resident in HBM (a pool of 64 drawn steps,
cycled).  Prints one JSON line.

The headline is cache-cold: independent pools of the workload's shape are used
in turn (three for this one, 480 MB), more than the 256 MiB last-level cache
holds, so each step reads its state from HBM as a model with several layers
does.  The timed steps are a whole number of fold periods of every pool; the
headline is the median of --repeats (5) such timed windows, all listed.

Also measured in the same run: the same step on one pool (its working set can
stay in the last-level cache: reported as cache-resident), the eager comparator
(dl_eager_step, read and write the whole state every step) on the same inputs,
cold and cache-resident, read ceilings over the same pools (a torch sum over
1 GiB; the probes of libdlprobe.so: one workgroup per tile reading it, with its
log, or writing it back, and persistent workgroups streaming the same bytes
through LDS), plain copies,
dl_prefill of a long prompt, dl_merge_on on full logs with each arithmetic unit
of the fold, and the fp64 CPU oracle on the host cores.

  python bench.py [--gpus 1] [--steps 1024] [--warmup 32] [--workload 2]
                  [--no-cpu-baseline] [--graph]
                  [--only deltalog|warm|eager|ceiling|copy|prefill|merge]
                  [--base-dtype f32|bf16] [--log-len L] [--trace]

`--only merge` times dl_merge_on on full logs with each arithmetic unit of the
fold (vector FMAs, fp32 MFMA) and prints their times.

`--trace` runs the cache-cold leg on the tracing build (libdeltalog_trace.so, made
by `python -m linear_attention_recurrent_amd.build --trace`) and prints, for two
consecutive launches at half-full logs and two that fold, each workgroup's phase
times and the launch's timeline (span, start spread, gap between the launches).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from inputs import VARIANT_NAMES, WORKLOADS, make_inputs  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD's published figure
MALL_BYTES = 256 << 20  # MI355X last-level (Infinity) cache
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["linear_attention_recurrent_amd/csrc/decode.hip",
                  "linear_attention_recurrent_amd/csrc/dl_device.hpp"]


# ------------------------------------------------------------ byte model ----
def entry_bytes(variant: int, dk: int, dv: int) -> int:
    """Bytes of one log entry: key (bf16), factor (fp32; RWKV6: v in bf16), cumulative decay."""
    if variant == 0:
        return 2 * dk + 4 * dv + 4
    if variant == 1:
        return 2 * dk + 4 * dv + 4 * dk
    return 2 * dk + 2 * dv + 4 * dk


def input_bytes(variant: int, dk: int, dv: int, batch: int) -> float:
    """q, k, v (bf16), decay, beta (fp32) per state-step; RWKV6's bonus is per head."""
    b = 2 * dk * 2 + 2 * dv
    if variant == 0:
        b += 4 + 4
    elif variant == 1:
        b += 4 * dk + 4
    else:
        b += 4 * dk + 4 * dk / batch
    return b


def deltalog_bytes_per_state_step(variant, dk, dv, L, batch, base_bytes=4) -> dict:
    """Algorithmic HBM bytes per (sequence, head, token), averaged over a period of L steps.
    base_bytes: 4 for the fp32 base, 2 for the bf16 base."""
    E = entry_bytes(variant, dk, dv)
    state = base_bytes * dk * dv
    parts = dict(
        base_read=state,
        inputs=input_bytes(variant, dk, dv, batch),
        log_read=(L - 1) / 2 * E,           # the n entries present, n uniform over 0..L-1
        fill=8,
        output=4 * dv,
        append=(L - 1) / L * E,             # every step but the folding one
        fold_write=state / L,               # the folding step rewrites the base
    )
    parts["total"] = sum(parts.values())
    parts["state_writes"] = parts["append"] + parts["fold_write"]
    return parts


def eager_bytes_per_state_step(variant, dk, dv, batch) -> dict:
    state = 4 * dk * dv
    parts = dict(state_read=state, state_write=state, inputs=input_bytes(variant, dk, dv, batch), output=4 * dv)
    parts["total"] = sum(parts.values())
    parts["state_writes"] = state
    return parts


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_profile_name(workload_name: str, bf16_base: bool, log_len=None) -> str:
    tag = "" if log_len is None else f"_L{log_len}"
    return f"decode_{workload_name}{tag}{'_bf16base' if bf16_base else ''}_counters.txt"


PREFILL_SOURCES = ["linear_attention_recurrent_amd/csrc/prefill.hip",
                   "linear_attention_recurrent_amd/csrc/dl_device.hpp"]


def prefill_source_hash() -> str:
    h = hashlib.sha256()
    for rel in PREFILL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _read_kv(path):
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    return vals


def read_prefill_counters(workload_name: str, tokens: int):
    """HBM bytes per prefill launch from the committed counter summary, if it was taken on
    the current kernel source at this prompt length (else None)."""
    path = os.path.join(PROFILE_DIR, f"prefill_{workload_name}_T{tokens}_counters.txt")
    if not os.path.exists(path):
        return None
    vals = _read_kv(path)
    return vals if vals.get("kernel_source_sha256") == prefill_source_hash() else None


def read_counter_profile(workload_name: str, bf16_base: bool = False, log_len=None):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source (else None)."""
    path = os.path.join(PROFILE_DIR, counter_profile_name(workload_name, bf16_base, log_len))
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return vals


# ----------------------------------------------------------- CPU baseline ---
_CPU_JOB = {}


def _cpu_worker(i, barrier, queue):
    import oracle  # the fp64 oracle, timed as it stands
    job = _CPU_JOB
    barrier.wait()
    t0 = time.perf_counter()
    oracle.run_eager(job["inp"], job["steps"], sel=job["chunks"][i], keep_outputs=False)
    queue.put((i, time.perf_counter() - t0, len(job["chunks"][i]) * job["steps"]))


def cpu_baseline(workload: int, target_s: float = 25.0) -> dict:
    """Time the fp64 eager oracle on the host cores over a bounded sample of the workload.

    The inputs are drawn once in this process; forked workers (one per core, at
    most 16) each run the oracle on a contiguous share of the tiles, starting
    together at a barrier.  Throughput = all tile-steps / the slowest worker's time.
    """
    import multiprocessing as mp

    import oracle
    w = WORKLOADS[workload]
    B, H = w["batch"], w["heads"]
    cores = min(len(os.sched_getaffinity(0)), 16)
    probe = make_inputs(workload, 2, pool=2, batch=1, heads=min(H, 8))
    sel = [(0, h) for h in range(probe.heads)]
    t0 = time.perf_counter()
    oracle.run_eager(probe, 2, sel=sel, keep_outputs=False)
    per = (time.perf_counter() - t0) / (2 * len(sel))          # seconds per tile-step, one core
    all_tiles = [(b, h) for b in range(B) for h in range(H)]
    steps = int(min(4096, max(2, target_s * cores / (per * len(all_tiles)))))
    per_core = (len(all_tiles) + cores - 1) // cores
    _CPU_JOB.update(inp=make_inputs(workload, steps, pool=min(steps, 64)), steps=steps,
                    chunks=[all_tiles[i * per_core:(i + 1) * per_core] for i in range(cores)])
    ctx = mp.get_context("fork")
    barrier, queue = ctx.Barrier(cores), ctx.Queue()
    procs = [ctx.Process(target=_cpu_worker, args=(i, barrier, queue)) for i in range(cores)]
    for p in procs:
        p.start()
    res = [queue.get() for _ in procs]
    for p in procs:
        p.join()
    wall = max(r[1] for r in res)
    work = sum(r[2] for r in res)
    rates = sorted(r[2] / r[1] for r in res)  # one core each, all cores busy
    _CPU_JOB.clear()
    return {"value": work / wall, "unit": "state-steps/s", "cores": cores, "kind": "oracle",
            "single_core_value": rates[len(rates) // 2],
            "sample": f"fp64 NumPy eager oracle on the same workload: {steps} steps (inputs cycling "
                      f"over 64 drawn steps) x all {B}x{H} tiles, tiles split over {cores} forked "
                      f"single-threaded workers, {wall:.1f} s (slowest worker; input drawing not timed); "
                      f"single_core_value: the median worker's own rate"}


# -------------------------------------------------------------- GPU legs ----
def gpu_setup(workload, pool_slots, log_len=None, dk=None, dv=None):
    import torch

    from linear_attention_recurrent_amd import deltalog as dl
    w = WORKLOADS[workload]
    inp = make_inputs(workload, pool_slots, pool=pool_slots, log_len=log_len, dk=dk, dv=dv)
    dev = torch.device("cuda", 0)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    T = dict(q=bf(inp.q), k=bf(inp.k), v=bf(inp.v), decay=torch.from_numpy(inp.decay).to(dev),
             beta=None if inp.beta is None else torch.from_numpy(inp.beta).to(dev),
             bonus=None if inp.bonus is None else torch.from_numpy(inp.bonus).to(dev),
             s0=torch.from_numpy(inp.s0).to(dev),
             out=torch.empty((inp.batch, inp.heads, inp.dv), dtype=torch.float32, device=dev))
    T["eta"] = None if inp.eta is None else torch.from_numpy(inp.eta).to(dev)
    ios = [dl.make_step_io(inp.variant, inp.batch, inp.heads, inp.dk, inp.dv, dev, T["q"][p], T["k"][p],
                           T["v"][p], T["decay"][p], None if T["beta"] is None else T["beta"][p],
                           T["bonus"], T["out"], None if T["eta"] is None else T["eta"][p], inp.eps)
           for p in range(pool_slots)]
    return inp, T, ios, w


def time_loop(fn, steps, warmup, graph_chunk=0):
    """Run fn(t) for warmup untimed steps then `steps` timed ones; returns seconds (events)."""
    import torch
    for t in range(warmup):
        fn(t)
    torch.cuda.synchronize()
    if graph_chunk:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for t in range(graph_chunk):
                    fn(warmup + t)
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    if graph_chunk:
        for _ in range(steps // graph_chunk):
            g.replay()
    else:
        for t in range(steps):
            fn(warmup + t)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3


def read_ceilings(pools, tiles, tile_bytes, log_bytes, launches):
    """Memory rates on this machine for the decode step's access shapes, in the same run: a
    torch sum over 1 GiB, and the probes of libdlprobe.so (one workgroup per tile, every
    load issued first, no arithmetic) over the base tensors of `pools`, used in turn as the
    decode step uses them: the tile read alone, the tile read plus `log_bytes` of log per
    tile (the mean the step reads), the tile read and written back (the eager step's
    traffic), the same bytes read as 16 KiB blocks by one workgroup each (tiles larger
    than that), and the same bytes streamed through LDS by one persistent workgroup per
    CU with three 16 KiB units in flight.  For 128 x 128 fp32 tiles also the owned stream:
    persistent workgroups that each own whole tiles, as a decode step does, one wave
    streaming their units into LDS and four forming the column sums (tiles strided over the
    workgroups, the same with each tile's units in a rotated order, or a contiguous run of
    tiles per workgroup), and the same kernel taking the units in the stream's order; and
    one workgroup per 16 KiB quarter tile storing its partial column sums, without and with
    their sum per tile inside the launch (agent-scope fences and a count)."""
    import ctypes

    import torch
    dev = torch.device("cuda", 0)
    out = {}
    x = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
    secs = time_loop(lambda t: x.sum(), 10, 3)
    out["torch_sum_gbs"] = (1 << 30) * 10 / secs / 1e9
    del x
    if not pools:
        return out
    lib = ctypes.CDLL(os.path.join(ROOT, "linear_attention_recurrent_amd", "libdlprobe.so"))
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.dl_probe_tile_read.argtypes = [vp, ci, ci, vp, vp]
    lib.dl_probe_tile_read_log.argtypes = [vp, ci, ci, vp, ci, ci, vp, vp]
    lib.dl_probe_tile_rw.argtypes = [vp, ci, ci, vp]
    lib.dl_probe_tile_stream.argtypes = [vp, ci, ci, vp, vp]
    lib.dl_probe_owned_stream.argtypes = [vp, ci, ci, vp, ci, vp]
    lib.dl_probe_quarter_split.argtypes = [vp, ci, ci, vp, vp, vp, vp]
    sink = torch.zeros(256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    NP = len(pools)
    lb = min(65536, -(-int(log_bytes) // 16) * 16)
    logs = [torch.zeros(tiles * lb // 4 + 4, dtype=torch.float32, device=dev) for _ in range(NP)]

    def check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed ({rc})")
    legs = {
        "tile_read": (lambda t: check(lib.dl_probe_tile_read(pools[t % NP].base.data_ptr(), tile_bytes, tiles,
                                                             sink.data_ptr(), stream), "dl_probe_tile_read"),
                      tile_bytes * tiles),
        "tile_read_log": (lambda t: check(lib.dl_probe_tile_read_log(pools[t % NP].base.data_ptr(), tile_bytes, tiles,
                                                                     logs[t % NP].data_ptr(), lb, lb, sink.data_ptr(),
                                                                     stream), "dl_probe_tile_read_log"),
                          (tile_bytes + lb) * tiles),
        "tile_rw": (lambda t: check(lib.dl_probe_tile_rw(pools[t % NP].base.data_ptr(), tile_bytes, tiles, stream),
                                    "dl_probe_tile_rw"), 2 * tile_bytes * tiles),
        # the same bytes as 16 KiB units streamed through LDS by one persistent workgroup per
        # CU, three units in flight
        "tile_stream": (lambda t: check(lib.dl_probe_tile_stream(pools[t % NP].base.data_ptr(),
                                                                 tile_bytes * tiles // 16384, 256, sink.data_ptr(),
                                                                 stream), "dl_probe_tile_stream"),
                        tile_bytes * tiles // 16384 * 16384),
    }
    if tile_bytes > 16384:  # the same bytes read as 16 KiB blocks, one workgroup each
        legs["block16k_read"] = (lambda t: check(lib.dl_probe_tile_read(pools[t % NP].base.data_ptr(), 16384,
                                                                         tiles * tile_bytes // 16384, sink.data_ptr(),
                                                                         stream), "dl_probe_tile_read"),
                                 tile_bytes * tiles)
    owned = tile_bytes == 65536 and tiles % 256 == 0 and pools[0].base.dtype == torch.float32
    if owned:  # 128 x 128 fp32 tiles: the tile-owning stream, and its unit order for comparison
        colsums = torch.empty(tiles * 128, dtype=torch.float32, device=dev)
        for order, name in ((0, "owned_stream"), (1, "owned_stream_unit_order"), (2, "owned_stream_rotated"),
                            (3, "owned_stream_contiguous")):
            legs[name] = (lambda t, o=order: check(lib.dl_probe_owned_stream(pools[t % NP].base.data_ptr(), tiles, o,
                                                                             colsums.data_ptr(), 256, stream),
                                                   "dl_probe_owned_stream"), tile_bytes * tiles)
        # one workgroup per 16 KiB quarter, in pool order; partial column sums stored, and
        # with the exchange added up per tile inside the launch behind agent-scope fences
        qpart = torch.empty(tiles * 4 * 256, dtype=torch.float32, device=dev)
        qcnt = torch.zeros(tiles, dtype=torch.int32, device=dev)
        qout = torch.empty(tiles * 256, dtype=torch.float32, device=dev)
        for ex, name in ((0, "quarter_split"), (1, "quarter_split_exchange")):
            legs[name] = (lambda t, e=ex: check(lib.dl_probe_quarter_split(pools[t % NP].base.data_ptr(), tiles, e,
                                                                           qpart.data_ptr(), qcnt.data_ptr(),
                                                                           qout.data_ptr(), stream),
                                                "dl_probe_quarter_split"), tile_bytes * tiles)
    for name, (fn, nbytes) in legs.items():
        secs = time_loop(fn, launches, 2 * NP)
        out[f"{name}_gbs"] = nbytes * launches / secs / 1e9
    out["probe_shape"] = (f"{tiles} tiles of {tile_bytes} B per launch, {NP} pools in turn; read_log adds {lb} B "
                          f"of log per tile; rw writes the tile back (the eager step's traffic); block16k_read "
                          f"reads the same bytes as 16 KiB blocks, one workgroup each; stream reads "
                          f"the same bytes as 16 KiB units with 256 persistent workgroups, three units in "
                          f"flight per CU through LDS"
                          + ("; owned_stream: 256 persistent workgroups owning whole tiles, one wave streaming "
                             "16 KiB units into LDS three ahead, four forming column sums; its unit_order leg "
                             "reads the pool's units in the stream's order, rotated starts each tile at unit "
                             "w mod 4, contiguous gives each workgroup a run of whole tiles; quarter_split: one "
                             "workgroup per 16 KiB quarter in pool order storing partial column sums, its "
                             "exchange leg adding each tile's four up inside the launch behind agent-scope "
                             "fences" if owned else ""))
    return out


TRACE_TICK_NS = 10.0  # s_memrealtime counts at 100 MHz


def trace_summary(buf, tiles: int) -> dict:
    """Timeline of two consecutive decode launches from the tracing build's stamps:
    buf[launch][workgroup] = (start, after the log-coefficient phase, after the column
    sums, end, hardware id)."""
    us = TRACE_TICK_NS / 1e3
    order = sorted(range(2), key=lambda i: int(buf[i, :, 0].min()))
    t0 = int(buf[order[0], :, 0].min())
    pct = lambda a, q: float(np.percentile(a, q)) * us
    launches = []
    for i in order:
        t = buf[i, :, :4].astype(np.int64) - t0
        ph = np.diff(t, axis=1)
        hw = buf[i, :, 4]
        cu = ((hw >> np.uint64(32)) << np.uint64(8)) | ((hw >> np.uint64(8)) & np.uint64(0xF)) << np.uint64(4) \
            | ((hw >> np.uint64(13)) & np.uint64(0x7)) << np.uint64(1) | ((hw >> np.uint64(12)) & np.uint64(0x1))
        launches.append({
            "start_us": float(t[:, 0].min()) * us, "end_us": float(t[:, 3].max()) * us,
            "span_us": float(t[:, 3].max() - t[:, 0].min()) * us,
            "start_spread_us": {"p50": pct(t[:, 0] - t[:, 0].min(), 50), "p90": pct(t[:, 0] - t[:, 0].min(), 90),
                                "max": float(t[:, 0].max() - t[:, 0].min()) * us},
            "workgroup_us": {"p50": pct(t[:, 3] - t[:, 0], 50), "p90": pct(t[:, 3] - t[:, 0], 90)},
            "phase_us_p50": {"log_coefficients": pct(ph[:, 0], 50), "column_sums": pct(ph[:, 1], 50),
                             "output_append_fold": pct(ph[:, 2], 50)},
            "phase_us_p90": {"log_coefficients": pct(ph[:, 0], 90), "column_sums": pct(ph[:, 1], 90),
                             "output_append_fold": pct(ph[:, 2], 90)},
            "compute_units_used": int(len(np.unique(cu))),
        })
    return {"launches": launches, "gap_us": launches[1]["start_us"] - launches[0]["end_us"],
            "workgroups_per_launch": tiles}


def trace_leg(args, inp, ios, base_dt) -> dict:
    """The cache-cold leg on the tracing build: warm up whole fold periods of every pool,
    then stop twice, after two launches at fill L/2 and after two that fold, and read the
    stamps of those two launches each time."""
    import ctypes

    import torch

    from linear_attention_recurrent_amd import build, deltalog as dl
    if not os.path.exists(build.TRACE_LIB):
        raise SystemExit(f"{build.TRACE_LIB} is not built: run `python -m linear_attention_recurrent_amd.build --trace`")
    lib = dl.load_library(build.TRACE_LIB, make_default=True)
    lib.dl_trace_copy.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.dl_trace_copy.restype = ctypes.c_int
    dev = torch.device("cuda", 0)
    B, H, dk, dv, L, var = inp.batch, inp.heads, inp.dk, inp.dv, inp.log_len, inp.variant
    tiles = B * H
    if tiles > 65536:
        raise SystemExit("--trace records at most 65,536 workgroups per launch")
    eb = 2 if base_dt == dl.BASE_BF16 else 4
    NP = 1 + -(-MALL_BYTES // (tiles * (eb * dk * dv + L * entry_bytes(var, dk, dv) + 4)))
    pools = [dl.DeltaLogPool(var, B, H, dk, dv, L, dev, base_dt) for _ in range(NP)]
    for p_ in pools:
        dl.dl_init_state(p_, torch.from_numpy(inp.s0).to(dev), inp.fill0)
    P = len(ios)
    t = 0

    def run_to(stop):
        nonlocal t
        while t < stop:
            dl.dl_decode_step(pools[t % NP], ios[t % P])
            t += 1
        torch.cuda.synchronize()
        buf = np.zeros((2, tiles, 5), dtype=np.uint64)
        rc = lib.dl_trace_copy(buf.ctypes.data, tiles)
        if rc != 0:
            raise RuntimeError(f"dl_trace_copy failed ({rc})")
        return trace_summary(buf, tiles)
    warm = NP * L * max(1, -(-args.warmup // (NP * L)))
    out = {"mid_log": run_to(warm + NP * (L // 2) + 2)}  # the last two launches: fill L/2
    out["fold"] = run_to(warm + 2 * NP * L)  # the last two launches: fill L - 1, they fold
    out["note"] = ("tracing build: each workgroup's thread 0 stamps s_memrealtime (100 MHz) at its start, "
                   "after the log-coefficient barrier, after the column-sum barrier and at its end; "
                   f"{NP} pools in turn (cache-cold), log length {L}")
    return out


BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, AMD's published figure
PREFILL_CHUNK = 32


def prefill_model(dk: int, dv: int, C: int = PREFILL_CHUNK, variant: int = 0) -> dict:
    """Per (sequence, head, prompt token): HBM bytes, the chunkwise method's flops (each
    product counted once, as the kernel orders them), and the bf16 MFMA flops the kernel
    issues: an exact bf16 operand against a two-way split one takes 2 products, two split
    operands 3, and the decay-weighted C x C products (KDA, RWKV6; three-way splits, the
    three lower 16 x 16 blocks) 6."""
    byts = 2 * dk * 2 + 2 * dv + 4 * (1 if variant == 0 else dk) + (4 if variant != 2 else 0) + 4 * dv
    lower = 3 * 16 * 16 * dk * 2  # flops of one decay-weighted product over the three lower blocks
    if variant == 2:  # P, (R o G) S, P V, state update
        method = 2 * C * C * dk + 2 * C * dk * dv + 2 * C * C * dv + 2 * C * dk * dv
        issued = lower * 6 + 2 * C * dk * dv * 3 + 2 * C * C * dv * 2 + 2 * C * dk * dv * 2
    elif variant == 1:  # A and P, X = (K o G) S, (Q o G) S, T diag(b) (V - X), P U, state update
        method = 2 * C * C * dk * 2 + 2 * C * C * dv * 2 + 2 * C * dk * dv * 3
        issued = (2 * lower * 6 + 2 * C * dk * dv * 3 * 2 + 2 * C * C * dv * 3 + 2 * C * C * dv * 3
                  + 2 * C * dk * dv * 3)
    else:  # K K^T, Q K^T (lower blocks), X = K S, Q S, T diag(b) (V - diag(g) X), P U, K^T U
        method = 2 * C * C * dk * 2 + 2 * C * C * dv * 2 + 2 * C * dk * dv * 3
        issued = (2 * lower + 2 * C * dk * dv * 2 * 2 + 2 * C * C * dv * 3 + 2 * C * C * dv * 3
                  + 2 * C * dk * dv * 2)
    return {"bytes": byts, "method_flops": method / C, "issued_flops": issued / C}


def prefill_leg(args, inp, Tn, base_dt, reps: int = 5) -> dict:
    """Time dl_prefill of a prompt of --prefill-tokens tokens on every tile of the workload
    (prompt rows cycle over the drawn steps already on the device)."""
    import torch

    from linear_attention_recurrent_amd import deltalog as dl
    B, H, dk, dv, L = inp.batch, inp.heads, inp.dk, inp.dv, inp.log_len
    Tp = args.prefill_tokens
    dev = torch.device("cuda", 0)
    P = Tn["q"].shape[0]
    idx = torch.arange(Tp, device=dev) % P
    tm = lambda x: None if x is None else x.index_select(0, idx).transpose(0, 1).contiguous()
    q, k, v, decay, beta, eta = (tm(Tn[n]) for n in ("q", "k", "v", "decay", "beta", "eta"))
    out = torch.empty((B, Tp, H, dv), dtype=torch.float32, device=dev)
    pool = dl.DeltaLogPool(inp.variant, B, H, dk, dv, L, dev, base_dt)
    dl.dl_init_state(pool, Tn["s0"], None)
    io = dl.make_prefill_io(pool, q, k, v, decay, beta, out, eta, inp.eps, bonus=Tn["bonus"])
    for _ in range(2):
        dl.dl_prefill(pool, io)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        dl.dl_prefill(pool, io)
    end.record(stream)
    torch.cuda.synchronize()
    secs = start.elapsed_time(end) / 1e3 / reps
    m = prefill_model(dk, dv, variant=inp.variant)
    units = B * H * Tp
    gbs = m["bytes"] * units / secs / 1e9
    tf_issued = m["issued_flops"] * units / secs / 1e12
    prof = read_prefill_counters(WORKLOADS[args.workload]["name"], Tp) if base_dt == dl.BASE_F32 else None
    traffic = None if prof is None else (float(prof["fetch_bytes_per_launch"])
                                         + float(prof["write_bytes_per_launch"]))
    return {"value": units / secs, "unit": "state-steps/s (B x H x prompt tokens per s)",
            "ms_per_prefill": secs * 1e3, "tokens": Tp, "reps": reps,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": traffic},
            "mfma": {"issued_tflops": tf_issued, "peak": BF16_MFMA_PEAK_TFLOPS, "frac": tf_issued / BF16_MFMA_PEAK_TFLOPS,
                     "method_tflops": m["method_flops"] * units / secs / 1e12},
            "bytes_per_state_step": m["bytes"], "issued_flops_per_state_step": m["issued_flops"]}


def merge_leg(args, inp, Tn, ios, base_dt, reps: int = 20) -> dict:
    """Time dl_merge_on with each arithmetic unit on full logs: every tile holds L - 1
    real entries (the most a log holds between calls).  Before each merge the fill and
    the base are restored by device copies outside the events, so every timed merge
    does the same work; only the merge launch is between the events."""
    import torch

    from linear_attention_recurrent_amd import deltalog as dl
    B, H, dk, dv, L, var = inp.batch, inp.heads, inp.dk, inp.dv, inp.log_len, inp.variant
    dev = torch.device("cuda", 0)
    P = len(ios)
    pool = dl.DeltaLogPool(var, B, H, dk, dv, L, dev, base_dt)
    dl.dl_init_state(pool, Tn["s0"], None)
    for t in range(L - 1):
        dl.dl_decode_step(pool, ios[t % P])
    fill0, base0 = pool.fill.clone(), pool.base.clone()
    stream = torch.cuda.current_stream()
    eb = 2 if base_dt == dl.BASE_BF16 else 4
    nbytes = B * H * (2 * eb * dk * dv + (L - 1) * entry_bytes(var, dk, dv) + 8)
    out = {"workload": f"{VARIANT_NAMES[var]} B={B} H={H} dk={dk} dv={dv}, {L - 1} entries per tile"
                       + (", bf16 base" if base_dt == dl.BASE_BF16 else ""),
           "bytes_per_merge": nbytes, "reps": reps}
    for unit, name in ((dl.UNIT_VALU, "valu"), (dl.UNIT_MFMA, "mfma")):
        evs = []
        for _ in range(reps + 2):
            pool.fill.copy_(fill0)
            pool.base.copy_(base0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dl.dl_merge_on(pool, 1, unit)
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        us = float(np.mean([a.elapsed_time(b) for a, b in evs[2:]])) * 1e3
        out[name] = {"us_per_merge": us, "hbm_gbs_algorithmic": nbytes / us / 1e3}
    out["mfma_speedup"] = out["valu"]["us_per_merge"] / out["mfma"]["us_per_merge"]
    return out


def serving_leg(args, cpu) -> dict:
    """The 48-layer serving pool: one pool per layer (B = 512, H = 32, 128/128, ragged
    start fills shared by a sequence's layers), one step = one dl_decode_step per layer.
    A pool of drawn step inputs is reused across steps and layers (values do not change
    the traffic).  The eager comparator keeps one fp32 state per layer."""
    import torch

    from linear_attention_recurrent_amd import deltalog as dl
    w = WORKLOADS[5]
    layers = w["layers"]
    P = min(args.pool_slots, 16)
    inp, T, ios, _ = gpu_setup(5, P, args.log_len)
    B, H, dk, dv, L, var = inp.batch, inp.heads, inp.dk, inp.dv, inp.log_len, inp.variant
    tiles = B * H
    dev = torch.device("cuda", 0)
    bf16_base = args.base_dtype == "bf16"
    base_dt = dl.BASE_BF16 if bf16_base else dl.BASE_F32
    pools = [dl.DeltaLogPool(var, B, H, dk, dv, L, dev, base_dt) for _ in range(layers)]
    for p_ in pools:
        dl.dl_init_state(p_, T["s0"], inp.fill0)
    # ragged start fills spread the folds over every step; the timed steps are still a
    # whole number of fold periods
    K = -(-args.steps // L) * L
    W = args.warmup

    def step(t):
        io = ios[t % P]
        for p_ in pools:
            dl.dl_decode_step(p_, io)
    secs = time_loop(step, K, W)
    del pools
    torch.cuda.empty_cache()
    if args.only == "deltalog":
        print(json.dumps({"ms_per_step": secs / K * 1e3, "timed_steps": K, "layers": layers}))
        raise SystemExit(0)
    Ke = max(1, K // 4)
    states = [T["s0"].clone() for _ in range(layers)]

    def eager(t):
        io = ios[t % P]
        for st in states:
            dl.dl_eager_step(var, st, io)
    secs_e = time_loop(eager, Ke, min(W, 4))
    del states

    mdl = deltalog_bytes_per_state_step(var, dk, dv, L, B, 2 if bf16_base else 4)
    eag = eager_bytes_per_state_step(var, dk, dv, B)
    t_step, t_eager = secs / K, secs_e / Ke
    work = tiles * layers
    achieved = mdl["total"] * tiles / (t_step / layers) / 1e9
    prof = read_counter_profile(w["name"], bf16_base, L)
    traffic = None
    if prof is not None:
        traffic = float(prof["fetch_bytes_per_launch"]) + float(prof["write_bytes_per_launch"])
    return {
        "metric": "decode state-steps/s (B×H×layers per s)",
        "value": work / t_step,
        "unit": "state-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "timed_steps": K,
        "warmup": W,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w['name']}: GDN decode, {layers} layers, B={B} H={H} dk={dk} dv={dv} "
                               f"L={L}, ragged start fills U{{0..L-1}} per sequence"
                               + (", bf16 base" if bf16_base else ""),
                   "base": "bf16, rounded at each fold" if bf16_base else "f32",
                   "variant": VARIANT_NAMES[var], "layers": layers, "batch": B, "heads": H, "dk": dk,
                   "dv": dv, "log_len": L, "input_pool_steps": P},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic},
        "cpu_baseline": cpu,
        "bytes_per_state_step_model": {"deltalog": mdl["total"], "eager": eag["total"]},
        "state_write_bytes_per_state_step": {
            "deltalog_model": mdl["state_writes"], "eager_model": eag["state_writes"],
            "cut_model": eag["state_writes"] / mdl["state_writes"]},
        "eager": {"value": work / t_eager, "ms_per_step": t_eager * 1e3, "steps": Ke,
                  "hbm_gbs_algorithmic": eag["total"] * work / t_eager / 1e9,
                  "deltalog_speedup": t_eager / t_step},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5, 6],
                    help="5 = the 48-layer serving pool (B=512, ragged fills); --log-len picks its L")
    ap.add_argument("--log-len", type=int, default=None)
    ap.add_argument("--dk", type=int, default=None, choices=[64, 128],
                    help="override the workload's key head size (merge leg)")
    ap.add_argument("--dv", type=int, default=None, choices=[64, 128],
                    help="override the workload's value head size (merge leg)")
    ap.add_argument("--pool-slots", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="replay the step loop as a HIP graph")
    ap.add_argument("--only", choices=["deltalog", "warm", "eager", "copy", "prefill", "merge", "ceiling"],
                    default=None, help="run one leg only (for profiling runs): deltalog = the cache-cold "
                                       "headline leg, warm = one pool (cache-resident)")
    ap.add_argument("--prefill-tokens", type=int, default=4096,
                    help="prompt length of the prefill leg (GDN workloads)")
    ap.add_argument("--base-dtype", choices=["f32", "bf16"], default="f32",
                    help="storage of the dense base: fp32 (exact path) or bf16 (low-bit base, "
                         "rounded at each fold; log and arithmetic stay fp32)")
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed windows of the cold headline leg; the line reports their median")
    ap.add_argument("--trace", action="store_true",
                    help="time the cache-cold leg's launches workgroup by workgroup on the tracing build")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Decode tiles are independent, so N GPUs would each run this same kernel on their own "
              "share of sequences with no communication.", file=sys.stderr)
        sys.exit(2)

    cpu = None
    if not args.no_cpu_baseline and args.only is None and not args.trace:
        cpu = cpu_baseline(args.workload)  # before any GPU work: forked workers never touch the GPU

    import torch

    from linear_attention_recurrent_amd import deltalog as dl
    dl.load_library()
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    dev = torch.device("cuda", 0)

    if args.only == "copy":
        # plain copy of known size, for scaling rocprofv3's FETCH_SIZE / WRITE_SIZE counters
        n = 256 << 20
        a = torch.ones(n // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n, "launches": 5}))
        return

    if args.workload == 5:
        if args.trace or args.only not in (None, "deltalog"):
            raise SystemExit("the serving pool (--workload 5) runs its own leg only: no --trace or --only other than "
                             "deltalog")
        print(json.dumps(serving_leg(args, cpu)))
        return

    if (args.dk or args.dv) and args.only != "merge":
        raise SystemExit("--dk/--dv apply to the merge leg only (--only merge)")
    inp, T, ios, w = gpu_setup(args.workload, args.pool_slots, args.log_len, args.dk, args.dv)
    B, H, dk, dv, L, var = inp.batch, inp.heads, inp.dk, inp.dv, inp.log_len, inp.variant
    P = args.pool_slots
    tiles = B * H
    K, W = args.steps, args.warmup
    bf16_base = args.base_dtype == "bf16"
    base_dt = dl.BASE_BF16 if bf16_base else dl.BASE_F32
    if args.only == "merge":
        print(json.dumps(merge_leg(args, inp, T, ios, base_dt)))
        return
    if args.only == "prefill":
        print(json.dumps(prefill_leg(args, inp, T, base_dt)))
        return
    if args.trace:
        print(json.dumps(trace_leg(args, inp, ios, base_dt)))
        return

    # Cache-cold (the headline): NP independent pools used in turn, so that between two
    # steps on one pool the other pools' traffic exceeds the 256 MiB last-level cache and
    # every step reads its state from HBM, as a model with several layers would.  Every
    # pool goes through whole fold periods: the timed steps are a multiple of NP * L.
    eb = 2 if bf16_base else 4
    pool_bytes = tiles * (eb * dk * dv + L * entry_bytes(var, dk, dv) + 4)
    NP = 1 + -(-MALL_BYTES // pool_bytes)
    period = NP * L
    Kc = -(-K // period) * period
    Wc = -(-W // period) * period
    chunk = 0
    if args.graph:
        chunk = period * max(1, 64 // period)
        Kc = -(-Kc // chunk) * chunk
    result = {}
    pools = []
    if args.only in (None, "deltalog", "ceiling"):
        pools = [dl.DeltaLogPool(var, B, H, dk, dv, L, dev, base_dt) for _ in range(NP)]
        for p_ in pools:
            dl.dl_init_state(p_, T["s0"], inp.fill0)
    if args.only in (None, "deltalog"):
        # the median of `repeats` timed windows, each a whole number of fold periods of every
        # pool (so every pool is back at fill 0 between windows)
        reps = [time_loop(lambda t: dl.dl_decode_step(pools[t % NP], ios[t % P]), Kc, Wc if r == 0 else 0, chunk)
                for r in range(args.repeats)]
        result["cold_repeats"] = reps
        result["cold"] = float(np.median(reps))
    if args.only in (None, "ceiling"):
        result["ceiling"] = read_ceilings(pools, tiles, eb * dk * dv, (L - 1) / 2 * entry_bytes(var, dk, dv), Kc)
    del pools
    # Cache-resident: one pool, whose working set may stay in the last-level cache.
    Kw = -(-K // L) * L
    Ww = -(-W // L) * L
    if args.only in (None, "warm"):
        pool = dl.DeltaLogPool(var, B, H, dk, dv, L, dev, base_dt)
        dl.dl_init_state(pool, T["s0"], inp.fill0)
        result["warm"] = time_loop(lambda t: dl.dl_decode_step(pool, ios[t % P]), Kw, Ww,
                                   L * max(1, 64 // L) if args.graph else 0)
        del pool
    # The eager comparator, on as many states as the cold leg has pools, and on one.
    if args.only in (None, "eager"):
        NE = 1 + -(-MALL_BYTES // (tiles * 4 * dk * dv))
        states = [T["s0"].clone() for _ in range(NE)]
        result["eager_cold"] = time_loop(lambda t: dl.dl_eager_step(var, states[t % NE], ios[t % P]), Kw, W)
        result["eager_warm"] = time_loop(lambda t: dl.dl_eager_step(var, states[0], ios[t % P]), Kw, W)
        del states
    torch.cuda.empty_cache()
    if args.only is not None:
        out = {k: v / (Kc if k == "cold" else Kw) * 1e3 for k, v in result.items()
               if k not in ("ceiling", "cold_repeats")}
        out.update({"unit": "ms per step", "timed_steps_cold": Kc, "timed_steps": Kw})
        if "cold_repeats" in result:
            out["cold_repeats"] = [v / Kc * 1e3 for v in result["cold_repeats"]]
        if "ceiling" in result:
            out["ceiling"] = result["ceiling"]
        print(json.dumps(out))
        return
    result["prefill"] = prefill_leg(args, inp, T, base_dt)

    # copy ceilings on this machine: a plain device copy that fits the last-level cache
    # (2 x 64 MiB) and one that does not (2 x 1 GiB); read + write bytes over time
    copy = {}
    for label, nbytes in (("fits_cache", 64 << 20), ("cold", 1 << 30)):
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        reps = 20 if nbytes < (256 << 20) else 5
        secs_copy = time_loop(lambda t: dst.copy_(src), reps, 3)
        copy[label] = 2 * nbytes * reps / secs_copy / 1e9
        del src, dst

    mdl = deltalog_bytes_per_state_step(var, dk, dv, L, B, eb)
    eag = eager_bytes_per_state_step(var, dk, dv, B)
    launch_bytes = mdl["total"] * tiles
    t_cold = result["cold"] / Kc
    t_warm = result["warm"] / Kw
    t_ecold = result["eager_cold"] / Kw
    t_ewarm = result["eager_warm"] / Kw
    achieved = launch_bytes / t_cold / 1e9
    achieved_warm = launch_bytes / t_warm / 1e9
    ceil = result["ceiling"]
    prof = read_counter_profile(w["name"], bf16_base)
    traffic = None
    counter_write = None
    if prof is not None:
        traffic = float(prof["fetch_bytes_per_launch"]) + float(prof["write_bytes_per_launch"])
        counter_write = {"deltalog": float(prof["write_bytes_per_launch"]) / tiles,
                         "eager": float(prof.get("eager_write_bytes_per_launch", "nan")) / tiles,
                         "source": f"profiles/{counter_profile_name(w['name'], bf16_base)}"}
    line = {
        "metric": "decode state-steps/s (B×H per s)",
        "value": tiles / t_cold,
        "unit": "state-steps/s",
        "n_gpus": 1,
        "steps": K,
        "timed_steps": Kc,
        "warmup": W,
        "ms_per_step": t_cold * 1e3,
        "repeats": args.repeats,
        "ms_per_step_repeats": [v / Kc * 1e3 for v in result["cold_repeats"]],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w['name']}: {VARIANT_NAMES[var]} decode B={B} H={H} dk={dk} dv={dv} L={L}"
                               + (" (Kaczmarz step size)" if inp.eta is not None else "")
                               + (", bf16 base" if bf16_base else "")
                               + f", cache-cold: {NP} pools of this shape used in turn, so each step reads "
                                 f"its state from HBM",
                   "base": "bf16, rounded at each fold" if bf16_base else "f32",
                   "variant": VARIANT_NAMES[var], "batch": B, "heads": H, "dk": dk, "dv": dv,
                   "log_len": L, "initial_fill": "0 for every sequence" if not np.any(inp.fill0) else "ragged",
                   "pools_in_turn": NP, "input_pool_steps": P, "hip_graph": bool(chunk)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic},
        "cpu_baseline": cpu,
        "hbm_gbs_algorithmic": achieved,
        "hbm_target": {"frac_of_peak_needed": 0.70, "measured_cold_frac": achieved / HBM_PEAK_GBS,
                       "met": achieved / HBM_PEAK_GBS >= 0.70,
                       "frac_of_tile_read_ceiling": achieved / ceil["tile_read_gbs"],
                       "frac_of_tile_read_log_ceiling": achieved / ceil["tile_read_log_gbs"],
                       "frac_of_tile_stream_ceiling": achieved / ceil["tile_stream_gbs"],
                       "frac_of_owned_stream_ceiling": (achieved / ceil["owned_stream_gbs"]
                                                        if "owned_stream_gbs" in ceil else None),
                       "frac_of_torch_sum_ceiling": achieved / ceil["torch_sum_gbs"]},
        "read_ceiling_gbs": ceil,
        "cache_resident": {"value": tiles / t_warm, "ms_per_step": t_warm * 1e3, "timed_steps": Kw,
                           "hbm_gbs_algorithmic": achieved_warm, "frac": achieved_warm / HBM_PEAK_GBS,
                           "note": "one pool, working set inside the 256 MiB last-level cache: "
                                   "not an HBM rate"},
        "bytes_per_state_step_model": {"deltalog": mdl["total"], "eager": eag["total"]},
        "bytes_per_launch_model": launch_bytes,
        "state_write_bytes_per_state_step": {
            "deltalog_model": mdl["state_writes"], "eager_model": eag["state_writes"],
            "cut_model": eag["state_writes"] / mdl["state_writes"], "counters": counter_write},
        "eager": {"value": tiles / t_ecold, "ms_per_step": t_ecold * 1e3, "timed_steps": Kw,
                  "hbm_gbs_algorithmic": eag["total"] * tiles / t_ecold / 1e9,
                  "deltalog_speedup": t_ecold / t_cold,
                  # the speed-up if each step ran at its access shape's probe rate (decode: tile
                  # plus mean log read; eager: tile read and written back)
                  "deltalog_speedup_at_probe_rates": (eag["total"] / ceil["tile_rw_gbs"])
                                                     / (mdl["total"] / ceil["tile_read_log_gbs"]),
                  "cache_resident": {"ms_per_step": t_ewarm * 1e3, "deltalog_speedup": t_ewarm / t_warm}},
        "copy_ceiling_gbs": copy,
        "prefill": result.get("prefill"),
        "merge": merge_leg(args, inp, T, ios, base_dt),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
