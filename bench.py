#!/usr/bin/env python
"""Benchmark of the fused MoE finalize + residual add + RMSNorm on one MI355X.

One step = one call of the fused op over one batch of synthetic input (all of
its steps: gather, weighted sum, shared and residual adds, rounding, RMSNorm).
The headline workload is the 8192-token prefill chunk (H=6144, K=8, scale 2.5,
1% of residual rows x100; 1.21 GB per call, larger than the 256 MB Infinity
Cache, so every call streams its inputs from HBM). Inputs are resident in HBM
before the timed region; HIP events on the launch stream bracket exactly
--steps calls on one buffer set.

Printed (stdout, one JSON line): effective HBM GB/s = algorithmic bytes per
call / time per call, the roofline object for the fused kernel, the oracle's
CPU baseline on the same workload (one core, and every core in threads over
disjoint token ranges), and, as context, decode-latency figures for
T = 1..64 and the 512-token batch, a measured copy ceiling, the dense tail and
the FP8-output calls at T = 8192, the host cost of the torch deferred path,
the headline workload with its gathered rows grouped by expert instead of
randomly placed, and the chunk and the batch in other input states (buffer
sets cycled, outputs and inputs cycled apart, Infinity Cache flushed).

Modes used with rocprofv3 (see profiles/):
  --pmc-run          a short run of the fused kernel plus a 1 GiB copy of known
                     size, for counter collection (FETCH_SIZE / WRITE_SIZE)
  --latency-run      eager calls at the decode sizes and the 512 batch (and the
                     dense, FP8-output and dense FP8-output calls at T=28 and
                     8192), to trace
  --shape-sweep      every launch shape (vectors per thread x store policy, and
                     the persistent kernel) at T = 64..8192, HBM-cold; with
                     --alternatives, the alternatives to the shipped launch
                     (a per-CU workgroup cap, per-XCD token ranges, every
                     store encoding, the persistent kernel) at T = 512..8192;
                     with --eager, plain launches for a kernel trace
  --persist-counters-run  the automatic and the persistent launch at T = 512,
                     2048 and 8192, then the copy probe, for counters
  --state-run        eager launches of the input states, for counters
  --cold-table       µs per call against T = 1..8192 (fused, FP8-output and
                     dense calls), fresh inputs on every call
  --summarize-trace  per-(kernel, grid) durations from a kernel_trace.csv
  --summarize-phases durations or counters of a phase run (shape sweep,
                     persistent counters, input states) by dispatch order
  --summarize-pmc    turn counter_collection.csv files into profiles/ traffic data
  --pmc-variants-run the dense tail, the FP8-output call and the dense tail with
                     FP8 output at T=8192, plus the copy probe, for the same
                     two counters
  --summarize-pmc-variants  their calibrated traffic against their own bytes
  --summarize-counters  join shader and L2 counter passes (occupancy, VALU busy,
                     instructions per wave, LDS bank conflicts, L2 hit rate)
"""
import argparse
import csv
import hashlib
import json
import os
import struct
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused MoE-finalize+RMSNorm µs/call and effective HBM GB/s (% of peak), 1 MI355X"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
FUSED_KERNEL_PREFIX = "mfr_"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_kernel_prefill_T8192_traffic.json")
HEADLINE_CFG, HEADLINE_T = "prefill", 8192


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def _elf_sections(b):
    """{name: bytes} of the sections of a 64-bit little-endian ELF image
    (NOBITS sections map to b""), or None if b is not one."""
    if b[:4] != b"\x7fELF" or b[4] != 2 or b[5] != 1:
        return None
    shoff, = struct.unpack_from("<Q", b, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", b, 0x3A)

    def header(i):
        return struct.unpack_from("<IIQQQQIIQQ", b, shoff + i * shentsize)
    strtab = header(shstrndx)
    names = b[strtab[4]:strtab[4] + strtab[5]]
    out = {}
    for i in range(shnum):
        h = header(i)
        name = names[h[0]:names.index(b"\0", h[0])].decode()
        out[name] = b"" if h[1] == 8 else b[h[4]:h[4] + h[5]]
    return out


def _offload_bundle(b):
    """[(target triple, code object bytes)] of an uncompressed clang offload
    bundle (the .hip_fatbin section of a HIP library)."""
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    if b[:len(magic)] != magic:
        return None
    n, = struct.unpack_from("<Q", b, len(magic))
    off, out = len(magic) + 8, []
    for _ in range(n):
        o, size, tl = struct.unpack_from("<QQQ", b, off)
        off += 24
        out.append((b[off:off + tl].decode(), b[o:o + size]))
        off += tl
    return out


# Sections of a gfx950 code object that hold the kernels' machine code, their
# descriptors and their metadata. The symbol tables are left out: they name a
# per-build identifier derived from the build path.
CODE_SECTIONS = (".text", ".rodata", ".note")


def kernel_code_hash(lib_path=None):
    """Hash of the machine code of the gfx950 kernels in a built library: the
    .text, .rodata and .note sections of every gfx950 code object in its
    offload bundle. It changes when the kernels' code, resources or
    metadata change, and is the same for the same source built at any path.
    Traffic figures measured on other kernel code are not reported."""
    if lib_path is None:
        from top_finalize_residual_amd import build as bld
        lib_path = bld.LIB
    if not os.path.exists(lib_path):
        return None
    with open(lib_path, "rb") as f:
        host = _elf_sections(f.read())
    bundle = _offload_bundle(host.get(".hip_fatbin", b"")) if host else None
    if not bundle:
        return None
    h = hashlib.sha256()
    found = False
    for triple, co in bundle:
        if "gfx950" not in triple:
            continue
        secs = _elf_sections(co)
        if secs is None:
            return None
        found = True
        h.update(triple.encode())
        for name in CODE_SECTIONS:
            data = secs.get(name, b"")
            h.update(name.encode() + struct.pack("<Q", len(data)) + data)
    return h.hexdigest()[:16] if found else None


# ---------------------------------------------------------------------------
# device helpers
# ---------------------------------------------------------------------------

def to_device(d):
    import numpy as np
    import torch

    def bf16(u):
        return torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).view(torch.bfloat16).cuda()
    return dict(expert_out=bf16(d["expert_out"]), perm_idx=torch.from_numpy(d["perm_idx"]).cuda(),
                topk_w=torch.from_numpy(d["topk_w"]).cuda(), shared_out=bf16(d["shared_out"]),
                residual=bf16(d["residual"]), gamma=bf16(d["gamma"]))


def make_caller(dd, eps, scale):
    """A zero-allocation closure that enqueues one fused call on the current stream."""
    import torch
    import top_finalize_residual_amd as mfr
    T, K = dd["perm_idx"].shape
    H = dd["gamma"].shape[0]
    r_out = torch.empty_like(dd["residual"])
    n_out = torch.empty_like(dd["residual"])
    args = [dd[k].data_ptr() for k in ("expert_out", "perm_idx", "topk_w", "shared_out",
                                       "residual", "gamma")]
    ro, no = r_out.data_ptr(), n_out.data_ptr()
    dev = dd["gamma"].get_device()
    raw_stream = torch._C._cuda_getCurrentRawStream  # the current stream's handle, no object

    def call():
        rc = mfr.moe_finalize_rmsnorm_raw(*args, eps, scale, ro, no, T, H, K, raw_stream(dev))
        if rc != 0:
            raise RuntimeError(mfr.strerror(rc))
    # the closure holds raw addresses: keep every tensor it writes or reads alive
    # for as long as the closure lives
    call.keep = (dd, r_out, n_out)
    return call, (r_out, n_out)


def time_calls(calls, n, warmup):
    """Mean device ms per call over n calls (events on the launch stream)."""
    import torch
    for i in range(warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for i in range(n):
        calls[i % len(calls)]()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def time_graph(calls, per_call, replays):
    """Mean device ms per call inside a captured graph that runs the list of
    calls in turn, per_call times each (rotating buffer sets keep it cold)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_call):
            for c in calls:
                c()
    g.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(replays):
        g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (per_call * len(calls) * replays)


def _probe_lib():
    import ctypes
    from top_finalize_residual_amd import build as b
    lib = ctypes.CDLL(b.PROBE_LIB)
    for fn in (lib.mfr_copy_probe, lib.mfr_read_probe, lib.mfr_touch_probe):
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                       ctypes.c_void_p]
    lib.mfr_write_probe.restype = ctypes.c_int
    lib.mfr_write_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_int,
                                    ctypes.c_void_p]
    lib.mfr_empty_probe.restype = ctypes.c_int
    lib.mfr_empty_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.mfr_mix_probe.restype = ctypes.c_int
    lib.mfr_mix_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.POINTER(ctypes.c_int64),
                                  ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p]
    return lib


def probe_ceilings(nbytes=1 << 30, reps=10):
    """GB/s of the copy probe (read + write bytes), the read-only probe and
    the write-only probe, on 1 GiB buffers (4x the Infinity Cache, so all
    three stream from HBM). Each is the best over three grid sizes (2, 8 and
    32 workgroups per CU): the write rate in particular depends on it."""
    import torch
    lib = _probe_lib()
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grids = (cus * 2, cus * 8, cus * 32)
    sink = torch.empty(max(grids), dtype=torch.int32, device="cuda")
    best = {"copy": 0.0, "read": 0.0, "write": 0.0}
    for grid in grids:
        def copy():
            if lib.mfr_copy_probe(src.data_ptr(), dst.data_ptr(), nbytes, grid,
                                  torch.cuda.current_stream().cuda_stream) != 0:
                raise RuntimeError("copy probe failed")

        def read():
            if lib.mfr_read_probe(src.data_ptr(), sink.data_ptr(), nbytes, grid,
                                  torch.cuda.current_stream().cuda_stream) != 0:
                raise RuntimeError("read probe failed")

        def write():
            if lib.mfr_write_probe(dst.data_ptr(), nbytes, 0x3F803F80, grid,
                                   torch.cuda.current_stream().cuda_stream) != 0:
                raise RuntimeError("write probe failed")
        for name, fn, moved in (("copy", copy, 2 * nbytes), ("read", read, nbytes),
                                ("write", write, nbytes)):
            gbs = moved / (time_calls([fn], reps, 2) * 1e-3) / 1e9
            best[name] = max(best[name], gbs)
    del src, dst, sink
    torch.cuda.empty_cache()
    return best["copy"], best["read"], best["write"]


# The mixed-stream probe at the headline chunk's bytes: its reads (rows,
# shared and residual) against its writes with bf16 output, or with FP8 codes
# (residual_out plus one byte per element). Per thread and unit of work, each
# one token of the fused op at 256 threads: 30 vectors read for 6 written
# with bf16 output; 30 read for 3 written and three 8-byte stores to a
# second region (the codes form) with FP8 output.
MIX_WT, MIX_PIPE, MIX_CODES = 1, 2, 4  # mfr_mix_probe flags
MIX_PAIRS = {"bf16": (30, 6), "fp8": (30, 3)}
MIX_FORM = {"bf16": 0, "fp8": MIX_CODES}
MIX_READ_BYTES = 8192 * 8 * 6144 * 2 + 2 * 8192 * 6144 * 2  # rows, shared, residual
MIX_WRITE_BYTES = {"bf16": 2 * 8192 * 6144 * 2, "fp8": 8192 * 6144 * 3}


class _MixProbe:
    """The mixed-stream probe on one pair of buffers of the chunk's sizes."""

    def __init__(self):
        import torch
        self.lib = _probe_lib()
        self.src = torch.empty(MIX_READ_BYTES, dtype=torch.uint8, device="cuda")
        self.dst = torch.empty(MIX_WRITE_BYTES["bf16"], dtype=torch.uint8, device="cuda")
        self.src.fill_(1)
        self.cus = torch.cuda.get_device_properties(0).multi_processor_count

    def gbs_us(self, reads, writes, flags, grid, per_cu, reps=10):
        """(GB/s of read + write bytes, µs per call), or None where the
        residency cannot be set that way."""
        import ctypes
        import torch
        rb, wb = ctypes.c_int64(0), ctypes.c_int64(0)
        fp8 = bool(flags & MIX_CODES) or reads * 3 == writes * 20
        wbytes = MIX_WRITE_BYTES["fp8" if fp8 else "bf16"]
        rc = []

        def call():
            r = self.lib.mfr_mix_probe(self.src.data_ptr(), MIX_READ_BYTES, self.dst.data_ptr(),
                                       wbytes, reads, writes, flags, grid, per_cu, ctypes.byref(rb),
                                       ctypes.byref(wb), torch.cuda.current_stream().cuda_stream)
            if r == 3:
                rc.append(r)
                return
            if r != 0:
                raise RuntimeError(f"mix probe failed ({r})")
        call()
        torch.cuda.synchronize()
        if rc:
            return None
        ms = time_calls([call], reps, 2)
        return (rb.value + wb.value) / (ms * 1e-3) / 1e9, ms * 1e3

    def close(self):
        import torch
        del self.src, self.dst
        torch.cuda.empty_cache()


def mix_probe_ceilings(reps=10):
    """GB/s (read + write bytes) of the mixed-stream probe at the headline
    chunk's own byte counts, with bf16 output and with FP8 codes (each in
    units of one token of the fused op), in the headline's cache state (one
    buffer set, calls back to back). Best over
    write-back and write-through stores and four launch shapes: one workgroup
    per unit of work (as the fused op launches one per token), the same capped
    at 2 workgroups per CU through reserved LDS (as the fused op at this
    size), and grids of 2 and 8 workgroups per CU that walk the units; every
    combination is returned too, as {name: [GB/s, µs]}."""
    probe = _MixProbe()
    cus = probe.cus
    out = {}
    for mode, (a, b) in MIX_PAIRS.items():
        best, detail = 0.0, {}
        for wt in (0, MIX_WT):
            for grid, per_cu, shape in ((0, 0, "per-unit"), (0, 2, "per-unit-cap2"),
                                        (2 * cus, 0, "2-per-cu"), (8 * cus, 0, "8-per-cu")):
                r = probe.gbs_us(a, b, wt | MIX_FORM[mode], grid, per_cu, reps)
                if r is None:
                    continue
                detail[f"{'wt' if wt else 'wb'}-{shape}"] = [round(r[0], 1), round(r[1], 2)]
                best = max(best, r[0])
        out[mode] = {"gbs": round(best, 1), "shapes": detail}
    probe.close()
    return out


# The depth sweep: vectors in flight per thread (reads of one unit, with a
# fifth as many writes) against workgroups per CU, for the one-unit-per-
# workgroup form (capped through reserved LDS) and the pipelined form (a
# grid of that many workgroups per CU walking the units).
MIX_DEPTHS = (10, 15, 20, 25, 30, 40)
MIX_CAPS = (1, 2, 3, 4)


def mix_sweep(reps=3):
    """Median GB/s over reps interleaved repetitions of every depth x
    residency of the mixed-stream probe (bf16 proportion, write-through
    stores), the one-unit form with no cap, and the FP8 proportion at its
    two depths and in the FP8-code form (one token with FP8 output); keys
    "unit/A<reads>/cap<n>", "pipe/A<reads>/<n>-per-cu", "unit/A<reads>/nocap",
    "fp8/A<reads>/cap<n>" and "fp8codes/A30/cap<n>"."""
    import statistics
    probe = _MixProbe()
    runs = {}
    for rep in range(reps):
        for a in MIX_DEPTHS:
            for n in MIX_CAPS:
                r = probe.gbs_us(a, a // 5, MIX_WT, 0, n)
                if r is not None:
                    runs.setdefault(f"unit/A{a}/cap{n}", []).append(r[0])
                r = probe.gbs_us(a, a // 5, MIX_WT | MIX_PIPE, n * probe.cus, 0)
                if r is not None:
                    runs.setdefault(f"pipe/A{a}/{n}-per-cu", []).append(r[0])
            r = probe.gbs_us(a, a // 5, MIX_WT, 0, 0)
            runs.setdefault(f"unit/A{a}/nocap", []).append(r[0])
        for a, b in ((20, 3), (40, 6)):
            for n in (1, 2, 3):
                r = probe.gbs_us(a, b, MIX_WT, 0, n)
                if r is not None:
                    runs.setdefault(f"fp8/A{a}/cap{n}", []).append(r[0])
        for n in (1, 2, 3):
            r = probe.gbs_us(30, 3, MIX_WT | MIX_CODES, 0, n)
            if r is not None:
                runs.setdefault(f"fp8codes/A30/cap{n}", []).append(r[0])
        log(f"mix sweep: repetition {rep + 1} of {reps}")
    probe.close()
    return {k: round(statistics.median(v), 1) for k, v in runs.items()}


def mix_sweep_lines(path):
    """Markdown tables of a mix_sweep record."""
    with open(path) as f:
        rec = json.load(f)
    lines = ["GB/s (read + write bytes) of the mixed-stream probe (`csrc/copy_probe.hip`) over "
             "the 8192-token chunk's bytes (1.007 GB read; 201 MB written with bf16 output, "
             "151 MB with FP8 codes), one buffer set, calls back to back, write-through stores, "
             "median of the interleaved repetitions. A unit is one workgroup's share: A "
             "16-byte vectors read per thread, all in flight at once, then A/5 written (A = 30 "
             "is one token of the fused op with bf16 output at 256 threads). The in-flight "
             "bytes per CU are the workgroups per CU times A x 4 KiB.", "",
             "One unit per workgroup (the fused op's launch), at most n workgroups per CU "
             "(reserved LDS; a dash where the registers allow fewer), and with no cap:", "",
             "| A (KiB per unit) | n = 1 | n = 2 | n = 3 | n = 4 | no cap |",
             "|---|---|---|---|---|---|"]
    for a in MIX_DEPTHS:
        row = [rec.get(f"unit/A{a}/cap{n}") for n in MIX_CAPS] + [rec.get(f"unit/A{a}/nocap")]
        lines.append(f"| {a} ({a * 4}) | " + " | ".join("—" if v is None else f"{v:,.0f}"
                                                         for v in row) + " |")
    lines += ["", "Pipelined (each workgroup walks its units and issues the next unit's loads "
              "before the current unit's stores, as the persistent multi-token kernel does), a "
              "grid of n workgroups per CU:", "",
              "| A (KiB per unit) | n = 1 | n = 2 | n = 3 | n = 4 |", "|---|---|---|---|---|"]
    for a in MIX_DEPTHS:
        row = [rec.get(f"pipe/A{a}/{n}-per-cu") for n in MIX_CAPS]
        lines.append(f"| {a} ({a * 4}) | " + " | ".join("—" if v is None else f"{v:,.0f}"
                                                         for v in row) + " |")
    lines += ["", "FP8 proportion (A read for 3A/20 written), one unit per workgroup; the codes "
              "form is one token with FP8 output (30 read, then 3 vectors and 3 half vectors "
              "written, the halves to a region of their own):", "",
              "| A (KiB per unit) | n = 1 | n = 2 | n = 3 |", "|---|---|---|---|"]
    for a, key in ((20, "fp8/A20"), (40, "fp8/A40"), (30, "fp8codes/A30")):
        row = [rec.get(f"{key}/cap{n}") for n in (1, 2, 3)]
        name = f"{a} ({a * 4}), codes form" if key.startswith("fp8codes") else f"{a} ({a * 4})"
        lines.append(f"| {name} | " + " | ".join("—" if v is None else f"{v:,.0f}"
                                                  for v in row) + " |")
    return lines


def summarize_mix(args):
    lines = [f"# {args.title}", "", "Commands ($REPO is the repository root, $OUT any output "
             "directory):", "", "```", args.command, "```", ""] + mix_sweep_lines(args.summarize_mix)
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def launch_floor_us(grid=1, threads=64):
    """Per-launch device µs of an empty kernel (grid workgroups of `threads`)
    inside a graph of 100 launches: the floor under any kernel of that launch
    shape, measured the way decode_latency measures."""
    import torch
    lib = _probe_lib()

    def empty():
        if lib.mfr_empty_probe(grid, threads, torch.cuda.current_stream().cuda_stream) != 0:
            raise RuntimeError("empty probe failed")
    return round(time_graph([empty], 100, 5) * 1e3, 2)


# ---------------------------------------------------------------------------
# modes
# ---------------------------------------------------------------------------

def cpu_baseline(d, min_seconds=10.0, max_passes=20):
    """The oracle as it stands (single-threaded fp64 C++) on the same workload,
    repeated whole until at least min_seconds of CPU work have been timed."""
    import oracle
    import synth
    nbytes = synth.algorithmic_bytes(d["perm_idx"], d["H"], d["K"])
    oracle.default()
    # one core: the oracle is single-threaded; pinning keeps the scheduler
    # from moving it between cores during the timed passes
    allowed = os.sched_getaffinity(0)
    core = min(allowed)
    os.sched_setaffinity(0, {core})
    try:
        t0 = time.perf_counter()
        passes = 0
        while passes < max_passes and (passes == 0 or time.perf_counter() - t0 < min_seconds):
            oracle.finalize_rmsnorm(d["expert_out"], d["perm_idx"], d["topk_w"], d["shared_out"],
                                    d["residual"], d["gamma"], d["eps"], d["scale"],
                                    want_exact=False)
            passes += 1
        dt = time.perf_counter() - t0
        # the smaller workloads beside their GPU figures: median of 3 runs each
        small = {}
        for cfg, T in (("decode", 28), ("batch512", 512)):
            ds = synth.config_inputs(cfg, T)
            runs = []
            for _ in range(3):
                t1 = time.perf_counter()
                oracle.finalize_rmsnorm(ds["expert_out"], ds["perm_idx"], ds["topk_w"],
                                        ds["shared_out"], ds["residual"], ds["gamma"], ds["eps"],
                                        ds["scale"], want_exact=False)
                runs.append(time.perf_counter() - t1)
            med = sorted(runs)[1]
            nb = synth.algorithmic_bytes(ds["perm_idx"], ds["H"], ds["K"])
            small[f"{cfg}_T{T}"] = {"us_per_call": round(med * 1e6, 1),
                                    "gbs": round(nb / med / 1e9, 4)}
    finally:
        os.sched_setaffinity(0, allowed)
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    cpu = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    all_cores = cpu_baseline_all_cores(d, nbytes)
    return {"value": round(nbytes * passes / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "all_cores": all_cores,
            "sample": f"the whole {d['T']}-token workload, {passes} passes, single thread pinned to "
                      f"core {core} ({dt:.1f} s; {dt / passes * 1e6:.0f} µs/call; host: {cpu}, "
                      f"{len(allowed)} of {os.cpu_count()} logical CPUs available)",
            "smaller_workloads": small}


def cpu_baseline_all_cores(d, nbytes, min_seconds=5.0, max_passes=50):
    """The same oracle routine on every core the process may use: one thread
    per core, each evaluating a disjoint, contiguous range of tokens (the
    oracle is per token, and its C entry point runs without the interpreter
    lock). Whole passes over the workload are repeated until at least
    min_seconds of wall time."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    n = len(os.sched_getaffinity(0))
    T = d["T"]
    bounds = [(T * i // n, T * (i + 1) // n) for i in range(n)]

    def part(b):
        t0, t1 = b
        oracle.finalize_rmsnorm(d["expert_out"], d["perm_idx"][t0:t1], d["topk_w"][t0:t1],
                                d["shared_out"][t0:t1], d["residual"][t0:t1], d["gamma"],
                                d["eps"], d["scale"], want_exact=False)
    with ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(part, bounds))  # warm-up pass
        t0 = time.perf_counter()
        passes = 0
        while passes < max_passes and (passes == 0 or time.perf_counter() - t0 < min_seconds):
            list(ex.map(part, bounds))
            passes += 1
        dt = time.perf_counter() - t0
    return {"value": round(nbytes * passes / dt / 1e9, 4), "unit": "GB/s", "cores": n,
            "sample": f"the whole {T}-token workload, {passes} passes, {n} threads over disjoint "
                      f"token ranges ({dt:.1f} s wall; {dt / passes * 1e6:.0f} µs/call)"}


def traffic_for_headline():
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    code = kernel_code_hash()
    if code is None or t.get("code_hash") != code:
        return None
    return t.get("traffic_bytes_per_launch")


DECODE_TS = (1, 4, 12, 28, 64)


def _raise_on(rc):
    if rc != 0:
        import top_finalize_residual_amd as mfr
        raise RuntimeError(mfr.strerror(rc))


def stacked_calls(d, n, mode="bf16"):
    """n distinct device copies of one input set, each with its own outputs,
    and one zero-allocation closure per copy. mode: "bf16" (the fused op),
    "fp8" (the fused op with only the FP8 normed output) or "dense" (the
    residual add + RMSNorm, with shared_out as its x)."""
    import torch
    import top_finalize_residual_amd as mfr
    dd = to_device(d)
    T, K = dd["perm_idx"].shape
    H = dd["gamma"].shape[0]
    # one set: the uploaded tensors themselves; more: copies made on the device
    st = {k: (v.unsqueeze(0) if n == 1 else v.unsqueeze(0).repeat((n,) + (1,) * v.dim()))
          for k, v in dd.items()}
    ro = torch.empty((n, T, H), dtype=torch.bfloat16, device="cuda")
    no = torch.empty_like(ro)
    q = torch.empty((n, T, H), dtype=torch.uint8, device="cuda")
    sc = torch.empty((n, max(T, 1)), dtype=torch.float32, device="cuda")
    eps, scale = d["eps"], d["scale"]
    names = ("expert_out", "perm_idx", "topk_w", "shared_out", "residual", "gamma")
    calls = []
    for i in range(n):
        a = [st[k][i].data_ptr() for k in names]
        r_i, n_i, q_i, s_i = ro[i].data_ptr(), no[i].data_ptr(), q[i].data_ptr(), sc[i].data_ptr()
        if mode == "bf16":
            def call(a=a, r_i=r_i, n_i=n_i):
                _raise_on(mfr.moe_finalize_rmsnorm_raw(*a, eps, scale, r_i, n_i, T, H, K,
                                                       torch.cuda.current_stream().cuda_stream))
        elif mode == "fp8":
            def call(a=a, r_i=r_i, q_i=q_i, s_i=s_i):
                _raise_on(mfr.moe_finalize_rmsnorm_fp8_raw(*a, eps, scale, r_i, None, q_i, s_i,
                                                           T, H, K,
                                                           torch.cuda.current_stream().cuda_stream))
        elif mode == "dense":
            def call(a=a, r_i=r_i, n_i=n_i):
                _raise_on(mfr.residual_add_rmsnorm_raw(a[3], a[4], a[5], eps, r_i, n_i, T, H,
                                                       torch.cuda.current_stream().cuda_stream))
        else:
            raise ValueError(mode)
        # the closure holds raw addresses: keep every tensor it touches alive
        call.keep = (st, ro, no, q, sc)
        calls.append(call)
    return calls


def touch(tensors):
    """Read every tensor once with ordinary (cache-allocating) loads, so that
    it is resident in the Infinity Cache afterwards."""
    import torch
    lib = _probe_lib()
    grid = 1024
    sink = torch.empty(grid, dtype=torch.int32, device="cuda")
    for t in tensors:
        nbytes = t.numel() * t.element_size()
        if nbytes % 16 or t.data_ptr() % 16:
            raise ValueError("touch needs 16-byte sizes and alignment")
        if lib.mfr_touch_probe(t.data_ptr(), sink.data_ptr(), nbytes, grid,
                               torch.cuda.current_stream().cuda_stream) != 0:
            raise RuntimeError("touch probe failed")
    torch.cuda.synchronize()


def scrub_infinity_cache(nbytes=512 << 20):
    """Read twice the 256 MB Infinity Cache of unrelated data with ordinary
    loads, so that no earlier data stays resident in it."""
    import torch
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    touch([buf])
    del buf


def decode_latency(cold_bytes=600_000_000):
    """Per-call device µs at the decode sizes (H=6144, K=8), graph-replayed,
    with the caches scrubbed first, for two input patterns:
      * same_inputs: 100 back-to-back calls on one buffer set (its pages stay
        mapped in the TLBs; the non-temporal row loads keep the data from
        settling in the caches, so the calls read it from memory);
      * fresh_inputs: one call on each of n distinct buffer sets (stacked
        copies, together above cold_bytes, more than twice the Infinity
        Cache), as a decode step reading rows nothing has touched since they
        were written.
      * producer_written: each call's rows and shared output were written by
        a producer kernel just before it (copies standing in for GEMM2 and
        the shared expert), the state a decode step meets inside a layer;
        the figure is the fused call's share of a graph of producer + call
        pairs, minus a graph of the producers alone.
    Also the FP8-output and dense variants at T = 28, and the empty-kernel
    floor. Context figures, not the headline."""
    import synth
    same, fresh, produced = {}, {}, {}
    variants = {}
    for T in DECODE_TS:
        d = synth.config_inputs("decode", T)
        modes = ("bf16", "fp8", "dense") if T == 28 else ("bf16",)
        nb = synth.algorithmic_bytes(d["perm_idx"], d["H"], d["K"])
        n = max(2, -(-cold_bytes // nb))
        for mode in modes:
            calls = stacked_calls(d, 1, mode)
            scrub_infinity_cache()
            a = round(time_graph(calls, 100, 5) * 1e3, 2)
            calls = stacked_calls(d, n, mode)
            scrub_infinity_cache()
            b = round(time_graph(calls, 1, 3) * 1e3, 2)
            del calls
            if mode == "bf16":
                same[f"T{T}"], fresh[f"T{T}"] = a, b
            else:
                variants[f"{mode}_T{T}"] = {"same_inputs": a, "fresh_inputs": b}
        produced[f"T{T}"] = producer_written_us(d)
    # the floor under each decode launch: an empty kernel of the token
    # path's launch shape (T workgroups of 768 threads at H = 6144)
    floor = {f"T{T}": launch_floor_us(T, 768) for T in DECODE_TS}
    return {"same_inputs": same, "fresh_inputs": fresh, "producer_written": produced, **variants,
            "empty_kernel_floor": floor}


def _graph_us(fn, calls_per_graph, replays=5):
    """Mean µs per call of a captured graph of fn(), which enqueues
    calls_per_graph calls (after one eager warm-up on a side stream)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(replays):
        g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (replays * calls_per_graph)


def producer_written_us(d, n=64):
    """The fused call's µs when a producer has just written its rows and
    shared output: n buffer sets, each rewritten by two device copies (the
    stand-ins for GEMM2 and the shared expert) right before its call. The
    result is the per-pair time minus the per-iteration time of the copies
    alone, both graph-replayed after a cache scrub."""
    calls = stacked_calls(d, n, "bf16")
    st = calls[0].keep[0]  # the stacked device inputs, [n, ...] per tensor
    rows, shared = st["expert_out"][0].clone(), st["shared_out"][0].clone()

    def produce(i):
        st["expert_out"][i].copy_(rows)
        st["shared_out"][i].copy_(shared)

    def pairs():
        for i in range(n):
            produce(i)
            calls[i]()

    def producers():
        for i in range(n):
            produce(i)
    scrub_infinity_cache()
    t_pair = _graph_us(pairs, n)
    scrub_infinity_cache()
    t_prod = _graph_us(producers, n)
    return round(t_pair - t_prod, 2)


def graph_ceiling_batch(reps=3):
    """The 512-token batch (H=6144, K=8): HBM-cold (a graph cycling over 8
    buffer sets, 604 MB > Infinity Cache) and cache-warm (one set). The cold
    figure is the median of reps timings (each 5 replays of 64 calls); their
    range is reported beside it."""
    import synth
    d = synth.config_inputs("batch512", 512)
    nbytes = synth.algorithmic_bytes(d["perm_idx"], d["H"], d["K"])
    sets = [to_device(d) for _ in range(8)]
    calls = [make_caller(dd, d["eps"], d["scale"])[0] for dd in sets]
    colds = sorted(time_graph(calls, 8, 5) * 1e3 for _ in range(reps))
    cold = colds[len(colds) // 2]
    warm = time_graph(calls[:1], 64, 5) * 1e3
    return {"us_cold": round(cold, 2), "gbs_cold": round(nbytes / (cold * 1e-6) / 1e9, 1),
            "frac_cold": round(nbytes / (cold * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "us_cold_range": [round(colds[0], 2), round(colds[-1], 2)], "reps": reps,
            "us_warm": round(warm, 2), "bytes": nbytes}


def make_dense_caller(d):
    """Zero-allocation closure for one dense residual add + RMSNorm call."""
    import numpy as np
    import torch
    import top_finalize_residual_amd as mfr

    def bf16(u):
        return torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).view(torch.bfloat16).cuda()
    x, res, g = bf16(d["x"]), bf16(d["residual"]), bf16(d["gamma"])
    ro, no = torch.empty_like(x), torch.empty_like(x)
    T, H, eps = d["T"], d["H"], d["eps"]

    def call():
        rc = mfr.residual_add_rmsnorm_raw(x.data_ptr(), res.data_ptr(), g.data_ptr(), eps,
                                          ro.data_ptr(), no.data_ptr(), T, H,
                                          torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(mfr.strerror(rc))
    call.keep = (x, res, g, ro, no)
    return call


def dense_figures():
    """The dense residual add + RMSNorm (no routed part) on the 8192-token
    chunk, HBM-cold (3 rotating buffer sets, 603 MB)."""
    import synth
    T, H = 8192, 6144
    d = synth.dense_inputs(T, H, seed=synth.seed_for("prefill", T), spike_frac=0.01)
    nbytes = synth.dense_algorithmic_bytes(T, H)
    calls = [make_dense_caller(d) for _ in range(3)]
    ms = time_calls(calls, 60, 6)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"prefill_T8192": {"us": round(ms * 1e3, 2), "gbs": round(gbs, 1),
                              "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes": nbytes}}


def _dense_fp8_caller(d):
    """A zero-allocation closure: one dense residual add + RMSNorm with FP8
    output (codes and scales, no bf16 normed output) on its own device copy."""
    import torch
    import top_finalize_residual_amd as mfr
    T, H = d["T"], d["H"]
    x, res, g = (torch.from_numpy(d[k].view("int16")).view(torch.bfloat16).cuda()
                 for k in ("x", "residual", "gamma"))
    ro = torch.empty_like(res)
    q = torch.empty((T, H), dtype=torch.uint8, device="cuda")
    sc = torch.empty((T,), dtype=torch.float32, device="cuda")

    def call():
        _raise_on(mfr.residual_add_rmsnorm_fp8_raw(
            x.data_ptr(), res.data_ptr(), g.data_ptr(), d["eps"], ro.data_ptr(), None,
            q.data_ptr(), sc.data_ptr(), T, H, torch.cuda.current_stream().cuda_stream))
    call.keep = (x, res, g, ro, q, sc)
    return call


def dense_fp8_figures():
    """The dense residual add + RMSNorm with its normalised output as per-token
    FP8 (no bf16 normed output) on the 8192-token chunk, HBM-cold (3 rotating
    buffer sets)."""
    import synth
    T, H = 8192, 6144
    d = synth.dense_inputs(T, H, seed=synth.seed_for("prefill", T), spike_frac=0.01)
    ms = time_calls([_dense_fp8_caller(d) for _ in range(3)], 60, 6)
    return {"prefill_T8192": dict(_rate(ms * 1e3, synth.dense_fp8_algorithmic_bytes(T, H)),
                                  bytes=synth.dense_fp8_algorithmic_bytes(T, H))}


def fp8_figures():
    """The fused op with its normalised output as per-token FP8 (no bf16 normed
    output) on the 8192-token chunk (HBM-cold by size)."""
    import torch
    import synth
    import top_finalize_residual_amd as mfr

    def caller(d):
        dd = to_device(d)
        T, K, H = d["T"], d["K"], d["H"]
        ro = torch.empty_like(dd["residual"])
        q = torch.empty((T, H), dtype=torch.uint8, device="cuda")
        sc = torch.empty((T,), dtype=torch.float32, device="cuda")
        a = [dd[k].data_ptr() for k in ("expert_out", "perm_idx", "topk_w", "shared_out",
                                        "residual", "gamma")]

        def call():
            rc = mfr.moe_finalize_rmsnorm_fp8_raw(*a, d["eps"], d["scale"], ro.data_ptr(), None,
                                                  q.data_ptr(), sc.data_ptr(), T, H, K,
                                                  torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(mfr.strerror(rc))
        call.keep = (dd, ro, q, sc)
        return call
    d = synth.config_inputs("prefill", 8192)
    nbytes = synth.fp8_algorithmic_bytes(d["perm_idx"], d["H"], d["K"])
    ms = time_calls([caller(d)], 60, 6)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"prefill_T8192": {"us": round(ms * 1e3, 2), "gbs": round(gbs, 1),
                              "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes": nbytes}}


def layout_figures(d, warmup=6, steps=60):
    """The headline workload in two row layouts, interleaved A/B/B/A: the
    uniformly random permutation the headline uses, and the rows grouped by
    expert as a grouped GEMM2 writes them (every value a token gathers is the
    same; only where the rows sit differs)."""
    import numpy as np
    import synth
    nbytes = synth.algorithmic_bytes(d["perm_idx"], d["H"], d["K"])
    sorted_perm = synth.expert_sorted_perm(d["experts"])
    moved = np.empty_like(d["expert_out"])
    moved[sorted_perm.reshape(-1)] = d["expert_out"][d["perm_idx"].reshape(-1)]
    ds = dict(d, expert_out=moved, perm_idx=sorted_perm)
    calls = {"random": make_caller(to_device(d), d["eps"], d["scale"])[0],
             "expert_sorted": make_caller(to_device(ds), d["eps"], d["scale"])[0]}
    us = {"random": [], "expert_sorted": []}
    for order in (("random", "expert_sorted"), ("expert_sorted", "random")):
        for n in order:
            us[n].append(time_calls([calls[n]], steps, warmup) * 1e3)
    return {"prefill_T8192": {n: _rate(sum(v) / len(v), nbytes) for n, v in us.items()}}


def _rate(us, nbytes):
    """µs per call, GB/s and fraction of the HBM peak for nbytes per call."""
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us": round(us, 2), "gbs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)}


def deferred_overhead():
    """Host cost of the torch-facing deferred path at one decode step (T=28):
    eager calls of fused_add_rmsnorm (the public consumer norm), of the same
    op through torch.ops directly (the dispatcher and the op's C++ kernel, as
    under torch.compile), and of the raw C call through the ctypes binding
    (pointers taken once, the current stream's handle per call), against the
    call replayed from a graph."""
    import torch
    import synth
    import top_finalize_residual_amd as mfr
    d = synth.config_inputs("decode", 28)
    dd = to_device(d)
    u = mfr.UnfinalizedMoEOutput(dd["expert_out"], dd["perm_idx"], dd["topk_w"], d["scale"])
    mo = mfr.MoEOutput(u, dd["shared_out"])
    ro, no = torch.empty_like(dd["residual"]), torch.empty_like(dd["residual"])
    op = torch.ops.mfr.moe_finalize_rmsnorm.default
    args = (dd["expert_out"], dd["perm_idx"], dd["topk_w"], dd["shared_out"], dd["residual"],
            dd["gamma"], d["eps"], d["scale"], ro, no)

    def via_public():
        mfr.fused_add_rmsnorm(mo, dd["residual"], dd["gamma"], d["eps"], residual_out=ro,
                              normed_out=no)

    def via_torch_ops():
        op(*args)
    raw, _ = make_caller(dd, d["eps"], d["scale"])
    out = {"T": 28}
    # interleaved, 3 rounds, median of each
    runs = {"eager_op_us": [], "torch_ops_us": [], "eager_raw_us": []}
    for _ in range(3):
        runs["eager_op_us"].append(time_calls([via_public], 300, 30) * 1e3)
        runs["torch_ops_us"].append(time_calls([via_torch_ops], 300, 30) * 1e3)
        runs["eager_raw_us"].append(time_calls([raw], 300, 30) * 1e3)
    for k, v in runs.items():
        out[k] = round(sorted(v)[1], 2)
    scrub_infinity_cache()  # the cache state of decode_latency's same_inputs
    out["graph_op_us"] = round(time_graph([via_public], 100, 5) * 1e3, 2)
    return out


SWEEP_TS = (64, 256, 257, 512, 1024, 2048, 8192)

# Alternatives to the shipped launch at the fused op's sizes, each reachable
# through the tuning interface as tuning.forced(**kwargs): a cap on the
# workgroups per CU (LDS reserved at launch), the per-XCD token ranges, every
# output store encoding, and the persistent kernel.
ALTERNATIVES = (
    ("auto", {}),
    ("no-cap", dict(residency=64)),
    ("cap-4-per-CU", dict(residency=4)),
    ("cap-3-per-CU", dict(residency=3)),
    ("cap-2-per-CU", dict(residency=2)),
    ("cap-1-per-CU", dict(residency=1)),
    ("xcd-ranges", dict(order=1)),
    ("store-wb", dict(store=1)),
    ("store-wt", dict(store=2)),
    ("store-nt", dict(store=3)),
    ("store-nt-wt", dict(store=4)),
    ("persist", dict(path=3)),
)
ALT_TS = (512, 1024, 2048, 4096, 8192)


def _shape_list():
    """The launch shapes of the shape sweep, as (name, tuning.forced kwargs)."""
    import top_finalize_residual_amd as mfr
    from top_finalize_residual_amd import tuning
    WB, WT = tuning.STORE_WRITE_BACK, tuning.STORE_WRITE_THROUGH
    shapes = [(f"v{v}-{'wb' if st == WB else 'wt'}", dict(path=mfr.PATH_STREAM, vpt=v, store=st))
              for v in (1, 2, 3, 4) for st in (WB, WT)]
    shapes += [("persist-wb", dict(path=mfr.PATH_PERSIST, store=WB)),
               ("persist-wt", dict(path=mfr.PATH_PERSIST, store=WT)), ("auto", {})]
    return shapes


def _sweep_workloads(ts, cold_bytes, states=False, H=6144, mode="bf16"):
    """(label, T, nbytes, calls, calls per set and graph, flushed) of each
    workload of a sweep at H (6144: the named workloads), K = 8. HBM-cold:
    one call on each of n
    buffer sets together above cold_bytes (more than twice the Infinity
    Cache); at T = 8192 one set (1.21 GB, cold by size) called 10 times in a
    row. With states, at T = 8192 also one set with the Infinity Cache
    flushed before every call (flushed: each call timed alone, see _sweep)
    and, for the bf16 fused op, one input set with two output sets
    alternated. mode: the call (stacked_calls)."""
    import synth
    for T in ts:
        cfg = None if H != 6144 else "prefill" if T == 8192 else "batch512" if T == 512 else None
        d = synth.config_inputs(cfg, T) if cfg else synth.generate(
            T, H, 8, scale=2.5, weights="top8_of_256",
            seed=synth.BASE_SEED + 9000 + T + (0 if H == 6144 else H))
        nb = (synth.algorithmic_bytes(d["perm_idx"], d["H"], d["K"]) if mode == "bf16" else
              synth.fp8_algorithmic_bytes(d["perm_idx"], d["H"], d["K"]) if mode == "fp8" else
              synth.dense_algorithmic_bytes(T, d["H"]))
        n = 1 if T == 8192 else max(2, -(-cold_bytes // nb))
        calls = stacked_calls(d, n, mode)
        yield str(T), T, nb, calls, 10 if n == 1 else 1, False
        if states and T == 8192:
            yield "8192, cache flushed", T, nb, calls, 5, True
            if mode == "bf16":
                del calls
                calls = mixed_calls(d, 1, 2)
                yield "8192, 2 output sets", T, nb, calls, 5, False
        del calls


def _flushed_us(call, n):
    """Median µs of n calls, each after 512 MB of unrelated reads and timed
    alone with events on its stream."""
    import torch
    st = torch.cuda.current_stream()
    ts = []
    for _ in range(n):
        scrub_infinity_cache()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        call()
        e1.record(st)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    return sorted(ts)[n // 2]


def _sweep(workloads, shapes, reps, phases, H=6144):
    """Times every shape on every workload: graphs of the workload's calls,
    after a cache scrub (or, for a flushed workload, each call alone after
    its own scrub), in forward then reverse shape order, reps times; the
    median per shape. With phases (a list), plain launches in the same order
    instead, each (workload, shape) group appended to phases as {label,
    dispatches, bytes}, so that a kernel trace of the run maps its
    dispatches to shapes by position."""
    import torch
    import top_finalize_residual_amd as mfr
    from top_finalize_residual_amd import tuning
    out = {}
    for label, T, nb, calls, per_call, flushed in workloads:
        times = {name: [] for name, _ in shapes}
        for r in range(reps):
            order = shapes if r % 2 == 0 else shapes[::-1]
            for name, force in order:
                scrub_infinity_cache()
                with tuning.forced(**force):
                    if phases is None:
                        times[name].append(_flushed_us(calls[0], per_call) if flushed else
                                           time_graph(calls, per_call, 3) * 1e3)
                        continue
                    for _ in range(per_call):
                        for c in calls:
                            if flushed:
                                scrub_infinity_cache()
                            c()
                    torch.cuda.synchronize()
                    phases.append({"label": f"T{label}/{name}",
                                   "dispatches": per_call * len(calls), "bytes": nb})
        if phases is not None:
            continue
        res = {name: round(sorted(v)[len(v) // 2], 2) for name, v in times.items()}
        auto_path = mfr.moe_finalize_rmsnorm_path(T, H, 8)
        res["auto_path"] = {1: "token", 2: "stream", 3: "persist"}.get(auto_path, "?")
        res["bytes"] = nb
        out[label] = res
        log(f"sweep {label}: " + ", ".join(f"{k} {v}" for k, v in res.items() if k != "bytes"))
    return out


def sweep_shapes(reps=3, cold_bytes=600_000_000, phases=None, ts=SWEEP_TS, H=6144):
    """Every launch shape at the fused op's workload sizes (K = 8; H = 6144
    unless asked otherwise): the one-token-per-workgroup kernel at 1..4
    vectors per thread (at H = 6144: 768, 384, 256 and 192 threads) with
    write-back and write-through stores, and the persistent kernel with both
    store policies, beside the automatic choice, in the HBM-cold harness of
    _sweep_workloads. The token and stream paths are automatic choices among
    these shapes.

    With phases (a list), the calls are launched eagerly instead (see
    _sweep)."""
    res = _sweep(_sweep_workloads(ts, cold_bytes, H=H), _shape_list(), reps, phases, H=H)
    return {"kind": "shapes", "H": H, "K": 8, "unit": "us", "reps": reps, "T": res}


def sweep_alternatives(reps=5, cold_bytes=600_000_000, phases=None, ts=ALT_TS, H=6144,
                       mode="bf16"):
    """The alternatives to the shipped launch (ALTERNATIVES) in the same
    harness, at T = 512..8192, and at T = 8192 also with the Infinity Cache
    flushed before every call and with two output sets alternated (the
    outputs then never meet their own lines in the Infinity Cache)."""
    res = _sweep(_sweep_workloads(ts, cold_bytes, states=True, H=H, mode=mode),
                 list(ALTERNATIVES), reps, phases, H=H)
    return {"kind": "alternatives", "mode": mode, "H": H, "K": 8, "unit": "us", "reps": reps,
            "T": res}


def run_sweep(args):
    import torch
    torch.cuda.set_device(0)
    alt = args.alternatives
    default_ts = ALT_TS if alt else SWEEP_TS
    ts = tuple(int(x) for x in args.sweep_ts.split(",")) if args.sweep_ts else default_ts
    kw = dict(reps=args.sweep_reps, ts=ts, H=args.sweep_h)
    if alt:
        fn, kw["mode"] = sweep_alternatives, args.sweep_mode
    else:
        fn = sweep_shapes
    if args.eager:
        phases = []
        fn(phases=phases, **kw)
        print(json.dumps({"phases": phases}), flush=True)
        return
    print(json.dumps({"shape_sweep": fn(**kw)}), flush=True)


COLD_TS = (1, 4, 16, 28, 64, 128, 256, 257, 384, 512, 513, 768, 1024, 2048, 4096, 8192)


def cold_table(ts=COLD_TS, reps=3, cold_bytes=600_000_000):
    """µs per call against T, automatic launch, H = 6144, K = 8, fresh
    inputs on every call: a graph of one call on each of n >= 2 buffer sets
    together above cold_bytes (more than twice the Infinity Cache), after a
    cache scrub; median of reps. For the fused op, its FP8-output form
    (codes and scales, no bf16 normed output) and the dense tail."""
    import torch
    import synth
    out = {}
    for T in ts:
        cfg = ("decode" if T in synth.CONFIGS["decode"]["Ts"] else "batch512" if T == 512 else
               "prefill" if T == 8192 else None)
        d = synth.config_inputs(cfg, T) if cfg else synth.generate(
            T, 6144, 8, scale=2.5, weights="top8_of_256", seed=synth.BASE_SEED + 9000 + T)
        row = {}
        for mode in ("bf16", "fp8", "dense"):
            nb = (synth.algorithmic_bytes(d["perm_idx"], d["H"], d["K"]) if mode == "bf16" else
                  synth.fp8_algorithmic_bytes(d["perm_idx"], d["H"], d["K"]) if mode == "fp8"
                  else synth.dense_algorithmic_bytes(T, d["H"]))
            n = max(2, -(-cold_bytes // nb))
            calls = stacked_calls(d, n, mode)
            ts_ = []
            for _ in range(reps):
                scrub_infinity_cache()
                ts_.append(time_graph(calls, 1, 3) * 1e3)
            del calls
            torch.cuda.empty_cache()
            us = sorted(ts_)[reps // 2]
            row[mode] = {"us": round(us, 2), "gbs": round(nb / (us * 1e-6) / 1e9, 1), "sets": n}
        out[str(T)] = row
        log(f"cold T={T}: " + ", ".join(f"{m} {v['us']}" for m, v in row.items()))
    return out


def cold_table_lines(path):
    """The cold_table JSON line as a table."""
    with open(path) as f:
        ct = next(json.loads(ln)["cold_table"] for ln in f if '"cold_table"' in ln)
    ts = list(ct)
    lines = ["µs per call (and TB/s of algorithmic bytes) against T, automatic launch, H = 6144, "
             "K = 8, fresh inputs on every call: graphs of one call on each of n buffer sets "
             "together above 600 MB, after a cache scrub, median of 3:", "",
             "| T | " + " | ".join(ts) + " |", "|---|" + "---|" * len(ts)]
    for mode, name in (("bf16", "fused, µs"), ("bf16", "fused, TB/s"), ("fp8", "FP8 output, µs"),
                       ("dense", "dense, µs")):
        key = "gbs" if "TB/s" in name else "us"
        cells = [f"{ct[t][mode][key] / 1000:.2f}" if key == "gbs" else f"{ct[t][mode][key]:.2f}"
                 for t in ts]
        lines.append(f"| {name} | " + " | ".join(cells) + " |")
    return lines


def summarize_cold(args):
    lines = [f"# {args.title}", "", "Commands ($REPO is the repository root, $OUT any output "
             "directory):", "", "```", args.command, "```", ""] + cold_table_lines(
                 args.summarize_cold) + ["", f"Kernel code hash of the library measured: "
                                             f"`{kernel_code_hash()}`."]
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# Input states of the bandwidth figures: (name, T, buffer sets cycled, calls
# per set and graph); see input_states().
STATE_PHASES = (
    ("prefill_T8192_1set", 8192, 1, 8),
    ("prefill_T8192_1set_cache_flushed", 8192, 1, 4),
    ("prefill_T8192_2sets", 8192, 2, 4),
    ("prefill_T8192_4sets", 8192, 4, 2),
    ("prefill_T8192_1input_2outputs", 8192, (1, 2), 4),
    ("prefill_T8192_2inputs_1output", 8192, (2, 1), 4),
    ("batch_T512_8sets_graph64", 512, 8, 8),
    ("batch_T512_32sets_graph64", 512, 32, 2),
    ("batch_T512_8sets_graph8", 512, 8, 1),
)


def mixed_calls(d, n_in, n_out):
    """Closures for the fused op that cycle n_in input sets and n_out output
    sets independently (call j reads input set j % n_in and writes output set
    j % n_out), max(n_in, n_out) of them, with n_in, n_out in {1, 2}."""
    import torch
    import top_finalize_residual_amd as mfr
    sets = [to_device(d) for _ in range(n_in)]
    T, K = sets[0]["perm_idx"].shape
    H = sets[0]["gamma"].shape[0]
    outs = [(torch.empty_like(sets[0]["residual"]), torch.empty_like(sets[0]["residual"]))
            for _ in range(n_out)]
    names = ("expert_out", "perm_idx", "topk_w", "shared_out", "residual", "gamma")
    calls = []
    for j in range(max(n_in, n_out)):
        a = [sets[j % n_in][k].data_ptr() for k in names]
        r, n = (t.data_ptr() for t in outs[j % n_out])

        def call(a=a, r=r, n=n):
            _raise_on(mfr.moe_finalize_rmsnorm_raw(*a, d["eps"], d["scale"], r, n, T, H, K,
                                                   torch.cuda.current_stream().cuda_stream))
        call.keep = (sets, outs)
        calls.append(call)
    return calls


def _state_sets(cache, T, n, inputs):
    """Calls over n device copies of the workload at T (shared between
    phases), or over (inputs, outputs) copies cycled independently."""
    import synth
    cfg = "prefill" if T == 8192 else "batch512"
    key = (T, n)
    if key not in cache:
        if T not in inputs:
            inputs[T] = synth.config_inputs(cfg, T)
        cache[key] = (mixed_calls(inputs[T], *n) if isinstance(n, tuple) else
                      stacked_calls(inputs[T], n, "bf16"))
    return cache[key]


def input_states(reps=3, eager=False, log_phase=None, prefill=None):
    """The fused op at T = 8192 and 512 in the input states its bandwidth
    depends on: one buffer set re-read call after call, or several distinct
    sets cycled (1, 2 and 4 sets of 1.41 GB at T = 8192; 8 and 32 sets of
    75.5 MB at T = 512); one set re-read with the Infinity Cache flushed
    before every call (512 MB of unrelated reads; each call then timed alone
    with events); and inputs and outputs cycled apart (one input set with two
    output sets, two input sets with one output set). Each other phase times graphs of n_sets x per_set calls
    (median of reps), or, with eager, plain launches in the same order (for
    a counter run, whose dispatches then map to phases by position)."""
    import synth
    cache = {}
    inputs = {} if prefill is None else {8192: prefill}
    out = {}
    import torch
    for name, T, n, per_set in STATE_PHASES:
        calls = _state_sets(cache, T, n, inputs)
        nb = synth.config_algorithmic_bytes("prefill" if T == 8192 else "batch512", T)
        flushed = name.endswith("_cache_flushed")
        if eager:
            for _ in range(per_set):
                for c in calls:
                    if flushed:
                        scrub_infinity_cache()
                    c()
            torch.cuda.synchronize()
            if log_phase:
                log_phase(name, per_set * len(calls))
            continue
        scrub_infinity_cache()
        if flushed:
            # one call at a time, each after 512 MB of unrelated reads, timed
            # alone with events on its stream
            st = torch.cuda.current_stream()
            ts = []
            for _ in range(2 * per_set + 1):
                scrub_infinity_cache()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(st)
                calls[0]()
                e1.record(st)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3)
            ts.sort()
            us = ts[len(ts) // 2]
            out[name] = {"us": round(us, 2),
                         "frac": round(nb / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4), "input_sets": 1,
                         "output_sets": 1, "calls_per_graph": None}
            continue
        ts = sorted(time_graph(calls, per_set, 3) * 1e3 for _ in range(reps))
        us = ts[len(ts) // 2]
        n_in, n_out = n if isinstance(n, tuple) else (n, n)
        out[name] = {"us": round(us, 2), "frac": round(nb / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                     "input_sets": n_in, "output_sets": n_out,
                     "calls_per_graph": len(calls) * per_set}
        if T == 8192 and n == 4:
            del cache[(T, 1)], cache[(T, 2)]  # keep the device footprint bounded
    return out


def run_states(args):
    """Eager launches of every input-state phase, in order, for a counter
    run; prints the phase table (name, dispatches) as JSON."""
    import torch
    torch.cuda.set_device(0)
    import synth
    phases = []

    def add(name, n):
        T = 8192 if "T8192" in name else 512
        nb = synth.config_algorithmic_bytes("prefill" if T == 8192 else "batch512", T)
        phases.append({"label": name, "dispatches": n, "bytes": nb})
    input_states(eager=True, log_phase=add)
    print(json.dumps({"phases": phases}), flush=True)


def run_persist_counters(args):
    """For a counter run: the automatic (grid of tokens) and the persistent
    launch of the fused op at T = 512, 2048 and 8192 (H = 6144, K = 8), a few
    calls each on one buffer set, then one 1 GiB copy of known size for the
    counters' calibration; prints the phase table."""
    import torch
    import synth
    import top_finalize_residual_amd as mfr
    from top_finalize_residual_amd import tuning
    torch.cuda.set_device(0)
    phases = []
    for T in (512, 2048, 8192):
        cfg = "prefill" if T == 8192 else "batch512" if T == 512 else None
        d = synth.config_inputs(cfg, T) if cfg else synth.generate(
            T, 6144, 8, scale=2.5, weights="top8_of_256", seed=synth.BASE_SEED + 9000 + T)
        nb = synth.algorithmic_bytes(d["perm_idx"], d["H"], d["K"])
        call = stacked_calls(d, 1, "bf16")[0]
        for name, path in (("auto", 0), ("persist", mfr.PATH_PERSIST)):
            with tuning.forced(path):
                for _ in range(args.steps):
                    call()
            torch.cuda.synchronize()
            phases.append({"label": f"T{T}/{name}", "dispatches": args.steps, "bytes": nb})
        del call
    probe_ceilings(reps=1)
    print(json.dumps({"phases": phases}), flush=True)


def run_latency(args):
    """Eager calls for a kernel trace, small sizes first so that no large call
    has flushed the caches before them: the fused op at the decode sizes, the
    FP8-output call and the dense tail at T = 28, the 512-token batch, then
    the dense tail and the FP8-output call at T = 8192, and last the dense
    tail with FP8 output at T = 28 and 8192."""
    import torch
    import synth
    torch.cuda.set_device(0)

    def run(call, n, what):
        for _ in range(n):
            call()
        torch.cuda.synchronize()
        log(f"{what}: {n} calls")
    for T in DECODE_TS:
        d = synth.config_inputs("decode", T)
        run(make_caller(to_device(d), d["eps"], d["scale"])[0], args.steps, f"T={T}")
    run(stacked_calls(synth.config_inputs("decode", 28), 1, "fp8")[0], args.steps, "fp8 output T=28")
    run(make_dense_caller(synth.dense_inputs(28, 6144, seed=synth.seed_for("prefill", 28))),
        args.steps, "dense T=28")
    d = synth.config_inputs("batch512", 512)
    run(make_caller(to_device(d), d["eps"], d["scale"])[0], args.steps, "T=512")
    run(make_dense_caller(synth.dense_inputs(8192, 6144, seed=synth.seed_for("prefill", 8192))),
        20, "dense T=8192")
    run(stacked_calls(synth.config_inputs("prefill", 8192), 1, "fp8")[0], 20, "fp8 output T=8192")
    run(_dense_fp8_caller(synth.dense_inputs(28, 6144, seed=synth.seed_for("prefill", 28))),
        args.steps, "dense fp8 output T=28")
    run(_dense_fp8_caller(synth.dense_inputs(8192, 6144, seed=synth.seed_for("prefill", 8192))),
        20, "dense fp8 output T=8192")


def run_bench(args):
    import numpy as np  # noqa: F401
    import torch
    import synth
    import top_finalize_residual_amd as mfr

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    torch.cuda.set_device(0)
    log(f"generating the {HEADLINE_T}-token prefill chunk (seeded, synthetic)")
    d = synth.config_inputs(HEADLINE_CFG, HEADLINE_T)
    nbytes = synth.algorithmic_bytes(d["perm_idx"], d["H"], d["K"])
    dd = to_device(d)
    path = mfr.moe_finalize_rmsnorm_path(d["T"], d["H"], d["K"])
    call, _ = make_caller(dd, d["eps"], d["scale"])
    log(f"warmup {args.warmup}, timing {args.steps} calls (path {path})")
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(args.steps):
        call()
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"{ms * 1e3:.1f} us/call, {gbs:.0f} GB/s")

    rec = {"metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "us_per_call": round(ms * 1e3, 2), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": "prefill chunk: T=8192 tokens, H=6144, K=8, scale 2.5, "
                                  "1% residual rows x100 (1.21 GB per call; one buffer set, "
                                  "calls back to back; other input states in input_states)",
                      "T": d["T"], "H": d["H"], "K": d["K"], "algorithmic_bytes": nbytes,
                      "path": {1: "token", 2: "stream"}.get(path, "?"),
                      "parallelism": "single GPU"}}
    rec["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                       "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                       "traffic": traffic_for_headline()}
    if not args.no_extras:
        log("measured ceilings (1 GiB copy, read and write probes)")
        cp, rd, wr = probe_ceilings()
        rec["probe_ceilings_gbs"] = {"copy": round(cp, 1), "read_only": round(rd, 1),
                                     "write_only": round(wr, 1)}
        # the headline against the copy kernel's ceiling of the same run
        rec["headline_of_copy_ceiling"] = round(gbs / cp, 4)
        log("mixed-stream probe at the chunk's read and write bytes (bf16 and FP8 output)")
        mix = mix_probe_ceilings()
        rec["probe_ceilings_gbs"]["mix_bf16"] = mix["bf16"]["gbs"]
        rec["probe_ceilings_gbs"]["mix_fp8"] = mix["fp8"]["gbs"]
        rec["mix_probe"] = mix
        rec["mix_probe"]["headline_of_mix"] = round(gbs / mix["bf16"]["gbs"], 4)
        log("decode latency, T = 1..64 (H=6144, K=8), graph-replayed, same and fresh inputs")
        rec["decode_latency_us"] = decode_latency()
        log("512-token batch, cold and warm")
        rec["batch_512"] = graph_ceiling_batch()
        log("dense residual add + RMSNorm (no routed part)")
        rec["dense_residual_rmsnorm"] = dense_figures()
        log("FP8 (E4M3 per-token) normalised output")
        rec["fp8_output"] = fp8_figures()
        rec["mix_probe"]["fp8_of_mix"] = round(
            rec["fp8_output"]["prefill_T8192"]["gbs"] / mix["fp8"]["gbs"], 4)
        log("dense residual add + RMSNorm with FP8 output")
        rec["dense_fp8_output"] = dense_fp8_figures()
        log("row layouts: random permutation against rows grouped by expert")
        rec["row_layouts"] = layout_figures(d)
        log("deferred-finalize torch path: host overhead")
        rec["deferred_path"] = deferred_overhead()
        log("input states: one buffer set re-read, or several cycled (T = 8192 and 512)")
        rec["input_states"] = input_states(prefill=d)
    if not args.no_cpu_baseline:
        log("oracle CPU baseline on the same workload (single thread)")
        rec["cpu_baseline"] = cpu_baseline(d)
    print(json.dumps(rec), flush=True)


def run_pmc(args):
    """Short run for counter collection: the headline fused call a few times,
    then one 1 GiB copy of known size."""
    import torch
    import synth
    torch.cuda.set_device(0)
    d = synth.config_inputs(HEADLINE_CFG, HEADLINE_T)
    dd = to_device(d)
    call, _ = make_caller(dd, d["eps"], d["scale"])
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    probe_ceilings(reps=1)
    log("pmc run done")


def run_pmc_variants(args):
    """Short run for counter collection on the 8192-token chunk: the dense
    residual add + RMSNorm, the FP8-output call, then one 1 GiB copy of known
    size."""
    import torch
    import synth
    torch.cuda.set_device(0)
    T = HEADLINE_T
    dense = make_dense_caller(synth.dense_inputs(T, 6144, seed=synth.seed_for(HEADLINE_CFG, T),
                                                 spike_frac=0.01))
    for _ in range(args.steps):
        dense()
    torch.cuda.synchronize()
    del dense
    fp8 = stacked_calls(synth.config_inputs(HEADLINE_CFG, T), 1, "fp8")[0]
    for _ in range(args.steps):
        fp8()
    torch.cuda.synchronize()
    del fp8
    dense_fp8 = _dense_fp8_caller(synth.dense_inputs(T, 6144, seed=synth.seed_for(HEADLINE_CFG, T),
                                                     spike_frac=0.01))
    for _ in range(args.steps):
        dense_fp8()
    torch.cuda.synchronize()
    del dense_fp8
    probe_ceilings(reps=1)
    log("pmc variants run done")


def summarize_trace(args):
    """Per (kernel, grid, workgroup) durations from a rocprofv3 kernel_trace.csv."""
    import statistics
    groups = {}
    for r in csv.DictReader(open(args.summarize_trace)):
        name = r["Kernel_Name"]
        if args.kernel_filter and args.kernel_filter not in name:
            continue
        key = (name, int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"# rocprofv3 kernel trace: {args.title}", "",
             "Commands ($REPO is the repository root, $OUT any output directory):", "",
             "```", args.command, "```", "",
             "| kernel | grid (threads) | workgroup | tokens | calls | avg µs | median µs | p10 µs | p90 µs | min µs | max µs |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for (name, grid, wg), v in sorted(groups.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        short = name.split("(")[0]  # without the argument list
        q = sorted(v)
        p10, p90 = q[int(0.1 * (len(q) - 1))], q[int(0.9 * (len(q) - 1))]
        lines.append(f"| `{short}` | {grid} | {wg} | {grid // wg} | {len(v)} | {statistics.mean(v):.2f} | "
                     f"{statistics.median(v):.2f} | {p10:.2f} | {p90:.2f} | {min(v):.2f} | {max(v):.2f} |")
    if args.stats_csv:
        with open(args.stats_csv) as f:
            stats = f.read().strip()
        lines += ["", "rocprofv3's own `--stats` summary of the same run (`*_kernel_stats.csv`, verbatim):",
                  "", "```", stats, "```"]
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


FUSED_KERNELS = ("mfr_fused_kernel", "mfr_persist_kernel")


def _dispatch_rows(path):
    """Rows of a rocprofv3 kernel_trace.csv or counter_collection.csv, in
    dispatch order."""
    rows = list(csv.DictReader(open(path)))
    key = "Dispatch_Id" if rows and "Dispatch_Id" in rows[0] else "Correlation_Id"
    if rows and key in rows[0]:
        rows.sort(key=lambda r: int(r[key]))
    return rows


def summarize_phases(args):
    """Durations (from a kernel trace) or counters (from counter runs) of the
    fused kernels of a phase run, attributed to its phases by dispatch order:
    the n-th fused-kernel dispatch of the run belongs to the phase whose
    dispatch range holds n. Counter files give one value per dispatch and
    counter; FETCH_SIZE and WRITE_SIZE are also calibrated on the 1 GiB copy
    probe of the same run when present, as traffic against each phase's
    algorithmic bytes."""
    import statistics
    with open(args.phases_json) as f:
        phases = None
        for ln in f:
            ln = ln.strip()
            if ln.startswith("{") and '"phases"' in ln:
                phases = json.loads(ln)["phases"]
    if phases is None:
        raise SystemExit(f"no phase table in {args.phases_json}")
    bounds, n = [], 0
    for ph in phases:
        bounds.append((n, n + ph["dispatches"], ph["label"]))
        n += ph["dispatches"]
    label_of = {}
    for a, b, label in bounds:
        for i in range(a, b):
            label_of[i] = label
    order = list(dict.fromkeys(ph["label"] for ph in phases))
    nbytes = {ph["label"]: ph.get("bytes") for ph in phases}
    lines = [f"# {args.title}", "", "Commands ($REPO is the repository root, $OUT any output "
             "directory):", "", "```", args.command, "```", ""]
    if args.trace_csv:
        rows = [r for r in _dispatch_rows(args.trace_csv)
                if any(k in r["Kernel_Name"] for k in FUSED_KERNELS)]
        if len(rows) != n:
            raise SystemExit(f"{len(rows)} fused-kernel dispatches in the trace, {n} in the phases")
        per = {}
        names = {}
        for i, r in enumerate(rows):
            lab = label_of[i]
            per.setdefault(lab, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            names.setdefault(lab, set()).add((r["Kernel_Name"].split("(")[0].replace("void ", ""),
                                              int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"])))
        lines += ["| phase | kernel (grid threads / workgroup) | dispatches | avg µs | median µs | "
                  "min µs | max µs | GB/s (median) |", "|---|---|---|---|---|---|---|---|"]
        for lab in order:
            v = per[lab]
            med = statistics.median(v)
            kn = "; ".join(f"`{k}` ({g}/{w})" for k, g, w in sorted(names[lab]))
            gbs = f"{nbytes[lab] / (med * 1e-6) / 1e9:,.0f}" if nbytes.get(lab) else ""
            lines.append(f"| {lab} | {kn} | {len(v)} | {statistics.mean(v):.2f} | {med:.2f} | "
                         f"{min(v):.2f} | {max(v):.2f} | {gbs} |")
    else:
        vals = {}  # (label, counter) -> values
        copy = {}
        for path in args.counter_csv:
            rows = _dispatch_rows(path)
            counters = sorted({r["Counter_Name"] for r in rows})
            for c in counters:
                fused = [r for r in rows if r["Counter_Name"] == c and
                         any(k in r["Kernel_Name"] for k in FUSED_KERNELS)]
                if len(fused) != n:
                    raise SystemExit(f"{path}: {len(fused)} fused-kernel values of {c}, "
                                     f"{n} dispatches in the phases")
                for i, r in enumerate(fused):
                    vals.setdefault((label_of[i], c), []).append(float(r["Counter_Value"]))
                cp = [float(r["Counter_Value"]) for r in rows if r["Counter_Name"] == c and
                      "mfr_copy_probe_kernel" in r["Kernel_Name"]]
                if cp:
                    copy[c] = sum(cp) / len(cp)
        counters = sorted({c for _, c in vals})
        lines += ["Mean per dispatch, by phase.", "",
                  "| phase | " + " | ".join(counters) + " |",
                  "|---|" + "---|" * len(counters)]
        for lab in order:
            lines.append(f"| {lab} | " + " | ".join(
                f"{statistics.mean(vals[(lab, c)]):,.1f}" if (lab, c) in vals else ""
                for c in counters) + " |")
        derived = [
            ("UTCL1 translation misses per request", "TCP_UTCL1_TRANSLATION_MISS_sum",
             "TCP_UTCL1_REQUEST_sum", 1.0, "{:.2e}"),
            ("TCP to L2 mean read latency (cycles)", "TCP_TCC_READ_REQ_LATENCY_sum",
             "TCP_TCC_READ_REQ_sum", 1.0, "{:,.0f}"),
            ("L2 to memory mean read latency (cycles)", "TCC_EA0_RDREQ_LEVEL_sum",
             "TCC_EA0_RDREQ_sum", 1.0, "{:,.0f}"),
            ("UTCL2 busy share of GPU-active cycles", "GRBM_UTCL2_BUSY", "GRBM_GUI_ACTIVE", 1.0,
             "{:.4f}"),
        ]
        have = [d for d in derived if any((lab, d[1]) in vals and (lab, d[2]) in vals
                                          for lab in order)]
        if have:
            lines += ["", "Derived, per phase (ratios of the per-dispatch means above):", "",
                      "| phase | " + " | ".join(d[0] for d in have) + " |",
                      "|---|" + "---|" * len(have)]
            for lab in order:
                cells = []
                for _, num, den, k, fmt in have:
                    if (lab, num) in vals and (lab, den) in vals:
                        d_ = statistics.mean(vals[(lab, den)])
                        cells.append(fmt.format(k * statistics.mean(vals[(lab, num)]) / d_)
                                     if d_ else "")
                    else:
                        cells.append("")
                lines.append(f"| {lab} | " + " | ".join(cells) + " |")
        if "FETCH_SIZE" in copy and "WRITE_SIZE" in copy:
            cf = (1 << 30) / (copy["FETCH_SIZE"] * 1024.0)
            cw = (1 << 30) / (copy["WRITE_SIZE"] * 1024.0)
            lines += ["", f"Calibrated on the 1 GiB copy probe of the same runs: FETCH_SIZE x "
                      f"{cf:.4f}, WRITE_SIZE x {cw:.4f} (KiB per dispatch to bytes).", "",
                      "| phase | traffic B per dispatch | algorithmic B | ratio |", "|---|---|---|---|"]
            for lab in order:
                if (lab, "FETCH_SIZE") in vals and (lab, "WRITE_SIZE") in vals:
                    t = (statistics.mean(vals[(lab, "FETCH_SIZE")]) * 1024.0 * cf +
                         statistics.mean(vals[(lab, "WRITE_SIZE")]) * 1024.0 * cw)
                    alg = nbytes.get(lab)
                    lines.append(f"| {lab} | {t:,.0f} | {alg:,} | {t / alg:.4f} |" if alg else
                                 f"| {lab} | {t:,.0f} | | |")
    if args.append_sweep:
        lines += [""] + sweep_table_lines(args.append_sweep)
    if args.append_states:
        lines += [""] + states_table_lines(args.append_states)
    lines += ["", f"Kernel code hash of the library measured: `{kernel_code_hash()}`."]
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_sweep(args):
    """A profiles/ page from the JSON line of bench.py --shape-sweep alone."""
    lines = [f"# {args.title}", "", "Commands ($REPO is the repository root, $OUT any output "
             "directory):", "", "```", args.command, "```", ""] + sweep_table_lines(
                 args.summarize_sweep) + ["", f"Kernel code hash of the library measured: "
                                              f"`{kernel_code_hash()}`."]
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def states_table_lines(path):
    """The input_states figures of a bench.py JSON line as a table."""
    with open(path) as f:
        st = next(json.loads(ln)["input_states"] for ln in f if '"input_states"' in ln)
    lines = ["Event timing of the same states in the benchmark run (`input_states` of the "
             "bench.py JSON line; graphs of the listed number of calls, median of 3, except "
             "the flushed state, timed one call at a time after 512 MB of unrelated reads):", "",
             "| state | input sets | output sets | calls per graph | µs per call | "
             "% of 8 TB/s |", "|---|---|---|---|---|---|"]
    for name, v in st.items():
        lines.append(f"| {name} | {v['input_sets']} | {v['output_sets']} | "
                     f"{v['calls_per_graph'] or 'one at a time'} | {v['us']:.2f} | "
                     f"{100 * v['frac']:.1f} |")
    return lines


def sweep_table_lines(path):
    """The graph-timed shape sweep (the JSON line of bench.py --shape-sweep)
    as a table: µs per call per shape and T, the fastest shape marked."""
    with open(path) as f:
        sw = next(json.loads(ln)["shape_sweep"] for ln in f if '"shape_sweep"' in ln)
    ts = list(sw["T"])
    shapes = [k for k in sw["T"][ts[0]] if k not in ("auto_path", "bytes")]
    alt = sw.get("kind") == "alternatives"
    what, flag = ("alternatives", "--shape-sweep --alternatives") if alt else ("shapes",
                                                                            "--shape-sweep")
    call = {"fp8": "the FP8-output call", "dense": "the dense tail"}.get(sw.get("mode"),
                                                                      "the fused op")
    lines = [f"Event timing of the same {what} for {call} at H = {sw['H']}, K = {sw['K']} "
             f"(`bench.py {flag}`: graphs of one call per "
             f"buffer set, or of 10 calls on one set at T = 8192 and 5 calls over two output "
             f"sets; with the cache flushed, the median of 5 calls each timed alone after 512 MB "
             f"of unrelated reads; median of {sw['reps']} interleaved repetitions), µs per call; "
             "the fastest "
             "of each column in bold, `auto` is the library's own choice (its path in the last "
             "row):", "",
             "| " + what[:-1] + " | " + " | ".join(f"T = {t}" for t in ts) + " |",
             "|---|" + "---|" * len(ts)]
    best = {t: min(v for k, v in sw["T"][t].items() if k in shapes) for t in ts}
    for sh in shapes:
        cells = []
        for t in ts:
            v = sw["T"][t][sh]
            cells.append(f"**{v:.2f}**" if v == best[t] else f"{v:.2f}")
        lines.append(f"| {sh} | " + " | ".join(cells) + " |")
    lines.append("| auto path | " + " | ".join(sw["T"][t]["auto_path"] for t in ts) + " |")
    return lines


def summarize_pmc(args):
    """FETCH_SIZE and WRITE_SIZE per dispatch (KiB), calibrated on the copy."""
    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r.get("Counter_Name") != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals
    fetch = per_kernel(args.fetch_csv, "FETCH_SIZE")
    write = per_kernel(args.write_csv, "WRITE_SIZE")

    def pick(vals, key):
        ks = [k for k in vals if key in k]
        if not ks:
            raise SystemExit(f"no kernel matching {key}")
        v = vals[ks[0]]
        return ks[0], sum(v) / len(v)
    copy_bytes = 1 << 30
    fk, f_fused = pick(fetch, "mfr_fused_kernel")
    _, w_fused = pick(write, "mfr_fused_kernel")
    _, f_copy = pick(fetch, "mfr_copy_probe_kernel")
    _, w_copy = pick(write, "mfr_copy_probe_kernel")
    cf = copy_bytes / (f_copy * 1024.0)
    cw = copy_bytes / (w_copy * 1024.0)
    import synth
    alg = synth.config_algorithmic_bytes(HEADLINE_CFG, HEADLINE_T)
    traffic = f_fused * 1024.0 * cf + w_fused * 1024.0 * cw
    out = {"kernel": fk, "code_hash": kernel_code_hash(),
           "fetch_kib_per_dispatch": f_fused, "write_kib_per_dispatch": w_fused,
           "copy_probe": {"bytes": copy_bytes, "fetch_kib": f_copy, "write_kib": w_copy,
                          "fetch_scale": cf, "write_scale": cw},
           "traffic_bytes_per_launch": round(traffic), "algorithmic_bytes": alg,
           "traffic_over_algorithmic": traffic / alg, "commands": args.command}
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def _fused_template_args(name):
    """(VPT, KT, OUT_AUX, QM, ROWS) of an mfr_fused_kernel name, as strings."""
    inside = name[name.index("<") + 1:name.index(">")]
    return tuple(a.strip() for a in inside.split(","))


def variant_algorithmic_bytes(name, T=HEADLINE_T):
    """Closed-form algorithmic bytes of one launch of a fused-kernel variant on
    the T-token prefill chunk: the dense tail (KT = -1), the FP8-output modes
    (QM 1: codes and scale, QM 2: also the bf16 normed output), else the
    bf16 fused op."""
    import synth
    _, kt, _, qm, _ = _fused_template_args(name)
    H = synth.CONFIGS[HEADLINE_CFG]["H"]
    if kt == "-1":
        if qm in ("1", "2"):
            return synth.dense_fp8_algorithmic_bytes(T, H, bf16_normed=qm == "2")
        return synth.dense_algorithmic_bytes(T, H)
    if qm in ("1", "2"):
        return synth.config_fp8_algorithmic_bytes(HEADLINE_CFG, T, bf16_normed=qm == "2")
    return synth.config_algorithmic_bytes(HEADLINE_CFG, T)


def summarize_pmc_variants(args):
    """FETCH_SIZE and WRITE_SIZE of every fused-kernel variant in the run,
    calibrated on the copy probe of the same run, against each variant's
    algorithmic bytes."""
    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r.get("Counter_Name") == counter:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in vals.items()}
    fetch = per_kernel(args.fetch_csv, "FETCH_SIZE")
    write = per_kernel(args.write_csv, "WRITE_SIZE")
    copy = [k for k in fetch if "mfr_copy_probe_kernel" in k]
    if not copy or copy[0] not in write:
        raise SystemExit("no copy probe in the counter files")
    copy_bytes = 1 << 30
    cf = copy_bytes / (fetch[copy[0]] * 1024.0)
    cw = copy_bytes / (write[copy[0]] * 1024.0)
    rows, out = [], {"code_hash": kernel_code_hash(), "fetch_scale": cf, "write_scale": cw,
                     "kernels": {}, "commands": args.command}
    for name in sorted(k for k in fetch if "mfr_fused_kernel" in k and k in write):
        short = name.split("(")[0].replace("void ", "")
        alg = variant_algorithmic_bytes(name)
        traffic = fetch[name] * 1024.0 * cf + write[name] * 1024.0 * cw
        out["kernels"][short] = {"fetch_kib": fetch[name], "write_kib": write[name],
                                 "traffic_bytes": round(traffic), "algorithmic_bytes": alg,
                                 "ratio": traffic / alg}
        rows.append(f"| `{short}` | {fetch[name]:,.0f} | {write[name]:,.0f} | {traffic:,.0f} | "
                    f"{alg:,} | {traffic / alg:.4f} |")
    lines = [f"# HBM traffic: {args.title}", "",
             "Commands ($REPO is the repository root, $OUT any output directory):", "",
             "```", args.command, "```", "",
             f"Calibration on the 1 GiB copy probe of the same run: FETCH_SIZE x {cf:.4f}, "
             f"WRITE_SIZE x {cw:.4f}. Traffic = calibrated fetch + write bytes per dispatch; "
             "the ratio is traffic over the variant's algorithmic bytes.", "",
             "| kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | traffic B | "
             "algorithmic B | ratio |", "|---|---|---|---|---|---|"] + rows
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    if args.json_out:
        with open(args.json_out, "w") as f:
            json.dump(out, f, indent=1)
    print("\n".join(lines))


# Shader-engine counters gathered in three rocprofv3 --pmc passes (each within
# one pass's per-block limits); the summary joins them per kernel launch shape.
COUNTER_PASSES = (
    ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR", "SQ_INSTS_LDS",
     "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_SALU"),
    ("TCC_HIT_sum", "TCC_MISS_sum"),
    ("VALUBusy", "OccupancyPercent"),
)


def summarize_counters(args):
    """Per (kernel, grid, workgroup): the mean of each counter over its
    dispatches, from any number of rocprofv3 counter_collection.csv files.
    Derived here: L2 hit rate = hits / (hits + misses), and instructions per
    wave. VALUBusy and OccupancyPercent are rocprofv3's own derived counters."""
    groups = {}
    for path in args.counter_csv:
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            if args.kernel_filter and args.kernel_filter not in name:
                continue
            key = (name.split("(")[0].replace("void ", ""), int(r["Grid_Size"]),
                   int(r["Workgroup_Size"]))
            g = groups.setdefault(key, {"vgpr": r["VGPR_Count"], "sgpr": r["SGPR_Count"],
                                        "lds": r["LDS_Block_Size"], "c": {}})
            g["c"].setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))

    def mean(g, c):
        v = g["c"].get(c)
        return sum(v) / len(v) if v else None

    def fmt(x, nd=1):
        return "—" if x is None else f"{x:,.{nd}f}"
    rows, out = [], {}
    for (name, grid, wg), g in sorted(groups.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        waves = mean(g, "SQ_WAVES")
        hit, miss = mean(g, "TCC_HIT_sum"), mean(g, "TCC_MISS_sum")
        l2 = 100.0 * hit / (hit + miss) if hit is not None and miss is not None and hit + miss > 0 else None

        def per_wave(c):
            v = mean(g, c)
            return v / waves if v is not None and waves else None
        n_disp = max(len(v) for v in g["c"].values())
        rec = {"dispatches": n_disp, "waves": waves, "vgpr": int(g["vgpr"]), "sgpr": int(g["sgpr"]),
               "lds_bytes": int(g["lds"]), "occupancy_pct": mean(g, "OccupancyPercent"),
               "valu_busy_pct": mean(g, "VALUBusy"), "valu_per_wave": per_wave("SQ_INSTS_VALU"),
               "salu_per_wave": per_wave("SQ_INSTS_SALU"),
               "vmem_rd_per_wave": per_wave("SQ_INSTS_VMEM_RD"),
               "vmem_wr_per_wave": per_wave("SQ_INSTS_VMEM_WR"), "lds_per_wave": per_wave("SQ_INSTS_LDS"),
               "lds_bank_conflict": mean(g, "SQ_LDS_BANK_CONFLICT"),
               "l2_hit_pct": l2,
               "l2_hit": hit, "l2_miss": miss}
        out[f"{name} grid={grid} wg={wg}"] = rec
        rows.append(f"| `{name}` | {grid // wg} × {wg} | {n_disp} | {rec['vgpr']} / {rec['sgpr']} / "
                    f"{rec['lds_bytes']} | {fmt(waves, 0)} | {fmt(rec['occupancy_pct'])} | "
                    f"{fmt(rec['valu_busy_pct'])} | {fmt(rec['valu_per_wave'])} | "
                    f"{fmt(rec['salu_per_wave'])} | {fmt(rec['vmem_rd_per_wave'])} | "
                    f"{fmt(rec['vmem_wr_per_wave'])} | {fmt(rec['lds_per_wave'])} | "
                    f"{fmt(rec['lds_bank_conflict'], 0)} | {fmt(l2)} |")
    lines = [f"# rocprofv3 counters: {args.title}", "",
             "Commands ($REPO is the repository root, $OUT any output directory):", "",
             "```", args.command, "```", "",
             "Per launch shape, means over its dispatches. VGPR / SGPR / LDS are rocprofv3's columns "
             "(LDS in bytes); on gfx950 its VGPR figure is half the compiler's allocation (143 registers "
             "show as 72), so waves per SIMD follow from the compiler's count. Occupancy and VALU busy are rocprofv3's derived `OccupancyPercent` "
             "and `VALUBusy`; per-wave columns are instruction counts divided by `SQ_WAVES`; the LDS "
             "column is `SQ_LDS_BANK_CONFLICT` per dispatch; L2 hit = `TCC_HIT_sum` / (`TCC_HIT_sum` + "
             "`TCC_MISS_sum`).", "",
             "| kernel | workgroups × threads | dispatches | VGPR / SGPR / LDS | waves | occupancy % | "
             "VALU busy % | VALU / wave | SALU / wave | VMEM rd / wave | VMEM wr / wave | LDS / wave | "
             "LDS bank conflict | L2 hit % |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"] + rows
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    if args.json_out:
        with open(args.json_out, "w") as f:
            json.dump(out, f, indent=1)
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extras", action="store_true", help="skip copy ceiling, decode sweep, 512 batch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-run", action="store_true")
    ap.add_argument("--shape-sweep", action="store_true",
                    help="time every launch shape at T = 64..8192 (H=6144, K=8), HBM-cold")
    ap.add_argument("--sweep-reps", type=int, default=3)
    ap.add_argument("--cold-table", action="store_true",
                    help="µs per call against T (fused, FP8-output, dense), fresh inputs")
    ap.add_argument("--mix-sweep", action="store_true",
                    help="depth x residency sweep of the mixed-stream probe (JSON)")
    ap.add_argument("--summarize-mix", default="",
                    help="a --mix-sweep record to write as a markdown summary (--out)")
    ap.add_argument("--summarize-cold", default="",
                    help="stdout of bench.py --cold-table: write it as a profiles/ table")
    ap.add_argument("--sweep-h", type=int, default=6144,
                    help="with --shape-sweep: the hidden size")
    ap.add_argument("--sweep-mode", default="bf16", choices=("bf16", "fp8", "dense"),
                    help="with --shape-sweep --alternatives: the fused op, its FP8-output form "
                         "or the dense tail")
    ap.add_argument("--alternatives", action="store_true",
                    help="with --shape-sweep: the alternatives to the shipped launch (per-CU cap, "
                         "per-XCD token ranges, store encodings, persistent) at T = 512..8192")
    ap.add_argument("--state-run", action="store_true",
                    help="eager launches of the input-state phases, for a counter run")
    ap.add_argument("--sweep-ts", default="", help="with --shape-sweep: comma-separated T values")
    ap.add_argument("--eager", action="store_true",
                    help="with --shape-sweep: eager launches for a trace; print the phase table")
    ap.add_argument("--persist-counters-run", action="store_true",
                    help="automatic and persistent launches at T = 512, 2048, 8192, then the copy")
    ap.add_argument("--summarize-phases", action="store_true")
    ap.add_argument("--phases-json", help="with --summarize-phases: stdout of the phase run")
    ap.add_argument("--trace-csv", help="with --summarize-phases: a kernel_trace.csv")
    ap.add_argument("--append-sweep", default="",
                    help="with --summarize-phases: stdout of bench.py --shape-sweep, as a table")
    ap.add_argument("--summarize-sweep", default="",
                    help="stdout of bench.py --shape-sweep: write it as a profiles/ table")
    ap.add_argument("--append-states", default="",
                    help="with --summarize-phases: a bench.py JSON line; its input_states table")
    ap.add_argument("--latency-run", action="store_true")
    ap.add_argument("--summarize-trace")
    ap.add_argument("--kernel-filter", default="mfr_")
    ap.add_argument("--summarize-pmc", action="store_true")
    ap.add_argument("--fetch-csv")
    ap.add_argument("--write-csv")
    ap.add_argument("--stats-csv", default="", help="with --summarize-trace: append this kernel_stats.csv")
    ap.add_argument("--title", default="")
    ap.add_argument("--command", default="")
    ap.add_argument("--pmc-variants-run", action="store_true")
    ap.add_argument("--summarize-pmc-variants", action="store_true")
    ap.add_argument("--summarize-counters", action="store_true")
    ap.add_argument("--counter-csv", action="append", default=[],
                    help="with --summarize-counters: a counter_collection.csv (repeatable)")
    ap.add_argument("--json-out", default="", help="with --summarize-counters: also write JSON")
    ap.add_argument("--out")
    args = ap.parse_args()
    if args.summarize_trace:
        return summarize_trace(args)
    if args.summarize_pmc:
        return summarize_pmc(args)
    if args.summarize_counters:
        return summarize_counters(args)
    if args.summarize_pmc_variants:
        return summarize_pmc_variants(args)
    if args.summarize_phases:
        return summarize_phases(args)
    if args.summarize_sweep:
        return summarize_sweep(args)
    if args.summarize_mix:
        summarize_mix(args)
        return
    if args.summarize_cold:
        return summarize_cold(args)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the fused op has no cross-GPU step to time here "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}). Run with --gpus 1.",
              file=sys.stderr, flush=True)
        sys.exit(2)
    if args.pmc_run:
        return run_pmc(args)
    if args.pmc_variants_run:
        return run_pmc_variants(args)
    if args.latency_run:
        return run_latency(args)
    if args.shape_sweep:
        return run_sweep(args)
    if args.cold_table:
        import torch
        torch.cuda.set_device(0)
        print(json.dumps({"cold_table": cold_table()}), flush=True)
        return
    if args.mix_sweep:
        import torch
        torch.cuda.set_device(0)
        print(json.dumps(mix_sweep()), flush=True)
        return
    if args.state_run:
        return run_states(args)
    if args.persist_counters_run:
        return run_persist_counters(args)
    return run_bench(args)


if __name__ == "__main__":
    main()
