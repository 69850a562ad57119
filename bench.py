#!/usr/bin/env python3
"""Benchmark of the MLX-affine quantized row product on one MI355X.

A step is one call of the row product over one activation window of the
workload (the LM-head matrix, N = 248320 x K = 2048, 6-bit codes, group 32,
one activation row, by default), with every input already resident in HBM.
The weights rotate over at least 1 GiB of distinct copies so that the
256 MB Infinity Cache cannot hold them, the calls are issued back to back
on one stream and bracketed by HIP events on that same stream.

Printed: one JSON line.  ``value`` is effective HBM GB/s = algorithmic bytes
per call / time per call, where the algorithmic bytes are what the call must
move once: codes + bf16 scales and biases + bf16 activations + fp32 outputs
(+ the routing table).  ``roofline.frac`` is that against the 8.0 TB/s HBM
peak; ``cpu_baseline`` is the fp64 CPU oracle on a bounded sample of the same
workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import struct
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0          # MI355X HBM3E, published
ROTATE_BYTES = 1 << 30     # at least 1 GiB of distinct weight copies
LIB_DEFAULT = os.path.join(ROOT, "bit_affine_quantized_amd", "libqgemv.so")
PROFILE_DIR = os.path.join(ROOT, "profiles")


def _elf_section_range(data: bytes, wanted: str):
    """(offset, size) of one section of a 64-bit little-endian ELF file, or None."""
    if data[:5] != b"\x7fELF\x02":
        return None
    shoff = struct.unpack_from("<Q", data, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)
    heads = [struct.unpack_from("<IIQQQQ", data, shoff + i * shentsize) for i in range(shnum)]
    names = heads[shstrndx][4]
    for name, _, _, _, off, size in heads:
        end = data.index(b"\0", names + name)
        if data[names + name:end].decode() == wanted:
            return off, size
    return None


def _elf_section(data: bytes, wanted: str):
    """Bytes of one section of a 64-bit little-endian ELF file, or None."""
    r = _elf_section_range(data, wanted)
    return None if r is None else data[r[0]:r[0] + r[1]]


BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def code_objects(fatbin: bytes):
    """The GPU code objects (ELF files) of a .hip_fatbin section: one clang
    offload bundle per translation unit, each a header (magic, entry count,
    then per entry its offset from the bundle start, size and target
    triple) followed by its entries."""
    out, pos = [], 0
    while True:
        start = fatbin.find(BUNDLE_MAGIC, pos)
        if start < 0:
            return out
        count = struct.unpack_from("<Q", fatbin, start + len(BUNDLE_MAGIC))[0]
        p = start + len(BUNDLE_MAGIC) + 8
        end = p
        for _ in range(count):
            off, size, tlen = struct.unpack_from("<QQQ", fatbin, p)
            triple = fatbin[p + 24:p + 24 + tlen].decode(errors="replace")
            p += 24 + tlen
            if "amdgcn" in triple and size:
                out.append(fatbin[start + off:start + off + size])
            end = max(end, start + off + size)
        pos = end


def kernel_hash(path: str | None = None) -> str:
    """Hash of the kernels' machine code in the library this run loads: the
    .text section of every GPU code object in its .hip_fatbin, in order.
    Symbol names that the compiler derives from the build path (and any other
    section) do not enter, so an identical rebuild elsewhere hashes the same;
    a counter summary applies to the run only when it was taken on the same
    machine code."""
    path = path or os.environ.get("QGEMV_LIB") or LIB_DEFAULT
    with open(path, "rb") as f:
        data = f.read()
    fatbin = _elf_section(data, ".hip_fatbin")
    h = hashlib.sha256()
    objs = code_objects(fatbin) if fatbin is not None else []
    texts = [_elf_section(obj, ".text") for obj in objs]
    if not objs or any(t is None for t in texts):
        raise SystemExit(f"{path}: no GPU code objects with a .text section found")
    for t in texts:
        h.update(struct.pack("<Q", len(t)))
        h.update(t)
    return h.hexdigest()[:16]


def device_info(torch) -> dict:
    """Name, architecture and compute units of the GPU, its peak shader and
    memory clocks (hipDeviceGetAttribute), and the shader and memory clock
    levels the driver reports as current (sysfs pp_dpm_*, when readable)."""
    props = torch.cuda.get_device_properties(0)
    info = {"name": props.name, "arch": props.gcnArchName, "compute_units": props.multi_processor_count}
    try:
        import ctypes
        hip = ctypes.CDLL("libamdhip64.so")
        dev = torch.cuda.current_device()

        def attr(a):
            v = ctypes.c_int(0)
            return v.value if hip.hipDeviceGetAttribute(ctypes.byref(v), a, dev) == 0 else None

        # hipDeviceAttribute_t values of ROCm 7's hip_runtime_api.h: ClockRate 5,
        # MemoryClockRate 60, MultiprocessorCount 63 (checked against torch's count)
        if attr(63) == props.multi_processor_count:
            info["peak_sclk_mhz"] = attr(5) // 1000
            info["peak_mclk_mhz"] = attr(60) // 1000
    except (OSError, TypeError, AttributeError):
        pass
    pci = f"{props.pci_domain_id:04x}:{props.pci_bus_id:02x}:{props.pci_device_id:02x}.0"
    for key, fname in (("current_sclk", "pp_dpm_sclk"), ("current_mclk", "pp_dpm_mclk")):
        try:
            with open(f"/sys/bus/pci/devices/{pci}/{fname}") as f:
                cur = [line.split(":", 1)[1].strip().rstrip("*").strip() for line in f if line.strip().endswith("*")]
            if cur:
                info[key] = cur[0]
        except OSError:
            pass
    return info


def algorithmic_bytes(runs, m, k, n_out, idx_bytes=0):
    """sum over runs of codes + scales + biases, + activations + outputs."""
    b = 0
    for bits, group, n in runs:
        b += n * k * bits // 8 + n * (k // group) * 4
    return b + m * k * 2 + m * n_out * 4 + idx_bytes


def read_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload (profiles/counters_<workload>.txt), if it was taken on the
    current kernel sources; else None."""
    path = os.path.join(PROFILE_DIR, f"counters_{workload}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#") and ":" in line:
            key, val = line.split(":", 1)
            rec[key.strip()] = val.strip()
    if rec.get("kernel_sha") != kernel_hash():
        return None
    try:
        return int(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


ARITH_NAMES = {1: "dot", 2: "mfma", 3: "wide"}


def parse_shape(text):
    """'BITS,GROUP,N,K' of --workload matrix -> (bits, group, n, k); raises
    ValueError for a shape the library refuses on its face (an unknown width
    or group, K not a multiple of the group)."""
    try:
        bits, group, n, k = (int(v) for v in text.split(","))
    except (AttributeError, ValueError):
        raise ValueError(f"--shape wants BITS,GROUP,N,K, got {text!r}") from None
    if bits not in (2, 3, 4, 5, 6, 8) or group not in (32, 64, 128):
        raise ValueError(f"no MLX affine width/group {bits}/{group}")
    if n < 1 or k < group or k % group:
        raise ValueError(f"shape N={n} K={k} does not fit {bits}-bit codes in groups of {group}")
    return bits, group, n, k


class Workload:
    """Device inputs of one workload plus rotating weight copies."""

    def __init__(self, name: str, m: int, torch, qgemv, synth, arith: int = 0, pair=None):
        self.name, self.m = name, m
        self.torch, self.qgemv = torch, qgemv
        self.arith = arith
        dev = "cuda"

        def t(a):
            a = np.ascontiguousarray(a)
            view = {np.dtype(np.uint32): np.int32, np.dtype(np.uint16): np.int16,
                    np.dtype(np.int32): np.int32}[a.dtype]
            return torch.from_numpy(a.view(view)).to(dev)

        if name in ("single", "sweep", "matrix"):
            # the single 2048 x 2048 4/64 matrix, one width/group pair of the
            # 4096 x 4096 sweep, or any one matrix (bits, group, N, K)
            if name == "single":
                d = synth.single(m=m)
            elif name == "sweep":
                d = synth.sweep(pair[0], pair[1], m=m)
            else:
                d = synth.matrix(7000 + pair[0] * 10 + pair[1], pair[0], pair[1], pair[2], pair[3], m)
            self.k = d["k"]
            self.runs = [(d["bits"], d["group"], d["n"])]
            self.n_out = d["n"]
            self.desc = f"{name} N={d['n']} K={d['k']} {d['bits']}-bit group {d['group']}, {m}-row window"
            base = [(t(d["words"]), t(d["scales"]), t(d["biases"]))]
            self.x = t(d["x"])
            self.y = torch.empty((m, d["n"]), dtype=torch.float32, device=dev)
            self.idx_bytes = 0
            self.kind = "plain"
            self.cols = [0]
        elif name == "lmhead":
            d = synth.lmhead(m=m)
            self.k = d["k"]
            self.runs = [(d["bits"], d["group"], d["n"])]
            self.n_out = d["n"]
            self.desc = (f"LM head N={d['n']} K={d['k']} {d['bits']}-bit group {d['group']}, "
                         f"{m}-row window")
            base = [(t(d["words"]), t(d["scales"]), t(d["biases"]))]
            self.x = t(d["x"])
            self.y = torch.empty((m, d["n"]), dtype=torch.float32, device=dev)
            self.idx_bytes = 0
            self.kind = "plain"
            self.cols = [0]
        elif name in ("stack", "stack3"):
            st = synth.stack(m=m)
            self.k = st["k"]
            self.runs = [(r["bits"], r["group"], r["n"]) for r in st["runs"]]
            self.n_out = st["ldy"]
            how = "one fused dispatch" if name == "stack" else "three strided calls"
            self.desc = ("fused stack K=2048: 4/64 x 2048, 5/128 x 6192 (6144 + 48), 6/64 x 48 into one "
                         f"8288-column row by {how}, {m}-row window")
            base = [tuple(t(r[key]) for key in ("words", "scales", "biases")) for r in st["runs"]]
            self.x = t(st["x"])
            self.y = torch.empty((m, st["ldy"]), dtype=torch.float32, device=dev)
            self.idx_bytes = 0
            self.kind = "strided" if name == "stack3" else "fused"
            self.cols = [r["col"] for r in st["runs"]]
            self.ldy = st["ldy"]
            self.members = [[(6144, 2048), (48, 8192)] if r["n"] == 6192 else [(r["n"], r["col"])]
                            for r in st["runs"]]
        elif name == "gateup":
            # the experts config's routing over a gate stack and an up stack
            # (the up weights are the next seed's draw), silu(g) * u per slot
            d = synth.experts()
            du = synth.matrix(5001, d["bits"], d["group"], d["n"], d["k"], 0, d["n_experts"])
            self.k = d["k"]
            distinct = len(np.unique(d["idx"]))
            self.runs = [(d["bits"], d["group"], d["n"] * distinct)] * 2
            m = d["idx"].shape[0]
            self.m = m
            self.slots = d["idx"].shape[1]
            self.n_out = self.slots * d["n"]
            self.desc = (f"indexed gate/up pair: 2 x {d['n_experts']} x (N={d['n']} K={d['k']} 4-bit group 64), "
                         f"{m} rows x {self.slots} slots ({distinct} distinct experts), silu(g) * u")
            base = [(t(d["words"]), t(d["scales"]), t(d["biases"])),
                    (t(du["words"]), t(du["scales"]), t(du["biases"]))]
            self.x = t(d["x"])
            self.idx = t(d["idx"])
            self.y = torch.empty((m, self.slots, d["n"]), dtype=torch.float32, device=dev)
            self.idx_bytes = d["idx"].size * 4
            self.kind = "gateup"
            self.n_experts = d["n_experts"]
            self.n_each = d["n"]
        elif name == "experts":
            d = synth.experts()
            self.k = d["k"]
            distinct = len(np.unique(d["idx"]))
            self.runs = [(d["bits"], d["group"], d["n"] * distinct)]
            m = d["idx"].shape[0]
            self.m = m
            self.slots = d["idx"].shape[1]
            self.n_out = self.slots * d["n"]
            self.desc = (f"indexed experts: {d['n_experts']} x (N={d['n']} K={d['k']} 4-bit group 64), "
                         f"{m} rows x {self.slots} slots ({distinct} distinct experts), relu2")
            base = [(t(d["words"]), t(d["scales"]), t(d["biases"]))]
            self.x = t(d["x"])
            self.idx = t(d["idx"])
            self.y = torch.empty((m, self.slots, d["n"]), dtype=torch.float32, device=dev)
            self.idx_bytes = d["idx"].size * 4
            self.kind = "indexed"
            self.n_experts = d["n_experts"]
            self.n_each = d["n"]
        else:
            raise SystemExit(f"unknown workload {name}")
        self.bytes = algorithmic_bytes(self.runs, self.m, self.k, self.n_out, self.idx_bytes)
        wbytes = sum(sum(a.numel() * a.element_size() for a in trip) for trip in base)
        copies = max(1, -(-ROTATE_BYTES // wbytes))
        self.copies = []
        for c in range(copies):
            trip_list = base if c == 0 else [tuple(a.clone() for a in trip) for trip in base]
            mats = []
            if self.kind == "fused":
                specs = [dict(bits=bits, group=group, n=n, k=self.k, w=w, scales=s, biases=b, members=mem)
                         for (w, s, b), (bits, group, n), mem in zip(trip_list, self.runs, self.members)]
                self.copies.append((trip_list, [qgemv.Stack(specs, self.ldy)]))
                continue
            for (w, s, b), run_ in zip(trip_list, self.runs if self.kind not in ("indexed", "gateup")
                                           else [None] * len(trip_list)):
                if self.kind in ("indexed", "gateup"):
                    mats.append(qgemv.Matrix(4, 64, self.n_each, self.k, w, s, b, n_experts=self.n_experts,
                                             arith=arith))
                else:
                    bits, group, n = run_
                    mats.append(qgemv.Matrix(bits, group, n, self.k, w, s, b, arith=arith))
            self.copies.append((trip_list, mats))
        self.flat = self.y.view(-1)
        first = self.copies[0][1][0]
        self.arith_used = "auto" if self.kind == "fused" else ARITH_NAMES[first.arith]

    def counts(self):
        """(weight elements streamed, multiply-adds) per step: rows x cols of
        every matrix read (the distinct experts for an indexed call), and
        window rows x output columns x K."""
        rows_cols = sum(n for _, _, n in self.runs) * self.k
        if self.kind in ("indexed", "gateup"):
            macs = self.m * self.slots * self.n_each * self.k * len(self.runs)
        else:
            macs = self.m * rows_cols
        return rows_cols, macs

    def step(self, i: int, stream: int):
        _, mats = self.copies[i % len(self.copies)]
        q = self.qgemv
        if self.kind == "plain":
            rc = q.qgemv_run(mats[0].h, self.x, self.m, self.y, 0, stream)
            assert rc == 0, q.qgemv_strerror(rc)
        elif self.kind == "fused":
            rc = q.qgemv_stack_run(mats[0].h, self.x, self.m, self.y, 0, stream)
            assert rc == 0, q.qgemv_strerror(rc)
        elif self.kind == "strided":
            for mat, col in zip(mats, self.cols):
                rc = q.qgemv_run_strided(mat.h, self.x, self.m, self.flat[col:], self.ldy, 0, stream)
                assert rc == 0, q.qgemv_strerror(rc)
        elif self.kind == "gateup":
            rc = q.qgemv_run_gateup_indexed(mats[0].h, mats[1].h, self.x, self.m, self.idx, self.slots,
                                            self.y, stream)
            assert rc == 0, q.qgemv_strerror(rc)
        else:
            rc = q.qgemv_run_indexed(mats[0].h, self.x, self.m, self.idx, self.slots, self.y,
                                     q.QGEMV_EPI_RELU2, stream)
            assert rc == 0, q.qgemv_strerror(rc)


def time_workload(wl: Workload, steps: int, warmup: int, torch):
    """W untimed warmup steps, then exactly K steps issued back to back on
    one stream, bracketed by a synchronize on both sides.  Events recorded
    on that stream split the K steps into five batches with no host wait in
    between, so the GPU never idles inside the timed region.  Returns the
    mean time per step over all K steps and the per-batch means."""
    stream = torch.cuda.current_stream()
    sid = stream.cuda_stream
    for i in range(warmup):
        wl.step(i, sid)
    torch.cuda.synchronize()
    nb = min(5, steps)
    bounds = [round(steps * b / nb) for b in range(nb + 1)]
    events = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    events[0].record(stream)
    for b in range(nb):
        for i in range(bounds[b], bounds[b + 1]):
            wl.step(warmup + i, sid)
        events[b + 1].record(stream)
    torch.cuda.synchronize()
    batches = [events[b].elapsed_time(events[b + 1]) / (bounds[b + 1] - bounds[b]) for b in range(nb)]
    ms = events[0].elapsed_time(events[nb]) / steps
    return ms, batches


def time_workload_graph(wl: Workload, steps: int, warmup: int, torch, min_ms: float = 100.0) -> float:
    """The same K steps captured once in a HIP graph and replayed: the device
    time per step without the host's issue cost, which is what a caller that
    captures its launch-bound calls sees.  Warmup steps run eagerly first,
    then three untimed replays; returns ms per step over the timed replays
    issued back to back: at least 5, and at least min_ms of them."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        wl.step(i, stream.cuda_stream)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for i in range(3):
            wl.step(warmup + i, side.cuda_stream)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sid = torch.cuda.current_stream().cuda_stream
        for i in range(steps):
            wl.step(warmup + i, sid)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    replays = max(5, int(min_ms / max(e0.elapsed_time(e1) / 3, 1e-3)) + 1)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (steps * replays)


def launch_floor(torch, kernels: int = 200, replays: int = 20) -> float:
    """Device-side interval between back-to-back trivial kernels (one-element
    adds), in microseconds: a captured graph of `kernels` launches is replayed
    so that the host's issue cost stays out of the measurement."""
    z = torch.zeros(1, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            z.add_(1.0)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(kernels):
            z.add_(1.0)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (kernels * replays)


_COPY_FLOOR = {}


def copy_floor(torch, nbytes: int, steps: int = 200) -> float:
    """Device time, in microseconds, of one library copy whose HBM traffic
    equals `nbytes` (nbytes / 2 read, nbytes / 2 written), the sources
    rotating over at least 1 GiB like the weights: a captured graph of
    `steps` copies replayed for at least 20 ms.  A dispatch that only
    streams that many bytes takes this long on the same device, so it is
    the floor for a call of that size in one dispatch."""
    half = max(4096, (nbytes // 2 + 4095) // 4096 * 4096)
    if half in _COPY_FLOOR:
        return _COPY_FLOOR[half]
    copies = max(2, -(-ROTATE_BYTES // half))
    src = torch.empty((copies, half), dtype=torch.uint8, device="cuda")
    dst = torch.empty((copies, half), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            dst[i % copies].copy_(src[i % copies])
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            dst[i % copies].copy_(src[(i * 7) % copies])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    replays = max(5, int(20.0 / max(e0.elapsed_time(e1) / 3, 1e-3)) + 1)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (steps * replays)
    del g, src, dst
    torch.cuda.empty_cache()
    _COPY_FLOOR[half] = round(us, 3)
    return _COPY_FLOOR[half]


def cpu_baseline(budget_s: float = 12.0):
    """The oracle, as it stands, on a bounded sample of LM-head columns at a
    1-row window, threads = host cores (capped at 16)."""
    import oracle
    from bit_affine_quantized_amd import synth

    threads = max(1, min(16, os.cpu_count() or 1))
    rng = np.random.default_rng(4000)
    k, bits, group = synth.LMHEAD_K, synth.LMHEAD_BITS, synth.LMHEAD_GROUP
    # calibrate on a small sample, then run a sample sized to the budget
    def sample(n):
        words = synth.draw_words(rng, (n,), k, bits)
        scales = synth.draw_scales(rng, (n, k // group))
        biases = synth.draw_biases(rng, (n, k // group))
        x = synth.draw_x(rng, 1, k)
        return words, scales, biases, x

    # one block of LM-head-shaped columns, passed over repeatedly until the
    # budget of oracle work is spent
    nblk = 32768
    w, s, b, x = sample(nblk)
    passes, t_total = 0, 0.0
    while t_total < budget_s and passes < 10000:
        t0 = time.perf_counter()
        oracle.gemv(w, s, b, x, bits, group, nblk, k, threads=threads)
        t_total += time.perf_counter() - t0
        passes += 1
    nbytes = algorithmic_bytes([(bits, group, nblk)], 1, k, nblk) * passes
    # the same sample on one thread, for about a third of the budget
    passes1, t1 = 0, 0.0
    while t1 < budget_s / 3 and passes1 < 10000:
        t0 = time.perf_counter()
        oracle.gemv(w, s, b, x, bits, group, nblk, k, threads=1)
        t1 += time.perf_counter() - t0
        passes1 += 1
    nbytes1 = algorithmic_bytes([(bits, group, nblk)], 1, k, nblk) * passes1
    return {"value": round(nbytes / t_total / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{passes} passes over {nblk} LM-head-shaped columns (K=2048, 6-bit group 32), "
                      f"1-row window, fp64 oracle, {t_total:.1f} s",
            "single_thread": {"value": round(nbytes1 / t1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"{passes1} passes over the same columns, {t1:.1f} s"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=1000,
                    help="untimed steps; the GPU clock needs tens of ms of load to settle")
    ap.add_argument("--workload", default="lmhead",
                    choices=["lmhead", "stack", "stack3", "experts", "gateup", "matrix"])
    ap.add_argument("--shape", default=None, metavar="BITS,GROUP,N,K",
                    help="the matrix of --workload matrix, e.g. 5,64,131072,2048")
    ap.add_argument("--m", type=int, default=1, help="window rows")
    ap.add_argument("--all", action="store_true", help="also time the other workloads and windows")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--arith", default="auto", choices=["auto", "dot", "mfma", "wide"],
                    help="arithmetic of the handles (the fused stack always uses the library's choice)")
    ap.add_argument("--graph", action="store_true",
                    help="time the main workload's K steps as one captured HIP graph replay")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (known bytes) for counter scaling")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the row product shards along output columns with no "
              "exchange, so a multi-GPU figure is one GPU's share; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    shape = None
    if args.workload == "matrix":
        try:
            shape = parse_shape(args.shape)
        except ValueError as e:
            print(f"bench.py: {e}", file=sys.stderr)
            sys.exit(2)
    elif args.shape is not None:
        print("bench.py: --shape belongs to --workload matrix", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_affine_quantized_amd import qgemv, synth

    if args.copy_calibration:
        # a copy kernel of known size: 1 GiB read and 1 GiB written per launch
        src = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": src.numel() * 4,
                          "copy_calibration_bytes_written": dst.numel() * 4, "launches": 5}))
        return

    qgemv.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    arith = {"auto": 0, "dot": 1, "mfma": 2, "wide": 3}[args.arith]
    wl = Workload(args.workload, args.m, torch, qgemv, synth, arith, shape)
    # The same K steps as one captured graph first (no host issue cost; 100
    # eager steps, 3 untimed replays of K steps, then timed replays: at least
    # 5 and at least 100 ms of them), then the W untimed warmup steps and the
    # K timed eager steps.  The graph leg also keeps the GPU busy for over
    # 100 ms before the eager measurement: the clocks climb (the shader clock
    # from about 1.2 to 2.3 GHz) over the first tens of milliseconds of load,
    # which a short warmup does not cover.
    ms_graph = time_workload_graph(wl, args.steps, 100, torch)
    ms, batches = time_workload(wl, args.steps, args.warmup, torch)
    if args.graph:
        ms, batches = ms_graph, [ms_graph]
    gbs = wl.bytes / (ms * 1e-3) / 1e9
    rows_cols, macs = wl.counts()
    traffic = read_traffic((f"matrix_b{shape[0]}g{shape[1]}n{shape[2]}k{shape[3]}" if shape else args.workload)
                           + f"_m{wl.m}")
    out = {
        "metric": "effective HBM GB/s (% of MI355X peak) for affine-quant GEMV, 1-16 row windows",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "ms_per_step_graph": round(ms_graph, 6),
        "timing": ("HIP graph replay" if args.graph else
                   "eager launches on one stream, after the graph-replay measurement of the same steps"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded uniform codes, bf16 scales/biases/activations)",
        "config": {"workload": wl.desc, "m": wl.m, "k": wl.k, "algorithmic_bytes": wl.bytes,
                   "weight_copies": len(wl.copies), "parallelism": "single GPU",
                   "arithmetic": f"exact codes as bf16, bf16 activations, fp32 sums ({wl.arith_used} form)"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_GBS, 4), "traffic": traffic},
        "rows_cols_per_s": round(rows_cols / (ms * 1e-3), 1),
        "mnk_per_s": round(macs / (ms * 1e-3), 1),
        "batch_ms": [round(b, 6) for b in batches],
        "kernel_sha": kernel_hash(),
        "device": device_info(torch),
    }
    if args.all:
        extra = {}
        for name, m, ar in [("lmhead", 1, arith), ("lmhead", 8, arith), ("lmhead", 16, arith),
                            ("lmhead", 1, 1), ("lmhead", 8, 1), ("lmhead", 16, 1),
                            ("lmhead", 1, 2), ("lmhead", 8, 2), ("lmhead", 16, 2),
                            ("lmhead", 1, 3), ("lmhead", 8, 3), ("lmhead", 16, 3),
                            ("stack", 1, arith), ("stack", 16, arith), ("stack3", 1, arith), ("stack3", 16, arith),
                            ("stack3", 16, 3),
                            ("experts", 16, arith), ("experts", 16, 1), ("experts", 16, 2), ("experts", 16, 3),
                            ("gateup", 16, arith), ("gateup", 16, 3)]:
            w2 = Workload(name, m, torch, qgemv, synth, ar)
            key = f"{name}_m{w2.m}_{w2.arith_used}"
            if key in extra or (name == args.workload and m == wl.m and w2.arith_used == wl.arith_used):
                del w2
                continue
            msg = time_workload_graph(w2, max(50, args.steps // 2), 100, torch, min_ms=20.0)
            ms2, _ = time_workload(w2, max(50, args.steps // 2), args.warmup, torch)
            g2 = w2.bytes / (ms2 * 1e-3) / 1e9
            rc2, mac2 = w2.counts()
            extra[key] = {"us_per_call": round(ms2 * 1e3, 3), "GB/s": round(g2, 1),
                          "rows_cols_per_s": round(rc2 / (ms2 * 1e-3), 1), "mnk_per_s": round(mac2 / (ms2 * 1e-3), 1),
                          "frac": round(g2 / PEAK_GBS, 4), "bytes": w2.bytes,
                          "us_per_call_graph": round(msg * 1e3, 3),
                          "frac_graph": round(w2.bytes / (msg * 1e-3) / 1e9 / PEAK_GBS, 4)}
            print(f"# {key}: {ms2 * 1e3:.3f} us, {g2:.1f} GB/s; graph {msg * 1e3:.3f} us", file=sys.stderr, flush=True)
            del w2
            torch.cuda.empty_cache()
        # the configs reported but not targeted: the single matrix, and every
        # width/group pair of the sweep at the config's windows of 1, 2, 3, 8
        # and 16 rows (the library's choice)
        for name, m, pair in [("single", 1, None)] + [("sweep", mm, pr) for pr in synth.PAIRS
                                                      for mm in (1, 2, 3, 8, 16)]:
            w2 = Workload(name, m, torch, qgemv, synth, 0, pair)
            msg = time_workload_graph(w2, max(50, args.steps // 2), 100, torch, min_ms=20.0)
            ms2, _ = time_workload(w2, max(50, args.steps // 2), args.warmup, torch)
            g2 = w2.bytes / (ms2 * 1e-3) / 1e9
            key = f"{name}_m{m}" + (f"_b{pair[0]}g{pair[1]}" if pair else "") + f"_{w2.arith_used}"
            extra[key] = {"us_per_call": round(ms2 * 1e3, 3), "GB/s": round(g2, 1),
                          "frac": round(g2 / PEAK_GBS, 4), "bytes": w2.bytes,
                          "us_per_call_graph": round(msg * 1e3, 3),
                          "frac_graph": round(w2.bytes / (msg * 1e-3) / 1e9 / PEAK_GBS, 4)}
            print(f"# {key}: {ms2 * 1e3:.3f} us, {g2:.1f} GB/s; graph {msg * 1e3:.3f} us", file=sys.stderr, flush=True)
            del w2
            torch.cuda.empty_cache()
        # the same traffic streamed by a library copy, for the calls small
        # enough that a dispatch's fixed costs matter
        for v in extra.values():
            if v["bytes"] <= (32 << 20):
                v["copy_floor_us"] = copy_floor(torch, v["bytes"])
        out["workloads"] = extra
        floor = launch_floor(torch)
        out["launch_floor_us"] = round(floor, 3)
        print(f"# launch floor (trivial kernels back to back, graph replay): {floor:.3f} us", file=sys.stderr,
              flush=True)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
