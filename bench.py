#!/usr/bin/env python3
"""Benchmark of the CSA/HCA Compressor (THD gated-softmax pooling) on MI355X.

One step = forward + backward of the Compressor over one THD pack (default:
3 x 8192 tokens, head_dim 512, ratio 4, coff 2), i.e. every kernel of the
path: forward, backward gradients (with the zero-ownership writes and dAPE
partials) and the dAPE reduce.  Inputs are synthetic (seeded N(0,1) bf16
kv/score/dout, N(0, 0.02) fp32 APE) and resident in HBM before timing.

Cache protocol: the 256 MB last-level cache would hold a whole pack, so the
timed region cycles through --sets independent buffer sets, running the
forwards of a group of sets and then their backwards (as a training step
does layer by layer); every kernel therefore reads inputs that at least
~400 MB of other traffic has passed through since they were last touched.

Order: the context legs (a 512 MiB device copy, the warm-cache kernel times,
hipGraph replays, the fp32 PyTorch eager comparison) run first; they also
bring the GPU clocks from idle to their loaded state, which takes ~10 ms.
Then W warm-up steps and the timed region of K steps.

Prints ONE JSON line: value = algorithmic HBM bytes of the step / time per
step (GB/s), from a timed region of K steps with nothing inside but the
work.  Further timed regions repeat the K steps with the segment table read
from the device copy of cu_seqlens (no host copy), and with HIP events
recorded on the launch stream around every kernel; the
per-kernel averages and the roofline object (for the dominant kernel) come
from the last.  The CPU oracle is timed on the host as a baseline.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--sets S]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak
METRIC = "fwd+bwd µs/call and HBM GB/s (% of MI355X peak), 3x8192-tok d512 r4 c2"
COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "gated_pooling_amd", "csrc", f) for f in
                  ("csa_kernels.hip", "csa_api.cpp", "csa_launch.h", "csa_walk.h")]


def consumed_slots(cu, r, c, d):
    """kv/score slots some window reads: (2 nb - 1) r d per segment at coff 2
    (the first block has no previous half), nb r d at coff 1."""
    total = 0
    for s in range(len(cu) - 1):
        nb = (cu[s + 1] - cu[s]) // r
        if nb:
            total += ((2 * nb - 1) if c == 2 else nb) * r * d
    return total


def algorithmic_bytes(cu, T, r, c, d, N):
    """Bytes the method itself must move, per kernel: every consumed kv/score
    slot read once, APE read, out written (forward); the same reads plus dout,
    and dkv/dscore written in full (backward gradients); dAPE written
    (reduce).  Workspace traffic (dAPE partials) is overhead, not counted."""
    W = c * d
    cons = consumed_slots(cu, r, c, d)
    fwd = 2 * 2 * cons + 4 * r * W + 2 * N * d
    grads = 2 * 2 * cons + 4 * r * W + 2 * N * d + 2 * 2 * T * W
    reduce = 4 * r * W
    return {"fwd": fwd, "bwd_grads": grads, "dape_reduce": reduce}


def sources_digest():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    counters, or None if absent or taken on different kernel sources."""
    try:
        with open(COUNTERS) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_digest():
        return None
    ent = rec.get("kernels", {}).get(workload, {}).get(kernel)
    return None if ent is None else ent.get("hbm_bytes_per_launch")


ROLE_OF_KERNEL = (("fwd_kernel", "fwd"), ("fwd128_kernel", "fwd"), ("bwd_kernel", "bwd_grads"),
                  ("bwd128_kernel", "bwd_grads"), ("dape_reduce_kernel", "dape_reduce"))
COPY_BYTES = 512 * 2 ** 20  # the context copy below moves 512 MiB each way


def role_of(kernel_name):
    return next((r for k, r in ROLE_OF_KERNEL if re.search(r"\b" + k + r"[<(]", kernel_name)), None)


def profile_rows(d, kind):
    """Rows of a rocprofv3 output directory, CSV or SQLite (rocpd) format:
    kind "counters" -> (kernel name, counter name, value) per dispatch;
    kind "trace" -> (kernel name, duration ns, vgpr, accum vgpr, sgpr, lds bytes, workgroup size, grid size)."""
    import csv
    import glob
    import sqlite3
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*.db"), recursive=True):
        con = sqlite3.connect(f)
        if kind == "counters":
            rows += [(n, c, float(v)) for n, c, v in
                     con.execute("select kernel_name, counter_name, value from counters_collection")]
        else:
            rows += [tuple(r) for r in con.execute(
                "select name, duration, vgpr_count, accum_vgpr_count, sgpr_count, lds_size, "
                "workgroup_x * workgroup_y * workgroup_z, grid_x * grid_y * grid_z from kernels")]
        con.close()
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv" if kind == "counters"
                                    else "*kernel_trace.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if kind == "counters":
                rows.append((row["Kernel_Name"], row["Counter_Name"], float(row["Counter_Value"])))
            else:
                rows.append((row["Kernel_Name"], int(row["End_Timestamp"]) - int(row["Start_Timestamp"]),
                             int(row.get("Arch_VGPR_Count", 0)), int(row.get("Accum_VGPR_Count", 0)),
                             int(row.get("SGPR_Count", 0)), int(row.get("LDS_Block_Size", 0)),
                             int(row.get("Workgroup_Size", 0)), int(row.get("Grid_Size", 0))))
    return rows


def summarize_trace(d):
    """Markdown table of a rocprofv3 --kernel-trace run: per kernel instance,
    dispatches and duration statistics (us), with the dispatch's resources."""
    import statistics
    by = {}
    for name, dur, vg, ag, sg, lds, wg, grid in profile_rows(d, "trace"):
        e = by.setdefault(name, {"d": [], "res": (vg, ag, sg, lds, wg, grid)})
        e["d"].append(dur / 1000.0)
    out = ["| kernel | dispatches | mean us | median us | min us | LDS B | workgroup | grid (threads) |",
           "|---|---|---|---|---|---|---|---|"]
    for name, e in sorted(by.items(), key=lambda kv: -sum(kv[1]["d"])):
        ds = e["d"]
        short = re.sub(r"\(.*$", "", name.replace("csa::(anonymous namespace)::", "").replace("void ", ""))
        out.append(f"| `{short}` | {len(ds)} | {statistics.mean(ds):.2f} | {statistics.median(ds):.2f} | "
                   f"{min(ds):.2f} | " + " | ".join(str(x) for x in e["res"][3:]) + " |")
    return "\n".join(out)


def summarize_occupancy(d):
    """Markdown table of a rocprofv3 --pmc MeanOccupancyPerCU OccupancyPercent
    run: per kernel instance, the mean of each counter over its dispatches."""
    by = {}
    for name, cname, v in profile_rows(d, "counters"):
        by.setdefault(name, {}).setdefault(cname, []).append(v)
    cols = sorted({c for e in by.values() for c in e})
    out = ["| kernel | dispatches | " + " | ".join(cols) + " |", "|---|---|" + "---|" * len(cols)]
    for name, e in sorted(by.items()):
        short = re.sub(r"\(.*$", "", name.replace("csa::(anonymous namespace)::", "").replace("void ", ""))
        n = max(len(v) for v in e.values())
        out.append(f"| `{short}` | {n} | " + " | ".join(f"{sum(e[c]) / len(e[c]):.2f}" if c in e else ""
                                                      for c in cols) + " |")
    return "\n".join(out)


def summarize_counters(fetch_dir, write_dir, workload):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE; counters in KiB per dispatch) into HBM bytes per launch for
    each kernel of the path, and store them in profiles/hbm_counters.json
    keyed by the sha256 of the kernel sources.  Each counter is scaled by what
    it reads for the 512 MiB device-to-device copy that the same run makes
    (known to fetch and to write exactly 512 MiB per dispatch)."""
    def per_kernel(d, counter):
        vals = {}
        for name, cname, value in profile_rows(d, "counters"):
            if cname != counter:
                continue
            role = role_of(name)
            if role is None and "copy" in name.lower():
                role = "copy"
            if role is not None:
                vals.setdefault(role, []).append(value * 1024.0)
        if "copy" in vals:  # keep the 512 MiB copies, not the small staging copies of the inputs
            top = max(vals["copy"])
            vals["copy"] = [v for v in vals["copy"] if v >= 0.25 * top]
        return {k: sum(v) / len(v) for k, v in vals.items()}, {k: len(v) for k, v in vals.items()}

    fetch, nf = per_kernel(fetch_dir, "FETCH_SIZE")
    write, nw = per_kernel(write_dir, "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise SystemExit("summarize_counters: no copy kernel in the counter runs")
    ff, wf = COPY_BYTES / fetch["copy"], COPY_BYTES / write["copy"]
    kern = {}
    for _, role in ROLE_OF_KERNEL:
        if role in fetch and role in write:
            kern[role] = {"fetch_bytes": round(fetch[role] * ff), "write_bytes": round(write[role] * wf),
                          "hbm_bytes_per_launch": round(fetch[role] * ff + write[role] * wf),
                          "dispatches": [nf[role], nw[role]]}
    try:
        with open(COUNTERS) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    if rec.get("sources_sha256") != sources_digest():
        rec = {}
    rec["sources_sha256"] = sources_digest()
    rec["scale"] = {"FETCH_SIZE": round(ff, 4), "WRITE_SIZE": round(wf, 4),
                    "copy_counter_bytes": {"FETCH_SIZE": round(fetch["copy"]), "WRITE_SIZE": round(write["copy"])}}
    rec.setdefault("kernels", {})[workload] = kern
    with open(COUNTERS, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec["kernels"][workload]))


class EagerCompressor:
    """The same operation written as plain PyTorch fp32 ops (gather the
    windows, mask the first block's previous half, softmax over the window,
    weighted sum; backward by autograd).  Timing context only: the pages
    compare their kernels with an fp32 eager region of this kind
    [PR710: Performance at ratio=2].  It is not part of libcsa and nothing in
    the library calls it.

    Index tensors for the windows are built once per pack (host side)."""

    def __init__(self, cu, T, r, c, d, device):
        import torch
        prev_rows, own_rows, masked = [], [], []
        for s in range(len(cu) - 1):
            for b in range((cu[s + 1] - cu[s]) // r):
                own = cu[s] + b * r
                own_rows.append([own + i for i in range(r)])
                prev_rows.append([own - r + i if b > 0 else own + i for i in range(r)])
                masked.append(b == 0)
        self.r, self.c, self.d = r, c, d
        self.N = len(own_rows)
        self.own = torch.tensor(own_rows, dtype=torch.long, device=device).reshape(-1, r)
        self.prev = torch.tensor(prev_rows, dtype=torch.long, device=device).reshape(-1, r)
        self.masked = torch.tensor(masked, dtype=torch.bool, device=device)

    def forward(self, kv, score, ape):
        """fp32 leaves kv [T, W], score [T, W], ape [r, W] -> out fp32 [N, d]."""
        import torch
        r, c, d = self.r, self.c, self.d
        if c == 2:
            x = torch.cat([score[self.prev][:, :, :d] + ape[:, :d], score[self.own][:, :, d:] + ape[:, d:]], dim=1)
            v = torch.cat([kv[self.prev][:, :, :d], kv[self.own][:, :, d:]], dim=1)
            mask = torch.zeros(self.N, 2 * r, 1, dtype=torch.bool, device=x.device)
            mask[:, :r] = self.masked.view(-1, 1, 1)
            x = x.masked_fill(mask, float("-inf"))
        else:
            x = score[self.own] + ape
            v = kv[self.own]
        p = torch.softmax(x, dim=1)
        return (p * v).sum(dim=1)

    def step(self, kv16, score16, ape, dout16):
        """One fp32 eager forward + backward from the bf16 inputs: returns
        (out, dkv, dscore, dape) in fp32."""
        kv = kv16.float().requires_grad_(True)
        score = score16.float().requires_grad_(True)
        ape = ape.detach().clone().requires_grad_(True)
        out = self.forward(kv, score, ape)
        out.backward(dout16.float())
        return out.detach(), kv.grad, score.grad, ape.grad


def eager_timing(wl, N, sets, stream, steps):
    """Mean µs per fp32 eager forward + backward step on the GPU, over the
    same rotating buffer sets as the library."""
    import torch
    ec = EagerCompressor(list(wl.cu_seqlens), wl.total_tokens, wl.ratio, wl.coff, wl.head_dim, sets[0]["kv"].device)
    assert ec.N == N
    for j in range(len(sets)):
        ec.step(sets[j]["kv"], sets[j]["sc"], sets[j]["ape"], sets[j]["dout"])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for k in range(steps):
        st = sets[k % len(sets)]
        ec.step(st["kv"], st["sc"], st["ape"], st["dout"])
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / steps


def cpu_baseline(wl, N, kv, sc, ape, dout, budget_s):
    """Time the CPU oracle (fp32 evaluation order, OpenMP over windows) on the
    same pack: forward + backward, repeated until about budget_s seconds."""
    import numpy as np

    import oracle
    from gated_pooling_amd import inputs

    args = (inputs.bits(kv), inputs.bits(sc), ape.numpy(), list(wl.cu_seqlens), wl.total_tokens,
            wl.ratio, wl.coff, wl.head_dim)
    doutb = inputs.bits(dout)
    out = np.zeros((N, wl.head_dim), np.uint16)
    outs = oracle.bwd_outputs(wl.total_tokens, wl.ratio, wl.coff, wl.head_dim, N)
    oracle.fwd_f32(*args, out=out)          # warm-up (page faults, caches)
    oracle.bwd_f32(*args, doutb, outs=outs)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.fwd_f32(*args, out=out)
        oracle.bwd_f32(*args, doutb, outs=outs)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 200:
            break
    return reps, el, oracle.num_threads()


def cpu_table(path):
    """The CPU oracle (fp32 evaluation order) timed on every workload: forward
    and backward separately, median of 3 after one warm-up, on all host
    threads and on one thread.  Writes a JSON record with the CPU model."""
    import platform
    import statistics

    import numpy as np

    import oracle
    from gated_pooling_amd import inputs

    model = ""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    full = oracle.num_threads()
    rec = {"cpu_model": model or platform.processor(), "threads_all": full, "host_cpus": os.cpu_count(),
           "what": "fp32-order C oracle (OpenMP over output rows), median of 3 after one warm-up", "workloads": {}}
    for name, wl in inputs.WORKLOADS.items():
        N = oracle.total_comp(wl.cu_seqlens, wl.ratio)
        kv, sc, ape, dout = inputs.make_tensors(wl, N)
        args = (inputs.bits(kv), inputs.bits(sc), ape.numpy(), list(wl.cu_seqlens), wl.total_tokens,
                wl.ratio, wl.coff, wl.head_dim)
        doutb = inputs.bits(dout)
        out = np.zeros((N, wl.head_dim), np.uint16)
        outs = oracle.bwd_outputs(wl.total_tokens, wl.ratio, wl.coff, wl.head_dim, N)
        ent = {}
        for threads in (full, 1):
            oracle.set_num_threads(threads)
            for leg, fn in (("fwd", lambda: oracle.fwd_f32(*args, out=out)),
                            ("bwd", lambda: oracle.bwd_f32(*args, doutb, outs=outs))):
                fn()
                ts = []
                for _ in range(3):
                    t0 = time.perf_counter()
                    fn()
                    ts.append(time.perf_counter() - t0)
                ent[f"{leg}_us_{'all' if threads == full else '1t'}"] = round(statistics.median(ts) * 1e6, 1)
        oracle.set_num_threads(full)
        rec["workloads"][name] = ent
        print(name, ent, flush=True)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # the clocks ramp up over the first few milliseconds of load: warm up
    # long enough that the timed steps see steady state
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--sets", type=int, default=5, help="rotating buffer sets (cold cache)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-warm", action="store_true")
    ap.add_argument("--no-eager", action="store_true", help="skip the fp32 PyTorch eager comparison")
    ap.add_argument("--no-graph", action="store_true", help="skip the hipGraph replay timing")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/hbm_counters.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-trace", metavar="DIR", help="print a kernel-trace summary (markdown) and exit")
    ap.add_argument("--summarize-occupancy", metavar="DIR", help="print an occupancy summary (markdown) and exit")
    ap.add_argument("--cpu-table", metavar="OUT.json",
                    help="time the CPU oracle on every workload (all threads and one thread) and exit")
    args = ap.parse_args()

    if args.cpu_table:
        cpu_table(args.cpu_table)
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.summarize_occupancy:
        print(summarize_occupancy(args.summarize_occupancy))
        return

    if args.summarize_counters:
        from gated_pooling_amd import inputs
        summarize_counters(*args.summarize_counters, args.workload or inputs.HEADLINE)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only (the Compressor path runs on a single "
              "device; --gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_pooling_amd as G
    from gated_pooling_amd import inputs

    wname = args.workload or inputs.HEADLINE
    wl = inputs.WORKLOADS[wname]
    cu, T, r, c, d = list(wl.cu_seqlens), wl.total_tokens, wl.ratio, wl.coff, wl.head_dim
    W, S = c * d, wl.num_segments
    N = G.csa_compressor_total_comp(cu, r)
    dev = torch.device("cuda:0")
    G.lib()

    kv, sc, ape, dout = inputs.make_tensors(wl, N)
    fwd_ws = G.csa_compressor_fwd_workspace_size(r, c, d, S, T, N)
    bwd_ws = G.csa_compressor_bwd_workspace_size(r, c, d, S, T, N)
    sets = []
    for _ in range(max(1, args.sets)):
        st = {
            "kv": kv.to(dev), "sc": sc.to(dev), "ape": ape.to(dev), "dout": dout.to(dev),
            "cu": torch.tensor(cu, dtype=torch.int32, device=dev),
            "out": torch.empty(N, d, dtype=torch.bfloat16, device=dev),
            "dkv": torch.empty(T, W, dtype=torch.bfloat16, device=dev),
            "dsc": torch.empty(T, W, dtype=torch.bfloat16, device=dev),
            "dape": torch.empty(r, W, dtype=torch.float32, device=dev),
            "fws": G.workspace(fwd_ws, dev), "bws": G.workspace(bwd_ws, dev),
        }
        st["p"] = {k: ctypes.c_void_p(v.data_ptr()) for k, v in st.items() if isinstance(v, torch.Tensor)}
        sets.append(st)
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    cur = {"s": sptr}  # launch stream (switched to the capture stream while a graph is captured)
    L = G.lib()
    cu_host = G.host_cu(cu)  # host copy: small packs get the segment table as kernel arguments

    def fwd(st, host=None):
        p = st["p"]
        rc = L.csa_compressor_fwd(p["kv"], p["sc"], p["ape"], p["cu"], cu_host if host is None else host, S, T, N,
                                  r, c, d, p["out"], p["fws"], st["fws"].numel(), cur["s"])
        assert rc == 0, G.csa_last_error()

    def grads(st, host=None):
        p = st["p"]
        rc = L.csa_compressor_bwd_grads(p["kv"], p["sc"], p["ape"], p["cu"], cu_host if host is None else host, S, T,
                                        N, r, c, d, p["dout"], p["dkv"], p["dsc"], p["bws"], st["bws"].numel(),
                                        cur["s"])
        assert rc == 0, G.csa_last_error()

    def reduce(st, s=None):
        p = st["p"]
        rc = L.csa_compressor_bwd_dape_reduce(r, c, d, S, T, N, p["dape"], p["bws"], st["bws"].numel(),
                                              cur["s"] if s is None else s)
        assert rc == 0, G.csa_last_error()

    nsets = len(sets)

    def run_steps(K):
        """K steps on one stream, in groups of nsets: the group's forwards,
        then its backwards (gradients, dAPE reduce)."""
        done = 0
        while done < K:
            grp = list(range(min(nsets, K - done)))
            for j in grp:
                fwd(sets[j])
            for j in grp:
                grads(sets[j])
                reduce(sets[j])
            done += len(grp)

    def timed_steps(K, runner):
        """Wall time per step and event time per step of K steps, bracketed
        by a device synchronization on both sides."""
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record(stream)
        runner(K)
        ev[1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall * 1e3 / K, ev[0].elapsed_time(ev[1]) / K

    def run_steps_timed(K):
        """The same K steps with each kernel's launches of a group issued back
        to back between two HIP events on the launch stream: per-kernel time =
        the group's event interval / launches, which includes no event or
        host overhead between the launches it averages."""
        spans = {"fwd": [], "bwd_grads": [], "dape_reduce": []}
        done = 0
        while done < K:
            grp = list(range(min(nsets, K - done)))
            for name, fn in (("fwd", fwd), ("bwd_grads", grads), ("dape_reduce", reduce)):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for j in grp:
                    fn(sets[j])
                b.record(stream)
                spans[name].append((a, b, len(grp)))
            done += len(grp)
        return spans

    # ---- context legs first: they also bring the GPU's clocks from idle to
    # their loaded state before the timed steps (the step time swings by up to
    # 25 % during the first ~10 ms of load after idling) ----
    t_ctx = time.perf_counter()
    K = args.steps

    # a plain device-to-device copy of 512 MiB (torch's copy kernel)
    src = torch.empty(256 * 2 ** 20, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(5):
        dst.copy_(src)
    b.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * 2 * 5 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst

    warm = None
    if not args.no_warm:  # one buffer set over and over (inputs cache-resident)
        warm = {}
        for name, fn in (("fwd", fwd), ("bwd_grads", grads), ("dape_reduce", reduce)):
            for _ in range(3):
                fn(sets[0])
            ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ea.record(stream)
            for _ in range(20):
                fn(sets[0])
            eb.record(stream)
            torch.cuda.synchronize()
            warm[name] = round(ea.elapsed_time(eb) * 1e3 / 20, 3)

    graph = None
    if not args.no_graph:
        # the same launches captured once into hipGraphs and replayed: a
        # forward-only graph and a forward + backward graph (one stream) over
        # the buffer sets
        def captured(fn):
            g = torch.cuda.CUDAGraph()
            cap = torch.cuda.Stream()
            cap.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cap):
                cur["s"] = ctypes.c_void_p(cap.cuda_stream)
                fn()  # warm-up on the side stream, as torch's capture pattern asks
            torch.cuda.current_stream().wait_stream(cap)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                cur["s"] = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                fn()
            cur["s"] = sptr
            torch.cuda.synchronize()
            return g

        def replay_us(g, reps):
            for _ in range(5):
                g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) * 1e3 / (reps * nsets)

        g_fwd = captured(lambda: [fwd(st) for st in sets])
        g_step = captured(lambda: run_steps(nsets))
        reps = max(40, K // nsets)
        graph = {"fwd_us": round(replay_us(g_fwd, reps), 3), "fwd_bwd_us": round(replay_us(g_step, reps), 3),
                 "replays": reps}
        del g_fwd, g_step

    eager = None
    if not args.no_eager:
        eager_us = eager_timing(wl, N, sets, stream, steps=20)
        eager = {"fwd_bwd_us": round(eager_us, 1),
                 "what": "PyTorch fp32 eager forward + autograd backward of the same op, same buffers"}
    torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_ctx) * 1e3

    # ---- warm-up, then the timed region: K steps, nothing but the work ----
    run_steps(max(args.warmup, 0))
    ms_per_step, gpu_ms_per_step = timed_steps(K, run_steps)

    # the same K steps with the segment table read from the device copy of
    # cu_seqlens (no host copy): what a graph replayed with new cu_seqlens runs
    nohost = ctypes.c_void_p(0)

    def run_steps_device_table(k):
        done = 0
        while done < k:
            grp = list(range(min(nsets, k - done)))
            for j in grp:
                fwd(sets[j], nohost)
            for j in grp:
                grads(sets[j], nohost)
                reduce(sets[j])
            done += len(grp)

    devtab_ms, _ = timed_steps(K, run_steps_device_table)

    # per-kernel region: the same K steps, per-kernel HIP events
    torch.cuda.synchronize()
    spans = run_steps_timed(K)
    torch.cuda.synchronize()

    abytes = algorithmic_bytes(cu, T, r, c, d, N)
    step_bytes = sum(abytes.values())
    kern = {}
    for name, sp in spans.items():
        per = [a.elapsed_time(b) * 1e3 / n for a, b, n in sp]
        avg = sum(a.elapsed_time(b) * 1e3 for a, b, _ in sp) / sum(n for _, _, n in sp)
        kern[name] = {"avg_us": round(avg, 3), "min_group_avg_us": round(min(per), 3),
                      "algorithmic_bytes": abytes[name],
                      "GBs": round(abytes[name] / (avg * 1e-6) / 1e9, 1)}
    dom = max(kern, key=lambda k: kern[k]["avg_us"])
    achieved = kern[dom]["GBs"]
    traffic = load_traffic(dom, wname)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    if eager is not None:
        eager["speedup"] = round(eager["fwd_bwd_us"] / (ms_per_step * 1e3), 1)

    cpu = None
    if not args.no_cpu_baseline:
        reps, el, cores = cpu_baseline(wl, N, kv, sc, ape, dout, args.cpu_seconds)
        cpu = {"value": round(step_bytes * reps / el / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
               "sample": f"{reps} x (forward + backward) of the full {wname} pack, fp32-order C oracle, "
                         f"{el:.1f} s", "ms_per_step": round(el * 1e3 / reps, 1)}

    fwd_us = kern["fwd"]["avg_us"]
    bwd_us = kern["bwd_grads"]["avg_us"] + kern["dape_reduce"]["avg_us"]
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wname, "cu_seqlens": cu if len(cu) <= 8 else f"{S} segments",
                   "total_tokens": T, "total_comp": N, "ratio": r, "coff": c, "head_dim": d,
                   "cache": f"cold ({nsets} rotating buffer sets)"},
        "us_per_call": {"fwd": fwd_us, "bwd": round(bwd_us, 3), "fwd_bwd": round(fwd_us + bwd_us, 3),
                        "step_wall": round(ms_per_step * 1e3, 3), "step_gpu": round(gpu_ms_per_step * 1e3, 3),
                        "step_device_table": round(devtab_ms * 1e3, 3)},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "step_algorithmic_bytes": step_bytes,
        "kernels": kern,
        "warm_us": warm,
        "copy_kernel_GBs": round(copy_gbs, 1),
        "graph_us": graph,
        "eager": eager,
        "clock_settle": {"ms": round(settle_ms, 1),
                         "what": "the context legs above (copy, warm, graph, eager) run before the warm-up steps"},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic},
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
