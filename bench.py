#!/usr/bin/env python3
"""Benchmark of the DB-SpMSpV hot path on one MI355X.

Headline step: the R-MAT scale-20 workload (2^20 vertices, edge factor 16,
a=0.57 b=0.19 c=0.19, symmetrized, no self-loops or duplicates) under the
OR-AND semiring, one SpMSpV call for each x density of the sweep 0.01%, 0.1%,
1%, 10%, 50% (positions uniform, seeded).  `value` is the step's effective
bandwidth: algorithmic bytes of all its kernels (byte model below) over the
step's wall time, inputs resident in HBM.

Times: wall times (`value`, call µs, BFS ms) come from passes with the
library's timing off; kernel durations (`roofline`, per-kernel µs) from a
second pass over the same calls with DBS_OPT_TIMING on, where each kernel
dispatch records its own start and end (those events cost the host and the
device a few µs per call, so they are kept out of the throughput passes).

Also reported (nested under "extra"): per-density numbers, with B_min (the
bytes without the pull's full scan of the tiles' column blocks, so that a
wasteful path choice shows); the selector ablation (the kernel with push and
with pull forced at every density, and the x-block ratio where they cross);
the same sweep on the R-MAT 20 graph with its vertices relabelled at random
(about one entry per tile; `--no-permuted` skips it); BFS on R-MAT scale 22 from 64 seeded sources
of the largest component (GTEPS) with an Auto / Push / Pull ablation on 8 of
them; the single-token decode layers 11008x4096 / 4096x11008 (µs per call,
warm and with rotating copies to defeat the on-package cache), also with the
activation sparsified by magnitude inside the metadata kernel (10% kept); the
format size against CSR and CSR + CSC; the Tiny configuration (4096^2, fp32,
x 1%); the Zipf/band stress matrix; GFLOP/s of the plus-times workloads in the
SpMV-equivalent count 2 nnz(A) and the useful count 2 nnz(A[:, J]); and the
tile-format ablation (COO-only / CSR-only / adaptive; `--no-ablations` skips
it).  The CPU baseline is the oracle's Boolean pull on one host thread, with
the same loop on every host core beside it.  Beside the published 8 TB/s, the roofline
object gives the box's measured bandwidth of a device copy (read + write) and
of a streaming read (the library's read probe over 1 GiB).

Byte model (bytes a kernel must move for the path it takes; per call):
  pull     16*segments + 4*T (column block of every tile) + 4*N_blk (masks)
           + sum over tiles with an active column block of (8 + payload)
           + |y|
  push     8*chunks + 8*active blocks + sum over tiles of active column
           blocks of (4 + 4 + 8 + payload)
  metadata 4*nnz_x (+ 2*value size*nnz_x for plus-times) + 8*active blocks
           + 8*chunks + |y| (the output is cleared there)
payload = stored bytes of the tile (pattern tiles other than COO: the 32 B
of masks one direction reads; pattern COO tiles of up to 4 entries: none, their
coordinates are in the 8-byte metadata word).
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

METRIC = "SpMSpV effective GB/s (% of HBM peak) vs x density; BFS GTEPS; decode-layer µs"
HBM_PEAK_GBS = 8000.0
DENSITIES = [0.0001, 0.001, 0.01, 0.1, 0.5]
KERNEL_SRC = ["spmspv.hip", "pattern_pull.h", "tile_kernels.h", "common.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- byte model
def _align(x, a):
    return (x + a - 1) // a * a


def payload_read_bytes(types, nnz, vk):
    """Bytes of each tile's payload one microkernel reads (see module doc)."""
    vs = {0: 4, 1: 2, 2: 0}[vk]
    types = types.astype(np.int64)
    nnz = nnz.astype(np.int64)
    if vk == 2:  # COO tiles of up to 4 entries live in the metadata word
        return np.where(types == 0, np.where(nnz <= 4, 0, _align(nnz, 4)), 32)
    coo = _align(nnz, 4) + _align(nnz * vs, 4)
    dense = np.full_like(nnz, 256 * vs)
    force = _align(48 + nnz * vs, 16)
    csr = _align(64 + _align(nnz, 16) + nnz * vs, 16)
    return np.select([types == 0, types == 1, types == 4], [coo, dense, csr], force)


class Format:
    """Host copy of the index views needed by the byte model."""

    def __init__(self, dbs, A, vk):
        st = dbs.dbs_get_stats(A)
        self.T = st["tiles"]
        self.nseg = st["segments"]
        self.nb = st["nb"]
        self.m = st["m"]
        meta = dbs.dbs_copy_array(A, dbs.DBS_ARR_T_META)
        self.t_cb = dbs.dbs_copy_array(A, dbs.DBS_ARR_T_CB).astype(np.int64)
        self.cb_ptr = dbs.dbs_copy_array(A, dbs.DBS_ARR_CB_PTR).astype(np.int64)
        csc2csr = dbs.dbs_copy_array(A, dbs.DBS_ARR_CSC2CSR).astype(np.int64)
        types = ((meta >> np.uint64(48)) & np.uint64(7)).astype(np.int64)
        nnz = ((meta >> np.uint64(40)) & np.uint64(0xFF)).astype(np.int64) + 1
        self.pay = payload_read_bytes(types, nnz, vk)
        # per column block: tiles and payload bytes (push), via the CSC view
        pay_csc = self.pay[csc2csr]
        cum = np.concatenate([[0], np.cumsum(pay_csc)])
        self.cb_tiles = np.diff(self.cb_ptr)
        self.cb_pay = cum[self.cb_ptr[1:]] - cum[self.cb_ptr[:-1]]
        self.cb_chunks = (self.cb_tiles + 63) // 64

    def pull_bytes_in(self, dbs, A, act_blocks, need_rb, ybytes):
        """Pull bytes of one call restricted to the tiles of the row blocks in
        need_rb (a BFS pull level reads no tile of a row block whose rows are
        all visited); the segment descriptors in proportion to those tiles."""
        if not hasattr(self, "t_rb"):
            rb_ptr = dbs.dbs_copy_array(A, dbs.DBS_ARR_RB_PTR).astype(np.int64)
            self.t_rb = np.repeat(np.arange(rb_ptr.shape[0] - 1), np.diff(rb_ptr))
        sel = need_rb[self.t_rb]
        active = np.zeros(self.nb, bool)
        active[act_blocks] = True
        at = active[self.t_cb] & sel
        nsel = int(sel.sum())
        return (16 * self.nseg * nsel // max(self.T, 1) + 4 * nsel + 4 * self.nb + 8 * int(at.sum())
                + int(self.pay[at].sum()) + ybytes)

    def call_bytes(self, act_blocks, nnz_x, ybytes, push, vsize=0):
        """(metadata bytes, compute bytes) of one call."""
        nact = act_blocks.shape[0]
        nch = int(self.cb_chunks[act_blocks].sum())
        meta_b = 4 * nnz_x + 2 * vsize * nnz_x + 8 * nact + 8 * nch + ybytes
        if push:
            comp = 8 * nch + 8 * nact + 16 * int(self.cb_tiles[act_blocks].sum()) + int(self.cb_pay[act_blocks].sum())
        else:
            active = np.zeros(self.nb, bool)
            active[act_blocks] = True
            at = active[self.t_cb]
            comp = 16 * self.nseg + 4 * self.T + 4 * self.nb + 8 * int(at.sum()) + int(self.pay[at].sum()) + ybytes
        return meta_b, comp


def kernel_src_sha():
    h = hashlib.sha256()
    for f in KERNEL_SRC:
        with open(os.path.join(ROOT, "spmspv_graph_traversal_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload):
    """HBM traffic per launch measured with rocprofv3 counters (profiles/), if
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_k_spmspv_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_src_sha") != kernel_src_sha():
        return None
    return d.get("bytes_per_launch")


# ---------------------------------------------------------------- workloads
def format_size(st, m, n, vsize):
    """Bytes of the blocked dual view against CSR and against CSR + CSC
    (int32 pointers and indices, values of vsize bytes)."""
    nnz = st["nnz"]
    csr = 4 * (m + 1) + 4 * nnz + vsize * nnz
    both = csr + 4 * (n + 1) + 4 * nnz + vsize * nnz
    return {"format_bytes": st["format_bytes"], "csr_bytes": csr, "csr_csc_bytes": both,
            "vs_csr": round(st["format_bytes"] / csr, 3), "vs_csr_csc": round(st["format_bytes"] / both, 3)}


def crossover(rows):
    """x-block ratio where the forced-push and forced-pull kernel times cross,
    interpolated linearly between the two measured densities around it."""
    for a, b in zip(rows, rows[1:]):
        da = a["push_kernel_us"] - a["pull_kernel_us"]
        db = b["push_kernel_us"] - b["pull_kernel_us"]
        if da < 0 <= db:
            f = -da / (db - da)
            return round(a["xb_ratio"] + f * (b["xb_ratio"] - a["xb_ratio"]), 4)
    return None


def gflops(nnz_all, nnz_active, seconds):
    """GFLOP/s of a call in the two counts: the SpMV-equivalent 2 nnz(A) (the
    DB-SpMSpV paper's evaluation count) and the useful 2 nnz(A[:, J]) (entries
    in the active columns)."""
    return {"GFLOPs_spmv_equiv": round(2.0 * nnz_all / seconds / 1e9, 2),
            "GFLOPs_useful": round(2.0 * nnz_active / seconds / 1e9, 2)}


def bench_tiny(dbs, torch, args):
    """Tiny: 4096 x 4096, 16 distinct uniform columns per row, fp32 U[-1,1];
    x with 1% entries (41) at uniform positions; plus-times.  A latency-bound
    configuration (about 1 MB per call)."""
    from synth import rng_for, sparse_x, uniform_csr

    n = 4096
    rp, ci, v = uniform_csr(n, n, 16, rng_for("tiny"))
    xi, xv = sparse_x(n, 0.01, rng_for("tiny", 1))
    dev = torch.device("cuda:0")
    A = dbs.dbs_build(n, n, torch.from_numpy(rp).to(dev), torch.from_numpy(ci).to(dev), torch.from_numpy(v).to(dev),
                      dbs.DBS_F32)
    st = dbs.dbs_get_stats(A)
    fmt = Format(dbs, A, 0)
    act = np.unique(xi // 16)
    push = 100 * act.shape[0] < fmt.nb
    mb, cb = fmt.call_bytes(act, xi.shape[0], 4 * n, push, vsize=4)
    useful = int(np.bincount(ci, minlength=n)[xi].sum())
    xi_d, xv_d = torch.from_numpy(xi).to(dev), torch.from_numpy(xv).to(dev)
    y = torch.empty(n, dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        dbs.dbs_spmspv(A, xi_d, xv_d, dbs.DBS_PLUS_TIMES, y)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        dbs.dbs_spmspv(A, xi_d, xv_d, dbs.DBS_PLUS_TIMES, y)
    ev1.record()
    torch.cuda.synchronize()
    call_ms = ev0.elapsed_time(ev1) / args.steps
    dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 1)
    for _ in range(args.steps):
        dbs.dbs_spmspv(A, xi_d, xv_d, dbs.DBS_PLUS_TIMES, y)
    s2 = dbs.dbs_get_stats(A)
    dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 0)
    kms = s2["sum_compute_ms"] / s2["timed_calls"]
    out = {"workload": "tiny: 4096x4096, 16 uniform nnz/row, fp32; x 1% (41 entries); plus-times",
           "nnz": int(rp[-1]), "nnz_active_columns": useful, "tiles": st["tiles"],
           "tiles_by_format": st["tiles_by_format"], "build_peak_bytes": st["build_peak_bytes"],
           "path": "push" if s2["last_path"] == 0 else "pull", "xb_ratio": round(s2["last_n_nzblk"] / fmt.nb, 4),
           "call_us": round(call_ms * 1e3, 2), "compute_kernel_us": round(kms * 1e3, 2),
           "meta_kernel_us": round(s2["sum_meta_ms"] / s2["timed_calls"] * 1e3, 2),
           "bytes": int(mb + cb), "compute_kernel_GBps": round(cb / (kms * 1e-3) / 1e9, 1),
           "compute_kernel_frac_of_hbm": round(cb / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "kernel": gflops(int(rp[-1]), useful, kms * 1e-3), "call": gflops(int(rp[-1]), useful, call_ms * 1e-3)}
    log(f"[bench] tiny: {out}")
    dbs.dbs_free(A)
    return out


def sweep_inputs(torch, fmt, n, key):
    """The sweep's x vectors (OR-AND: indices only; density k drawn from
    rng_for(*key, k)) with the byte model of each call.  `scan_bytes` is
    the pull's full scan term (segment descriptors, every tile's column-block
    word, the masks), which B_min leaves out so that a wasteful path choice
    shows."""
    from synth import rng_for, sparse_x

    xs = []
    for k, d in enumerate(DENSITIES):
        xi, _ = sparse_x(n, d, rng_for(*key, k), with_values=False)
        act = np.unique(xi // 16)
        push = 100 * act.shape[0] < fmt.nb
        mb, cb = fmt.call_bytes(act, xi.shape[0], n, push)
        scan = 0 if push else 16 * fmt.nseg + 4 * fmt.T + 4 * fmt.nb
        xs.append(dict(density=d, xi=xi, x=torch.from_numpy(xi).to("cuda"), nact=act.shape[0], push=push,
                       meta_bytes=mb, comp_bytes=cb, scan_bytes=scan))
    return xs


def sweep_per_density(dbs, torch, args, A, fmt, xs, y):
    """Per density: call and kernel times, bytes (and B_min), GB/s and the
    roofline fraction; then the kernel with push and with pull forced.
    call_us is the mean of back-to-back calls; call_us_each_median / _mean
    come from 100 calls each bracketed by its own events (which add a little
    time of their own)."""
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # per-density breakdown (separate loops, same kernels)
    per = []
    for x in xs:
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(args.steps):
            dbs.dbs_spmspv(A, x["x"], None, dbs.DBS_OR_AND, y)
        ev1.record()
        torch.cuda.synchronize()
        call_ms = ev0.elapsed_time(ev1) / args.steps
        # 100 calls, each between its own pair of events: median and mean
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(100)]
        for e_a, e_b in pairs:
            e_a.record()
            dbs.dbs_spmspv(A, x["x"], None, dbs.DBS_OR_AND, y)
            e_b.record()
        torch.cuda.synchronize()
        each = np.array([e_a.elapsed_time(e_b) for e_a, e_b in pairs]) * 1e3
        dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 1)
        for _ in range(args.steps):
            dbs.dbs_spmspv(A, x["x"], None, dbs.DBS_OR_AND, y)
        s2 = dbs.dbs_get_stats(A)
        dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 0)
        kms = s2["sum_compute_ms"] / s2["timed_calls"]
        mms = s2["sum_meta_ms"] / s2["timed_calls"]
        per.append({
            "density": x["density"], "nnz_x": int(x["xi"].shape[0]), "n_nzblk": s2["last_n_nzblk"],
            "xb_ratio": round(s2["last_n_nzblk"] / fmt.nb, 5), "path": "push" if s2["last_path"] == 0 else "pull",
            "call_us": round(call_ms * 1e3, 2), "call_us_each_median": round(float(np.median(each)), 2),
            "call_us_each_mean": round(float(each.mean()), 2), "compute_kernel_us": round(kms * 1e3, 2),
            "meta_kernel_us": round(mms * 1e3, 2),
            "bytes": int(x["meta_bytes"] + x["comp_bytes"]),
            "bytes_min": int(x["meta_bytes"] + x["comp_bytes"] - x["scan_bytes"]),
            "call_GBps": round((x["meta_bytes"] + x["comp_bytes"]) / (call_ms * 1e-3) / 1e9, 1),
            "compute_kernel_GBps": round(x["comp_bytes"] / (kms * 1e-3) / 1e9, 1),
            "compute_kernel_frac_of_hbm": round(x["comp_bytes"] / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        })
    # ablation of the global selector: the kernel with push and with pull
    # forced at every density, and the x-block ratio where the two cross
    forced = []
    for x in xs:
        row = {"density": x["density"]}
        for path, name in ((1, "push"), (2, "pull")):
            dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
            dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 1)
            for _ in range(args.steps):
                dbs.dbs_spmspv(A, x["x"], None, dbs.DBS_OR_AND, y)
            s2 = dbs.dbs_get_stats(A)
            row[f"{name}_kernel_us"] = round(s2["sum_compute_ms"] / s2["timed_calls"] * 1e3, 2)
            row["xb_ratio"] = round(s2["last_n_nzblk"] / fmt.nb, 5)
        forced.append(row)
    dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, 0)
    dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 0)
    return per, forced


def bench_rmat20(dbs, torch, args):
    from synth import rmat_csr, rng_for

    t0 = time.time()
    rp, ci = rmat_csr(20, 16, rng_for("rmat20"))
    n = 1 << 20
    log(f"[bench] rmat20 generated: nnz={int(rp[-1])} in {time.time() - t0:.1f}s")
    dev = torch.device("cuda:0")
    t0 = time.time()
    A = dbs.dbs_build(n, n, torch.from_numpy(rp).to(dev), torch.from_numpy(ci).to(dev), None, dbs.DBS_PATTERN)
    torch.cuda.synchronize()
    build_s = time.time() - t0
    st = dbs.dbs_get_stats(A)
    log(f"[bench] rmat20 built in {build_s:.2f}s: tiles={st['tiles']} segments={st['segments']} "
        f"format={st['format_bytes'] / 1e6:.1f} MB")
    fmt = Format(dbs, A, 2)
    xs = sweep_inputs(torch, fmt, n, ("rmat20", 1))
    y = torch.empty(n, dtype=torch.uint8, device=dev)

    def step():
        for x in xs:
            dbs.dbs_spmspv(A, x["x"], None, dbs.DBS_OR_AND, y)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # throughput: the library without its timing events (they cost each call
    # host time and a few us of device time)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    ms_per_step = total_ms / args.steps
    # kernel durations: the same steps again, each dispatch recording its
    # start and end (DBS_OPT_TIMING)
    dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 1)  # clears the kernel-time sums
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    st = dbs.dbs_get_stats(A)
    assert st["timed_calls"] == args.steps * len(xs)
    dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 0)
    step_bytes = sum(x["meta_bytes"] + x["comp_bytes"] for x in xs)
    comp_bytes = sum(x["comp_bytes"] for x in xs)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    kernel_ms = st["sum_compute_ms"] / st["timed_calls"]
    achieved = comp_bytes / len(xs) / (kernel_ms * 1e-3) / 1e9

    per, forced = ([], []) if args.headline_only else sweep_per_density(dbs, torch, args, A, fmt, xs, y)
    res = {
        "ms_per_step": ms_per_step, "value": value, "step_bytes": step_bytes,
        "kernel_avg_us": kernel_ms * 1e3, "achieved": achieved, "comp_bytes_per_launch": comp_bytes / len(xs),
        "per_density": per, "forced_paths": forced, "xb_crossover": crossover(forced), "build_s": build_s,
        "format": {"tiles": st["tiles"], "segments": st["segments"], "format_MB": round(st["format_bytes"] / 1e6, 1),
                   "size": format_size(st, n, n, 0), "build_peak_bytes": st["build_peak_bytes"],
                   "tiles_by_format": st["tiles_by_format"]},
        "graph": (rp, ci, n), "xs": xs,
    }
    return res


def bench_rmat20_permuted(dbs, torch, args, rp, ci, n):
    """The R-MAT 20 graph with its vertices relabelled at random (a secondary
    stress for the tile format: ~1.0 entries per tile instead of ~1.6), the
    same OR-AND sweep as the headline, per density and with the paths forced."""
    from synth import permute_vertices, rng_for

    t0 = time.time()
    prp, pci = permute_vertices(rp, ci, rng_for("rmat20", 2))
    log(f"[bench] rmat20 permuted: nnz={int(prp[-1])} in {time.time() - t0:.1f}s")
    dev = torch.device("cuda:0")
    t0 = time.time()
    A = dbs.dbs_build(n, n, torch.from_numpy(prp).to(dev), torch.from_numpy(pci).to(dev), None, dbs.DBS_PATTERN)
    torch.cuda.synchronize()
    build_s = time.time() - t0
    st = dbs.dbs_get_stats(A)
    fmt = Format(dbs, A, 2)
    xs = sweep_inputs(torch, fmt, n, ("rmat20", 3))
    y = torch.empty(n, dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        for x in xs:
            dbs.dbs_spmspv(A, x["x"], None, dbs.DBS_OR_AND, y)
    torch.cuda.synchronize()
    per, forced = sweep_per_density(dbs, torch, args, A, fmt, xs, y)
    kus = [p["compute_kernel_us"] for p in per]
    comp = [x["comp_bytes"] for x in xs]
    out = {
        "workload": "R-MAT scale 20, edge factor 16, symmetrized, vertices relabelled by a seeded random "
                    "permutation; OR-AND; the headline's x densities",
        "nnz": int(prp[-1]), "tiles": st["tiles"], "entries_per_tile": round(int(prp[-1]) / st["tiles"], 3),
        "segments": st["segments"], "tiles_by_format": st["tiles_by_format"], "build_s": round(build_s, 2),
        "size": format_size(st, n, n, 0), "build_peak_bytes": st["build_peak_bytes"],
        "per_density": per, "forced_paths": forced, "xb_crossover": crossover(forced),
        "sweep_kernel_frac_of_hbm": round(sum(comp) / (sum(kus) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
    }
    dbs.dbs_free(A)
    return out


def measure_read_gbps(dbs, torch, gib=1, reps=10):
    """Streaming read bandwidth: the library's read probe (16-byte loads over
    `gib` GiB, nothing written) timed with HIP events on the stream it runs
    on."""
    a = torch.ones(gib << 28, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    dbs.dbs_probe_read(a, sink)  # words of 1.0f XOR to 0, never 0xFFFFFFFF
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dbs.dbs_probe_read(a, sink)
    e1.record()
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    gbps = a.numel() * 4 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, sink
    torch.cuda.empty_cache()
    return round(gbps, 1)


def measure_copy_gbps(torch, gib=1, reps=10):
    """A plain device-to-device copy of `gib` GiB (torch's copy kernel), timed
    with HIP events: read + write bytes per second, the streaming bandwidth
    this box reaches, beside the published 8 TB/s."""
    a = torch.ones(gib << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    gbps = 2 * a.numel() * 4 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return round(gbps, 1)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_rmat20(res, seconds):
    """The oracle on the host: its Boolean pull over the same sweep, first on
    one thread (the oracle as it stands), then the same loop over every host
    core (OpenMP), each for about `seconds` (at most 50 steps)."""
    import oracle as orc
    import oracle.oracle as orc_mod

    rp, ci, n = res["graph"]

    def timed(fn):
        t0 = time.time()
        steps = 0
        while True:
            for x in res["xs"]:
                fn(x["xi"])
            steps += 1
            el = time.time() - t0
            if el >= seconds or steps >= 50:
                return el / steps, steps

    one, steps1 = timed(lambda xi: orc.or_and_pull(n, n, rp, ci, xi))
    threads = [1]

    def omp(xi):
        _, t = orc_mod.or_and_pull_all_cores(n, n, rp, ci, xi)
        threads[0] = t

    allc, steps_all = timed(omp)
    return {"value": round(res["step_bytes"] / one / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "ms_per_step": round(one * 1e3, 1),
            "sample": f"{steps1} full sweep steps (5 OR-AND calls each, CSR pull) on one host thread",
            "all_cores": {"value": round(res["step_bytes"] / allc / 1e9, 3), "unit": "GB/s", "cores": threads[0],
                          "ms_per_step": round(allc * 1e3, 1),
                          "sample": f"{steps_all} sweep steps, the same loop with its rows over OpenMP threads"},
            "nproc": os.cpu_count(), "cpu_model": cpu_model()}


def bench_bfs22(dbs, torch, args):
    from synth import largest_component_vertices, rmat_csr, rng_for
    import oracle as orc

    t0 = time.time()
    rp, ci = rmat_csr(22, 16, rng_for("rmat22"))
    n = 1 << 22
    log(f"[bench] rmat22 generated: nnz={int(rp[-1])} in {time.time() - t0:.1f}s")
    lcc = largest_component_vertices(rp, ci, n)
    deg = np.diff(rp.astype(np.int64))
    edges = int(deg[lcc].sum()) // 2
    srcs = rng_for("rmat22", 1).choice(lcc, args.bfs_sources, replace=False)
    dev = torch.device("cuda:0")
    t0 = time.time()
    A = dbs.dbs_build(n, n, torch.from_numpy(rp).to(dev), torch.from_numpy(ci).to(dev), None, dbs.DBS_PATTERN)
    torch.cuda.synchronize()
    build_s = time.time() - t0
    lv = torch.empty(n, dtype=torch.int32, device=dev)
    for s in srcs[:2]:
        dbs.dbs_bfs(A, int(s), lv)
    # parity spot check of the first source against the oracle
    t0 = time.time()
    ref = orc.bfs(n, rp, ci, int(srcs[0]))
    cpu_bfs_s = time.time() - t0
    dbs.dbs_bfs(A, int(srcs[0]), lv)
    ok = bool(np.array_equal(lv.cpu().numpy(), ref))
    reached = dbs.dbs_get_stats(A)["bfs_reached"]
    ok = ok and reached == int(np.count_nonzero(ref >= 0))
    times, ktimes, levels, pushl = [], [], [], []
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for s in srcs:  # BFS time without the library's timing events
        ev0.record()
        dbs.dbs_bfs(A, int(s), lv)
        ev1.record()
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1))
        st = dbs.dbs_get_stats(A)
        levels.append(st["bfs_levels"])
        pushl.append(st["bfs_push_levels"])
    dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 1)
    for s in srcs:  # the level kernels' time, a second pass with timing events
        dbs.dbs_bfs(A, int(s), lv)
        ktimes.append(dbs.dbs_get_stats(A)["bfs_kernel_ms"])
    dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 0)
    # DB-BFS with the path forced at every level (the first 8 sources)
    ablation = {}
    k = min(8, len(srcs))
    for path, name in ((0, "auto"), (1, "push"), (2, "pull")):
        dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
        tt = []
        for s in srcs[:k]:
            ev0.record()
            dbs.dbs_bfs(A, int(s), lv)
            ev1.record()
            torch.cuda.synchronize()
            tt.append(ev0.elapsed_time(ev1))
        g = edges / (np.array(tt) * 1e-3) / 1e9
        ablation[name] = {"gteps_harmonic_mean": round(float(len(g) / np.sum(1.0 / g)), 2),
                          "ms_median": round(float(np.median(tt)), 3)}
    dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, 0)
    times = np.array(times)
    gteps = edges / (times * 1e-3) / 1e9
    # bytes of the first source's BFS in the SpMSpV byte model: every level
    # a masked OR-AND SpMSpV of its frontier (push or pull by the th3 rule),
    # writing the next frontier's bitmap (n/8 B) and 4 B per found vertex,
    # plus the frontier metadata (bitmap scan and block list).  A pull level
    # reads only the row blocks that still hold an unvisited row with an
    # entry, so its tiles are counted in those row blocks only; within them
    # it may stop early (a long row block whose rows its first segment
    # found), so the model still bounds the level's reads from above.
    fmt = Format(dbs, A, 2)
    model_bytes = 0
    mbk = (n + 15) // 16
    for L in range(int(ref.max()) + 1):
        fr = np.nonzero(ref == L)[0]
        act = np.unique(fr // 16)
        nxt = int(np.count_nonzero(ref == L + 1))
        push = 100 * act.shape[0] < fmt.nb
        if push:
            _, cb = fmt.call_bytes(act, fr.shape[0], n // 8 + 4 * nxt, push)
        else:
            wanted = (deg > 0) & ((ref > L) | (ref < 0))
            need = np.zeros(16 * mbk, bool)
            need[:n] = wanted
            cb = fmt.pull_bytes_in(dbs, A, act, need.reshape(mbk, 16).any(axis=1), n // 8 + 4 * nxt)
        model_bytes += cb + n // 8 + 8 * act.shape[0]
    del fmt
    gc.collect()
    st = dbs.dbs_get_stats(A)
    return {"workload": "R-MAT scale 22, edge factor 16, symmetrized; " + f"{len(srcs)} sources in the largest component",
            "vertices_in_component": int(lcc.shape[0]), "undirected_edges_in_component": edges,
            "gteps_harmonic_mean": round(float(len(gteps) / np.sum(1.0 / gteps)), 2),
            "gteps_median": round(float(np.median(gteps)), 2),
            "ms_median": round(float(np.median(times)), 3), "ms_mean": round(float(times.mean()), 3),
            "level_kernels_ms_median": round(float(np.median(ktimes)), 3),
            "levels_median": int(np.median(levels)), "push_levels_median": int(np.median(pushl)),
            "first_source_matches_oracle": ok, "oracle_bfs_s_first_source": round(cpu_bfs_s, 2),
            "first_source_model_bytes": int(model_bytes),
            "first_source_GBps": round(model_bytes / (times[0] * 1e-3) / 1e9, 1),
            "first_source_frac_of_hbm": round(model_bytes / (times[0] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "first_source_level_kernels_frac_of_hbm": round(model_bytes / (ktimes[0] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "first_source_reached": int(reached),
            "build_peak_bytes": st["build_peak_bytes"], "size": format_size(st, n, n, 0),
            "oracle_gteps_first_source": round(edges / cpu_bfs_s / 1e9, 4), "build_s": round(build_s, 2),
            "path_ablation_first_8_sources": ablation}


def bench_decode(dbs, torch, args):
    from synth import decode_activation, decode_weight_csr, rng_for

    dev = torch.device("cuda:0")
    out = []
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for rows, cols in [(11008, 4096), (4096, 11008)]:
        for sp in (0.5, 0.7):
            rp, ci, bits = decode_weight_csr(rows, cols, sp, rng_for("decode", rows, int(sp * 10)))
            rp_d, ci_d = torch.from_numpy(rp).to(dev), torch.from_numpy(ci).to(dev)
            v_d = torch.from_numpy(bits.view(np.int16)).to(dev)
            copies = [dbs.dbs_build(rows, cols, rp_d, ci_d, v_d, dbs.DBS_BF16) for _ in range(args.decode_copies)]
            colcount = np.bincount(ci, minlength=cols)
            fmt = Format(dbs, copies[0], 1)
            st = dbs.dbs_get_stats(copies[0])
            y = torch.empty(rows, dtype=torch.float32, device=dev)
            for z in (0.1, 0.5, 0.9):
                x = decode_activation(cols, z, rng_for("decode", rows, int(sp * 10), int(z * 10)))
                xd = torch.from_numpy(x.view(np.int16)).to(dev)
                act = np.unique(np.nonzero(x)[0] // 16)
                mb, cb = fmt.call_bytes(act, 0, 4 * rows, False)
                mb += 2 * cols
                A = copies[0]
                for _ in range(args.warmup):
                    dbs.dbs_spmspv_dense(A, xd, dbs.DBS_PLUS_TIMES, y)
                torch.cuda.synchronize()
                ev0.record()
                for _ in range(args.steps):
                    dbs.dbs_spmspv_dense(A, xd, dbs.DBS_PLUS_TIMES, y)
                ev1.record()
                torch.cuda.synchronize()
                warm_us = ev0.elapsed_time(ev1) / args.steps * 1e3
                dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 1)  # kernel time: a second pass
                for _ in range(args.steps):
                    dbs.dbs_spmspv_dense(A, xd, dbs.DBS_PLUS_TIMES, y)
                s2 = dbs.dbs_get_stats(A)
                kus = s2["sum_compute_ms"] / s2["timed_calls"] * 1e3
                dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 0)
                # rotating copies: each call reads a different copy of the weights
                for c in copies:
                    dbs.dbs_spmspv_dense(c, xd, dbs.DBS_PLUS_TIMES, y)
                torch.cuda.synchronize()
                ev0.record()
                reps = max(args.steps, len(copies))
                for r in range(reps):
                    dbs.dbs_spmspv_dense(copies[r % len(copies)], xd, dbs.DBS_PLUS_TIMES, y)
                ev1.record()
                torch.cuda.synchronize()
                cold_us = ev0.elapsed_time(ev1) / reps * 1e3
                useful = int(colcount[np.nonzero(x)[0]].sum())
                out.append({"shape": [rows, cols], "weight_sparsity": sp, "activation_zeros": z,
                            "nnz": int(rp[-1]), "nnz_active_columns": useful,
                            "kernel_warm": gflops(int(rp[-1]), useful, kus * 1e-6),
                            "call_warm": gflops(int(rp[-1]), useful, warm_us * 1e-6),
                            "build_peak_bytes": st["build_peak_bytes"],
                            "path": "push" if s2["last_path"] == 0 else "pull",
                            "xb_ratio": round(s2["last_n_nzblk"] / fmt.nb, 4),
                            "us_warm": round(warm_us, 2), "compute_kernel_us_warm": round(kus, 2),
                            "us_rotating_copies": round(cold_us, 2),
                            "bytes": int(mb + cb),
                            "GBps_warm": round((mb + cb) / (warm_us * 1e-6) / 1e9, 1),
                            "GBps_rotating": round((mb + cb) / (cold_us * 1e-6) / 1e9, 1),
                            "tiles_by_format": st["tiles_by_format"], "size": format_size(st, rows, cols, 2)})
                log(f"[bench] decode {rows}x{cols} s={sp} z={z}: warm {warm_us:.2f} us, rotating {cold_us:.2f} us")
            if sp == 0.5:
                out.append(bench_decode_threshold(dbs, torch, args, copies[0], fmt, rows, cols, y))
            # free this layer's copies here, not inside the next layer's timed calls
            A = c = None
            del copies
            gc.collect()
            torch.cuda.synchronize()
    return out


def bench_decode_threshold(dbs, torch, args, A, fmt, rows, cols, y):
    """Fused activation sparsification: a dense bf16 activation without zeros,
    thresholded by magnitude inside the metadata kernel so that ~10% of it
    stays active (the activation density of the decoding evaluation)."""
    from synth import decode_activation, rng_for

    x = decode_activation(cols, 0.0, rng_for("decode", rows, 99))
    xf = np.abs((x.astype(np.uint32) << 16).view(np.float32))
    t = float(np.float32(np.quantile(xf, 0.9)))
    kept = np.nonzero(xf > t)[0]
    xd = torch.from_numpy(x.view(np.int16)).to(y.device)
    mb, cb = fmt.call_bytes(np.unique(kept // 16), 0, 4 * rows, False)
    mb += 2 * cols
    for _ in range(args.warmup):
        dbs.dbs_spmspv_dense_threshold(A, xd, t, dbs.DBS_PLUS_TIMES, y)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        dbs.dbs_spmspv_dense_threshold(A, xd, t, dbs.DBS_PLUS_TIMES, y)
    ev1.record()
    torch.cuda.synchronize()
    warm_us = ev0.elapsed_time(ev1) / args.steps * 1e3
    dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 1)
    for _ in range(args.steps):
        dbs.dbs_spmspv_dense_threshold(A, xd, t, dbs.DBS_PLUS_TIMES, y)
    s2 = dbs.dbs_get_stats(A)
    dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 0)
    log(f"[bench] decode {rows}x{cols} s=0.5 fused threshold (10% kept): warm {warm_us:.2f} us")
    return {"shape": [rows, cols], "weight_sparsity": 0.5, "activation": "dense, |x| > t keeps 10%",
            "threshold": t, "kept": int(kept.shape[0]), "path": "push" if s2["last_path"] == 0 else "pull",
            "xb_ratio": round(s2["last_n_nzblk"] / fmt.nb, 4), "us_warm": round(warm_us, 2),
            "compute_kernel_us_warm": round(s2["sum_compute_ms"] / s2["timed_calls"] * 1e3, 2),
            "meta_kernel_us_warm": round(s2["sum_meta_ms"] / s2["timed_calls"] * 1e3, 2),
            "bytes": int(mb + cb), "GBps_warm": round((mb + cb) / (warm_us * 1e-6) / 1e9, 1)}


FORMATS = {"adaptive": -1, "COO-only": 0, "CSR-only": 4}


def bench_format_ablation(dbs, torch, args):
    """Tile-format ablation (the DB-SpMSpV paper's Figure 10): every tile stored
    as COO, as patched CSR, or by the adaptive rule, on the R-MAT 20 sweep
    (kernel µs per density) and on the 11008x4096 decode layer at 50% weight
    sparsity (kernel µs per activation); at most 5 timed calls per point."""
    from synth import decode_activation, decode_weight_csr, rmat_csr, rng_for, sparse_x

    steps = min(args.steps, 5)

    dev = torch.device("cuda:0")
    out = {"rmat20_or_and": {}, "decode_11008x4096_s0.5": {}}
    rp, ci = rmat_csr(20, 16, rng_for("rmat20"))
    n = 1 << 20
    rp_d, ci_d = torch.from_numpy(rp).to(dev), torch.from_numpy(ci).to(dev)
    xs = [torch.from_numpy(sparse_x(n, d, rng_for("rmat20", 1, k), with_values=False)[0]).to(dev)
          for k, d in enumerate(DENSITIES)]
    y = torch.empty(n, dtype=torch.uint8, device=dev)
    for name, f in FORMATS.items():
        o = dbs.default_build_options()
        o.force_format = f
        A = dbs.dbs_build(n, n, rp_d, ci_d, None, dbs.DBS_PATTERN, options=o)
        st = dbs.dbs_get_stats(A)
        row = {"format_MB": round(st["format_bytes"] / 1e6, 1)}
        for d, x in zip(DENSITIES, xs):
            for _ in range(2):
                dbs.dbs_spmspv(A, x, None, dbs.DBS_OR_AND, y)
            dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 1)
            for _ in range(steps):
                dbs.dbs_spmspv(A, x, None, dbs.DBS_OR_AND, y)
            s2 = dbs.dbs_get_stats(A)
            dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 0)
            row[str(d)] = round(s2["sum_compute_ms"] / s2["timed_calls"] * 1e3, 2)
        out["rmat20_or_and"][name] = row
        dbs.dbs_free(A)
        log(f"[bench] format ablation rmat20 {name}: {row}")
    rows, cols = 11008, 4096
    rp, ci, bits = decode_weight_csr(rows, cols, 0.5, rng_for("decode", rows, 5))
    rp_d, ci_d = torch.from_numpy(rp).to(dev), torch.from_numpy(ci).to(dev)
    v_d = torch.from_numpy(bits.view(np.int16)).to(dev)
    y = torch.empty(rows, dtype=torch.float32, device=dev)
    acts = {z: torch.from_numpy(decode_activation(cols, z, rng_for("decode", rows, 5, int(z * 10))).view(np.int16)).to(dev)
            for z in (0.1, 0.5, 0.9)}
    for name, f in FORMATS.items():
        o = dbs.default_build_options()
        o.force_format = f
        A = dbs.dbs_build(rows, cols, rp_d, ci_d, v_d, dbs.DBS_BF16, options=o)
        st = dbs.dbs_get_stats(A)
        row = {"format_MB": round(st["format_bytes"] / 1e6, 2)}
        for z, xd in acts.items():
            for _ in range(2):
                dbs.dbs_spmspv_dense(A, xd, dbs.DBS_PLUS_TIMES, y)
            dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 1)
            for _ in range(steps):
                dbs.dbs_spmspv_dense(A, xd, dbs.DBS_PLUS_TIMES, y)
            s2 = dbs.dbs_get_stats(A)
            dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 0)
            row[f"zeros {z}"] = round(s2["sum_compute_ms"] / s2["timed_calls"] * 1e3, 2)
        out["decode_11008x4096_s0.5"][name] = row
        dbs.dbs_free(A)
        log(f"[bench] format ablation decode {name}: {row}")
    return out


def bench_decode_th1(dbs, torch, args):
    """Decode layers with the Dense threshold th1 at the paper's 128 and at 48
    (activation with 50% zeros): per call warm and with rotating copies, kernel
    time and format size.  On this GPU a patched-CSR tile costs about ten times
    the vector instructions of a Dense one, so the layers run faster as Dense
    tiles although those hold more bytes."""
    from synth import decode_activation, decode_weight_csr, rng_for

    dev = torch.device("cuda:0")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    steps, ncopy = max(args.steps, 10), 6
    out = []
    for rows, cols in [(11008, 4096), (4096, 11008)]:
        for sp in (0.5, 0.7):
            rp, ci, bits = decode_weight_csr(rows, cols, sp, rng_for("decode", rows, int(sp * 10)))
            rp_d, ci_d = torch.from_numpy(rp).to(dev), torch.from_numpy(ci).to(dev)
            v_d = torch.from_numpy(bits.view(np.int16)).to(dev)
            x = decode_activation(cols, 0.5, rng_for("decode", rows, int(sp * 10), 5))
            xd = torch.from_numpy(x.view(np.int16)).to(dev)
            y = torch.empty(rows, dtype=torch.float32, device=dev)
            for th1 in (128, 48):
                o = dbs.default_build_options()
                o.th1 = th1
                copies = [dbs.dbs_build(rows, cols, rp_d, ci_d, v_d, dbs.DBS_BF16, options=o) for _ in range(ncopy)]
                st = dbs.dbs_get_stats(copies[0])
                for c in copies:
                    for _ in range(2):
                        dbs.dbs_spmspv_dense(c, xd, dbs.DBS_PLUS_TIMES, y)
                torch.cuda.synchronize()
                ev0.record()
                for _ in range(steps):
                    dbs.dbs_spmspv_dense(copies[0], xd, dbs.DBS_PLUS_TIMES, y)
                ev1.record()
                torch.cuda.synchronize()
                warm = ev0.elapsed_time(ev1) / steps * 1e3
                ev0.record()
                for r in range(steps):
                    dbs.dbs_spmspv_dense(copies[r % ncopy], xd, dbs.DBS_PLUS_TIMES, y)
                ev1.record()
                torch.cuda.synchronize()
                cold = ev0.elapsed_time(ev1) / steps * 1e3
                dbs.dbs_set_option(copies[0], dbs.DBS_OPT_TIMING, 1)
                for _ in range(steps):
                    dbs.dbs_spmspv_dense(copies[0], xd, dbs.DBS_PLUS_TIMES, y)
                s2 = dbs.dbs_get_stats(copies[0])
                row = {"shape": [rows, cols], "weight_sparsity": sp, "th1": th1,
                       "tiles_by_format": st["tiles_by_format"], "size": format_size(st, rows, cols, 2),
                       "us_warm": round(warm, 2), "us_rotating_copies": round(cold, 2),
                       "compute_kernel_us_warm": round(s2["sum_compute_ms"] / s2["timed_calls"] * 1e3, 2)}
                out.append(row)
                log(f"[bench] decode th1 ablation: {row}")
                del copies
                gc.collect()
                torch.cuda.synchronize()
    return out


ZIPF_DENSITIES = [1e-5, 1e-4, 1e-3, 1e-2, 5e-2, 0.2]


def bench_zipf(dbs, torch, args):
    """Load-imbalance stress matrix (8,388,608^2, Zipf row lengths, band + 10%
    uniform), fp32 PLUS_TIMES at each x density; one line per density."""
    from synth import rng_for, sparse_x_with_dense_blocks, zipf_band_csr

    n = 1 << 23
    t0 = time.time()
    rp, ci, v = zipf_band_csr(n, rng_for("zipf"), band_frac=args.zipf_band_frac)
    gen_s = time.time() - t0
    lens = np.diff(rp.astype(np.int64))
    log(f"[bench] zipf generated: nnz={ci.shape[0]} max_row={int(lens.max())} in {gen_s:.1f}s")
    dev = torch.device("cuda:0")
    t0 = time.time()
    rp_d, ci_d, v_d = torch.from_numpy(rp).to(dev), torch.from_numpy(ci).to(dev), torch.from_numpy(v).to(dev)
    A = dbs.dbs_build(n, n, rp_d, ci_d, v_d, dbs.DBS_F32)
    torch.cuda.synchronize()
    build_s = time.time() - t0
    colcount = np.bincount(ci, minlength=n)
    del rp, ci, v
    st = dbs.dbs_get_stats(A)
    fmt = Format(dbs, A, 0)
    y = torch.empty(n, dtype=torch.float32, device=dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per, forced = [], []
    for k, d in enumerate(ZIPF_DENSITIES):
        xi, xv = sparse_x_with_dense_blocks(n, d, rng_for("zipf", 1, k))
        act = np.unique(xi // 16)
        push = 100 * act.shape[0] < fmt.nb
        mb, cb = fmt.call_bytes(act, xi.shape[0], 4 * n, push, vsize=4)
        xi_d, xv_d = torch.from_numpy(xi).to(dev), torch.from_numpy(xv).to(dev)
        for _ in range(args.warmup):
            dbs.dbs_spmspv(A, xi_d, xv_d, dbs.DBS_PLUS_TIMES, y)
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(args.steps):
            dbs.dbs_spmspv(A, xi_d, xv_d, dbs.DBS_PLUS_TIMES, y)
        ev1.record()
        torch.cuda.synchronize()
        call_ms = ev0.elapsed_time(ev1) / args.steps
        dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 1)  # kernel times: a second pass
        for _ in range(args.steps):
            dbs.dbs_spmspv(A, xi_d, xv_d, dbs.DBS_PLUS_TIMES, y)
        s2 = dbs.dbs_get_stats(A)
        dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 0)
        kms = s2["sum_compute_ms"] / s2["timed_calls"]
        useful = int(colcount[xi].sum())
        per.append({
            "density": d, "nnz_x": int(xi.shape[0]), "xb_ratio": round(s2["last_n_nzblk"] / fmt.nb, 5),
            "nnz_active_columns": useful, "kernel": gflops(int(lens.sum()), useful, kms * 1e-3),
            "call": gflops(int(lens.sum()), useful, call_ms * 1e-3),
            "path": "push" if s2["last_path"] == 0 else "pull", "call_us": round(call_ms * 1e3, 2),
            "compute_kernel_us": round(kms * 1e3, 2),
            "meta_kernel_us": round(s2["sum_meta_ms"] / s2["timed_calls"] * 1e3, 2),
            "bytes": int(mb + cb), "call_GBps": round((mb + cb) / (call_ms * 1e-3) / 1e9, 1),
            "compute_kernel_GBps": round(cb / (kms * 1e-3) / 1e9, 1),
            "compute_kernel_frac_of_hbm": round(cb / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        })
        log(f"[bench] zipf d={d}: {per[-1]}")
        # the selector's ablation: the kernel with push and with pull forced
        row = {"density": d, "xb_ratio": per[-1]["xb_ratio"]}
        for path, name in ((1, "push"), (2, "pull")):
            dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
            dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 1)
            for _ in range(min(args.steps, 5)):
                dbs.dbs_spmspv(A, xi_d, xv_d, dbs.DBS_PLUS_TIMES, y)
            s3 = dbs.dbs_get_stats(A)
            row[f"{name}_kernel_us"] = round(s3["sum_compute_ms"] / s3["timed_calls"] * 1e3, 2)
        forced.append(row)
        dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, 0)
        dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 0)
        log(f"[bench] zipf forced paths d={d}: {forced[-1]}")
    dbs.dbs_set_option(A, dbs.DBS_OPT_TIMING, 0)
    # tile-format ablation (the matrix is 99.99% COO tiles under the
    # adaptive rule, so COO-only is the same build): every tile patched CSR
    csr_only = None
    if not args.no_ablations:
        dbs.dbs_free(A)
        o = dbs.default_build_options()
        o.force_format = FORMATS["CSR-only"]
        B = dbs.dbs_build(n, n, rp_d, ci_d, v_d, dbs.DBS_F32, options=o)
        sb = dbs.dbs_get_stats(B)
        csr_only = {"format_MB": round(sb["format_bytes"] / 1e6, 1)}
        for k, d in enumerate(ZIPF_DENSITIES):
            if d not in (1e-3, 1e-2, 0.2):
                continue
            xi, xv = sparse_x_with_dense_blocks(n, d, rng_for("zipf", 1, k))
            xi_d, xv_d = torch.from_numpy(xi).to(dev), torch.from_numpy(xv).to(dev)
            dbs.dbs_spmspv(B, xi_d, xv_d, dbs.DBS_PLUS_TIMES, y)
            dbs.dbs_set_option(B, dbs.DBS_OPT_TIMING, 1)
            for _ in range(min(args.steps, 5)):
                dbs.dbs_spmspv(B, xi_d, xv_d, dbs.DBS_PLUS_TIMES, y)
            s3 = dbs.dbs_get_stats(B)
            dbs.dbs_set_option(B, dbs.DBS_OPT_TIMING, 0)
            csr_only[str(d)] = round(s3["sum_compute_ms"] / s3["timed_calls"] * 1e3, 2)
        dbs.dbs_free(B)
        log(f"[bench] zipf CSR-only: {csr_only}")
    del rp_d, ci_d, v_d
    hist = np.bincount(np.floor(np.log2(np.maximum(lens, 1))).astype(np.int64))
    bf = args.zipf_band_frac
    return {"workload": f"zipf(1.8) row lengths capped at 2^20, {100 * bf:g}% band + {100 * (1 - bf):g}% uniform, "
                        "8388608^2, fp32",
            "nnz": int(lens.sum()), "max_row": int(lens.max()),
            "row_length_log2_histogram": hist.tolist(), "generate_s": round(gen_s, 1), "build_s": round(build_s, 2),
            "tiles": st["tiles"], "tiles_by_format": st["tiles_by_format"], "segments": st["segments"],
            "format_MB": round(st["format_bytes"] / 1e6, 1), "size": format_size(st, n, n, 4),
            "build_peak_bytes": st["build_peak_bytes"], "per_density": per,
            "forced_paths": forced, "xb_crossover": crossover(forced), "format_ablation_csr_only_kernel_us": csr_only}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-bfs", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-zipf", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-ablations", action="store_true",
                    help="skip the tile-format ablation (COO-only / CSR-only / adaptive builds)")
    ap.add_argument("--no-tiny", action="store_true")
    ap.add_argument("--no-permuted", action="store_true",
                    help="skip the R-MAT 20 sweep on the randomly relabelled graph")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode layers (for profiling the decode kernel); prints their JSON")
    ap.add_argument("--bfs-only", action="store_true",
                    help="only the R-MAT 22 BFS (for profiling the level kernels); prints its JSON")
    ap.add_argument("--zipf-only", action="store_true",
                    help="only the Zipf/band stress matrix (for profiling its pull); prints its JSON")
    ap.add_argument("--permuted-only", action="store_true",
                    help="only the sweep on the relabelled R-MAT 20 graph (for profiling); prints its JSON")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the timed sweep (for profiling: every SpMSpV launch is one of the timed mix)")
    ap.add_argument("--zipf-band-frac", type=float, default=0.9,
                    help="share of each Zipf row's columns in its band (the rest uniform over all columns); "
                         "other values only to attribute the pull's memory traffic to the two parts")
    ap.add_argument("--bfs-sources", type=int, default=64)
    ap.add_argument("--decode-copies", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only a plain 256 MiB device copy (x3), the reference for scaling HBM byte counters")
    args = ap.parse_args()
    if args.copy_probe:
        import torch

        a = torch.ones(64 * 1024 * 1024, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_per_copy": 4 * a.numel(), "copies": 3}))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the method has no multi-GPU path here (--gpus {args.gpus} "
              "requested); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import spmspv_graph_traversal_amd as dbs

    torch.cuda.set_device(0)
    if args.decode_only:
        print(json.dumps({"decode": bench_decode(dbs, torch, args)}), flush=True)
        return
    if args.bfs_only:
        print(json.dumps({"bfs_rmat22": bench_bfs22(dbs, torch, args)}), flush=True)
        return
    if args.zipf_only:
        print(json.dumps({"zipf_band": bench_zipf(dbs, torch, args)}), flush=True)
        return
    if args.permuted_only:
        from synth import rmat_csr, rng_for

        rp, ci = rmat_csr(20, 16, rng_for("rmat20"))
        print(json.dumps({"rmat20_permuted": bench_rmat20_permuted(dbs, torch, args, rp, ci, 1 << 20)}), flush=True)
        return
    res = bench_rmat20(dbs, torch, args)
    log(f"[bench] rmat20 sweep: {res['ms_per_step']:.3f} ms/step, {res['value']:.1f} GB/s")
    extra = {"rmat20_per_density": res["per_density"], "rmat20_forced_paths": res["forced_paths"],
             "rmat20_xb_crossover": res["xb_crossover"],
             "rmat20_format": res["format"], "rmat20_build_s": round(res["build_s"], 2)}
    cpu = None
    if args.headline_only:
        args.no_cpu = args.no_bfs = args.no_decode = args.no_zipf = args.no_ablations = args.no_tiny = True
        args.no_permuted = True
    if not args.no_cpu:
        cpu = cpu_baseline_rmat20(res, args.cpu_seconds)
        log(f"[bench] cpu baseline: {cpu}")
    if not args.no_permuted:
        rp, ci, n = res["graph"]
        extra["rmat20_permuted"] = bench_rmat20_permuted(dbs, torch, args, rp, ci, n)
        log(f"[bench] rmat20 permuted: {extra['rmat20_permuted']}")
        del rp, ci
    del res["graph"], res["xs"]
    if not args.no_bfs:
        extra["bfs_rmat22"] = bench_bfs22(dbs, torch, args)
        log(f"[bench] bfs: {extra['bfs_rmat22']}")
    if not args.no_decode:
        extra["decode"] = bench_decode(dbs, torch, args)
    if not args.no_tiny:
        extra["tiny"] = bench_tiny(dbs, torch, args)
    if not args.no_zipf:
        extra["zipf_band"] = bench_zipf(dbs, torch, args)
    if not args.no_ablations:
        extra["format_ablation"] = bench_format_ablation(dbs, torch, args)
        extra["decode_dense_threshold_ablation"] = bench_decode_th1(dbs, torch, args)
    traffic = load_traffic("rmat20_sweep")
    copy_gbps = measure_copy_gbps(torch)
    log(f"[bench] device copy: {copy_gbps} GB/s (read + write)")
    read_gbps = measure_read_gbps(dbs, torch)
    log(f"[bench] device read: {read_gbps} GB/s")
    line = {
        "metric": METRIC,
        "value": round(res["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": "rmat20_or_and_density_sweep", "vertices": 1 << 20, "edge_factor": 16,
                   "rmat_abc": [0.57, 0.19, 0.19], "semiring": "or-and", "x_densities": DENSITIES,
                   "calls_per_step": len(DENSITIES), "tile": 16},
        "roofline": {"bound": "hbm", "achieved": round(res["achieved"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(res["achieved"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "k_spmspv<pattern, or-and>", "kernel_avg_us": round(res["kernel_avg_us"], 2),
                     "algorithmic_bytes_per_launch": int(res["comp_bytes_per_launch"]),
                     "measured_copy_GBps": copy_gbps,
                     "frac_of_measured_copy": round(res["achieved"] / copy_gbps, 4),
                     "measured_read_GBps": read_gbps,
                     "frac_of_measured_read": round(res["achieved"] / read_gbps, 4)},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
