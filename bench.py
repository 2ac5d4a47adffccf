"""Benchmark of the Tessera hot path on one MI355X.

A step is one velocity-Verlet MD step of the whole path: energy + forces of the 4-layer
l_max=2 model and the integrator, with the neighbour rebuild (Hilbert sort, cells, r_c+skin
candidate list) every 20 steps, as tess_md_steps runs it. The workload is salt60k: 60,000
atoms at 0.1 atoms/A^3 (one GPU's share of 30.7M atoms over 512 ranks), synthetic seeded
positions and random-init weights. The timed call runs --steps MD steps from device-resident
inputs.

Output: one JSON line with the throughput (atom-steps/s), the rebuild and E+F times, the
roofline position of the dominant kernel (HIP events around its launches, on the stream the
library launches it on), and the fp64 oracle timed on the host cores on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "atom-steps/s (E+F, 4-layer l<=2) at 60K atoms on 1 GPU; neighbor rebuild ms"
PEAK_FP32_VECTOR_TFLOPS = 157.3  # MI355X fp32 vector, 256 CUs x 2.4 GHz (packed issue)
PEAK_FP32_MFMA_TFLOPS = 157.3    # MI355X dense fp32 matrix cores
# the edge contractions run their channel sums on the matrix cores; the gradients are
# vector-ALU work
BOUND = {"edge_apply": "mfma", "edge_tapply": "mfma", "edge_grad": "alu", "edge_grad_last": "alu"}
PEAK_HBM_GBS = 8000.0


def edge_kernel_flops(spec, n_active: int) -> dict:
    """Algorithmic fp32 flops (FMA = 2) of the edge kernels over one E+F pass, counting only
    the defining contractions (lower-order per-edge terms are left out) and only the parts
    the energy depends on. The first layer's input features have only the l = 0 component,
    and the energy reads only the l = 0 channels of the last layer, whose m and m_bar are
    then needed only in component 0:
      edge_apply : sum_e alpha A_e h_j  -> C*D*D MAC per edge (first and last layers: C*D)
      edge_grad  : Abar^h = sum_c mbar (x) h_j -> C*D*D MAC per edge (first layer: C*D)
      edge_grad_last: the same at the last layer, one row of Abar -> C*D MAC per edge
      edge_tapply: A_e^T mbar -> C*D*D MAC per edge (layers 1..T-1; the last: C*D)
      logits     : <q_i, k_j> -> C MAC per edge (layers after the first; the first layer's
                   come from a per-species table)"""
    C, T = spec.channels, spec.n_layers
    D = (spec.l_max + 1) ** 2
    full, one = C * D * D, C * D
    mac = {"edge_apply": 0, "edge_grad": 0, "edge_grad_last": 0, "edge_tapply": 0,
           "logits": 0}
    for t in range(T):
        first, last = t == 0, t == T - 1 and t > 0
        mac["edge_apply"] += one if (first or last) else full
        mac["edge_grad_last" if last else "edge_grad"] += one if (first or last) else full
        if t > 0:
            mac["edge_tapply"] += one if last else full
        mac["logits"] += 0 if first else C
    return {k: 2.0 * n_active * v for k, v in mac.items()}


def cpu_baseline(n_sample: int = 8000) -> dict:
    """The fp64 oracle on the host cores: one rebuild + one E+F on a bounded sample."""
    import oracle
    from molecular_dynamics_hilbert_amd import workloads as W
    wl = W.salt_box(n_sample, 1103, W.big_model(), "salt%dk" % (n_sample // 1000))
    w = W.make_weights(wl.model, 2003)
    oracle.build()
    t0 = time.perf_counter()
    nb = oracle.build_neighbors(wl.box, wl.pos, wl.species, wl.model.r_cut, wl.skin)
    t1 = time.perf_counter()
    oracle.energy_forces(wl.model, w, wl.box, nb["pos"].astype(np.float64), nb["species"],
                         nb["row_ptr"], nb["col_shift"])
    t2 = time.perf_counter()
    t_rb, t_ef = t1 - t0, t2 - t1
    cores = oracle.num_threads()
    return {"value": n_sample / (t_ef + t_rb / 20.0), "unit": "atom-steps/s", "cores": cores,
            "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": ("%d atoms at the salt60k density and species mix (periodic box %.2f A), "
                       "same 4-layer 64-channel l_max=2 model; one rebuild (%.2f s) + one E+F "
                       "(%.2f s) in fp64; atom-steps/s = N / (t_EF + t_rebuild/20)"
                       % (n_sample, float(wl.box[0]), t_rb, t_ef))}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="salt60k")
    ap.add_argument("--temperature", type=float, default=300.0,
                    help="Maxwell velocities of the timed run (K)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-large", action="store_true",
                    help="skip the 500,000-atom rebuild and E+F timing")
    ap.add_argument("--graph", action="store_true",
                    help="replay each rebuild interval from a captured HIP graph "
                         "(TESS_MD_GRAPH); per-kernel timing then comes from a second, eager "
                         "pass of the same length")
    ap.add_argument("--curve", choices=("hilbert", "morton"), default="hilbert",
                    help="atom order of the rebuilds (morton: locality comparison)")
    ap.add_argument("--no-hooks", action="store_true",
                    help="time the MD steps without the per-kernel HIP events (A/B of their "
                         "cost); per-kernel timing then comes from a second pass")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the benchmark, copy this many MiB device-to-device once (a plain "
                         "copy kernel of known size, to scale HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (sharding is "
              "described in DESIGN.md); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    # all work on one created stream (default priority): HIP graphs cannot be captured on the
    # NULL stream, and eager and graph runs then share the same stream setup
    with torch.cuda.stream(torch.cuda.Stream()):
        run(args)


def run(args):
    import torch

    from molecular_dynamics_hilbert_amd import tess as T
    from molecular_dynamics_hilbert_amd import workloads as W

    dev = "cuda"
    T.set_curve(args.curve)
    wl = W.load(args.workload)
    seed = {"salt60k": 2003, "capsid39k": 2004, "salt500k": 2005}.get(args.workload, 2003)
    w = W.make_weights(wl.model, seed)
    vel0 = W.maxwell_velocities(wl.species, wl.masses(), args.temperature, 3003)
    s = T.System(wl, w, vel=None)
    vel = torch.from_numpy(vel0).to(dev)
    masses = torch.from_numpy(wl.masses().astype(np.float32)).to(dev)
    pa = torch.arange(wl.n, dtype=torch.int32, device=dev)
    ep = torch.zeros(max(args.steps, args.warmup, 1), dtype=torch.float64, device=dev)
    every = wl.rebuild_every

    skin_flags = [0]

    def md(nsteps, valid, graph=False, state=None):
        """Run nsteps as whole rebuild intervals (one tess_md_steps call per interval, each
        starting with a rebuild). Random weights bind nothing, so at 300 K the fastest H atoms
        can pass skin/2 inside an interval; the library then reports TESS_ERR_SKIN after
        finishing it. Such intervals are counted, not aborted."""
        ss, vv, pp = state if state is not None else (s, vel, pa)
        done = 0
        while done < nsteps:
            k = min(every, nsteps - done)
            st, _ = T.md_steps(ss.spec, ss.weights, ss.box, ss.r_cut, ss.skin, ss.pos, vv,
                               ss.species, masses, wl.dt_fs, k, every, pp, ss.forces, ss.row_ptr,
                               ss.col_shift, ss.rev, ss.ws, epot_trace=ep,
                               forces_valid=valid or done > 0, graph=graph, check=False)
            if st == T.ERR_SKIN:
                skin_flags[0] += 1
            elif st != T.OK:
                raise T.TessError(st, "tess_md_steps")
            done += k

    # warmup (first call computes the initial forces; with --graph it also captures the graph)
    md(max(args.warmup, 1), False, args.graph)
    torch.cuda.synchronize()
    skin_flags[0] = 0
    names = ("edge_radial", "logits", "edge_apply", "edge_grad", "edge_grad_last", "edge_tapply",
             "node_gemm", "radix_scatter", "nbr_count", "nbr_fill")
    # profile pass (same length): HIP events around every instrumented kernel, giving the
    # per-kernel times and the dominant edge kernel
    T.timing_enable(True)
    md(args.steps, True)
    torch.cuda.synchronize()
    kern = {k: T.timing_read(k) for k in names}
    T.timing_enable(False)
    dom = max(("edge_apply", "edge_grad", "edge_grad_last", "edge_tapply"),
              key=lambda k: kern[k][0])
    skin_flags[0] = 0
    # timed region: exactly `steps` MD steps, inputs resident in HBM. Only the dominant kernel
    # carries HIP events in it (its roofline numbers come from this region); --graph and
    # --no-hooks time a region without any events and take the dominant kernel's times from
    # the profile pass
    hooks_in_region = not (args.graph or args.no_hooks)
    if hooks_in_region:
        T.timing_only(dom)
        T.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    md(args.steps, True, args.graph)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t0
    skin_timed = skin_flags[0]
    if hooks_in_region:
        kern[dom] = T.timing_read(dom)
        T.timing_enable(False)
        T.timing_only(None)
    value = wl.n * args.steps / t_total
    ms_per_step = 1e3 * t_total / args.steps

    # The same timed region on a fresh copy of the workload with 50 K velocities: random
    # weights bind nothing, so at 300 K the fastest free-flying H atoms can pass skin/2 inside
    # a 20-step interval (the library finishes such an interval and reports it), and the
    # random-weight potential keeps accelerating the atoms it has run for a while; from the
    # generated start at 50 K no interval is flagged. The work per step is the same
    # fixed-shape pass, so the two throughputs agree within noise.
    skin_run = None
    if args.temperature != 50.0:
        s50 = T.System(wl, w)
        v50 = torch.from_numpy(W.maxwell_velocities(wl.species, wl.masses(), 50.0, 3003)).to(dev)
        p50 = torch.arange(wl.n, dtype=torch.int32, device=dev)
        md(max(args.warmup, 1), False, args.graph, (s50, v50, p50))
        torch.cuda.synchronize()
        skin_flags[0] = 0
        t0 = time.perf_counter()
        md(args.steps, True, args.graph, (s50, v50, p50))
        torch.cuda.synchronize()
        t50 = time.perf_counter() - t0
        del s50
        skin_run = {"temperature_K": 50.0, "value": round(wl.n * args.steps / t50, 1),
                    "ms_per_step": round(1e3 * t50 / args.steps, 4),
                    "skin_flagged_intervals": skin_flags[0],
                    "kernel_events_in_timed_region": None}

    # separate timings: rebuild alone and E+F alone (median of 5, HIP events on the stream)
    st = torch.cuda.current_stream()
    s.vel = None
    rb, ef = [], []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        s.rebuild()  # synchronises once inside (pair count)
        b.record(st)
        torch.cuda.synchronize()
        rb.append(a.elapsed_time(b))
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        s.energy_forces()
        b.record(st)
        torch.cuda.synchronize()
        ef.append(a.elapsed_time(b))
    # pairs inside r_cut (the edges the model works on), counted on the host from the CSR
    rp = s.row_ptr.cpu().numpy()
    n_cand = int(rp[-1])
    n_active = _count_active(s, n_cand)

    flops = edge_kernel_flops(wl.model, n_active)
    ef_calls = args.steps  # E+F passes inside the timed region (forces were valid on entry)
    rows = {}
    for k, (ms, cnt) in kern.items():
        if cnt:
            rows[k] = {"launches": cnt, "avg_ms": ms / cnt, "total_ms": ms}
    dom_ms, dom_cnt = kern[dom]
    dom_flops = flops[dom] * ef_calls
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12 if dom_ms > 0 else 0.0
    peak = PEAK_FP32_MFMA_TFLOPS if BOUND[dom] == "mfma" else PEAK_FP32_VECTOR_TFLOPS
    roofline = {"kernel": dom, "bound": BOUND[dom], "achieved": round(achieved, 3),
                "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": _traffic(dom, args.workload),
                "avg_launch_ms": dom_ms / max(dom_cnt, 1), "launches": dom_cnt,
                "flops_per_ef_pass": flops[dom]}
    # the same figures for every edge kernel (times from the profile pass, where each
    # instrumented kernel carries events; the dominant kernel's above come from the timed region)
    edge_rooflines = {}
    for k in ("edge_apply", "edge_grad", "edge_grad_last", "edge_tapply"):
        k_ms, k_cnt = kern[k]
        if k_ms <= 0:
            continue
        a = flops[k] * ef_calls / (k_ms * 1e-3) / 1e12
        pk = PEAK_FP32_MFMA_TFLOPS if BOUND[k] == "mfma" else PEAK_FP32_VECTOR_TFLOPS
        edge_rooflines[k] = {"bound": BOUND[k], "achieved": round(a, 3), "peak": pk,
                             "unit": "TFLOP/s", "frac": round(a / pk, 4),
                             "traffic": _traffic(k, args.workload),
                             "avg_launch_ms": round(k_ms / max(k_cnt, 1), 4), "launches": k_cnt}
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "atom-steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "n_atoms": wl.n, "box_A": float(wl.box[0]),
                   "layers": wl.model.n_layers, "channels": wl.model.channels,
                   "l_max": wl.model.l_max, "heads": wl.model.n_heads,
                   "rebuild_every": every, "dt_fs": wl.dt_fs, "pairs_r_c_plus_skin": n_cand,
                   "pairs_r_c": n_active, "temperature_K": args.temperature,
                   "skin_flagged_intervals": skin_timed,
                   "launch": "hip_graph" if args.graph else "eager", "curve": args.curve,
                   "kernel_events_in_timed_region": dom if hooks_in_region else None},
        "skin_holding_run": skin_run,
        "rebuild_ms": round(statistics.median(rb), 4),
        "ef_ms": round(statistics.median(ef), 4),
        "roofline": roofline,
        "edge_rooflines": edge_rooflines,
        "kernels_ms": {k: round(v["avg_ms"], 4) for k, v in rows.items()},
        "large_system": None if args.no_large else large_system(),
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(),
    }
    print(json.dumps(out), flush=True)
    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()


def large_system(name: str = "salt500k") -> dict:
    """Rebuild and E+F of the 500,000-atom box (edge 171 A, 4-layer model): medians of 5
    rebuilds and 3 E+F passes after one of each untimed, HIP events on the stream."""
    import torch

    from molecular_dynamics_hilbert_amd import tess as T
    from molecular_dynamics_hilbert_amd import workloads as W
    wl = W.load(name)
    s = T.System(wl, W.make_weights(wl.model, 2005))
    st = torch.cuda.current_stream()

    def timed(fn, reps):
        out = []
        for _ in range(reps + 1):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            fn()
            b.record(st)
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b))
        return statistics.median(out[1:])

    rb = timed(s.rebuild, 5)
    ef = timed(s.energy_forces, 3)
    n_cand = s.n_edges
    res = {"workload": name, "n_atoms": wl.n, "box_A": float(wl.box[0]),
           "pairs_r_c_plus_skin": n_cand, "rebuild_ms": round(rb, 4), "ef_ms": round(ef, 3),
           "ef_atom_steps_per_s": round(wl.n / (ef * 1e-3), 1)}
    del s
    torch.cuda.empty_cache()
    return res


def _traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (profiles/traffic_<kernel>_<workload>.json), or None when there is none or the sources
    it names (all of csrc/ if it names none) changed since the counters were taken."""
    from molecular_dynamics_hilbert_amd import profiling
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != profiling.source_digest(t.get("source_files")):
        return None
    return round(t["bytes_per_launch"], 1)


def _count_active(s, n_cand: int) -> int:
    """Pairs with r < r_cut, counted from the device CSR with fp32 geometry (as the library)."""
    pos = s.pos.cpu().numpy()
    rp = s.row_ptr.cpu().numpy()
    col = s.col_shift[:n_cand].cpu().numpy().view(np.uint32)
    i = np.repeat(np.arange(s.n), np.diff(rp))
    j = (col & 0x7FFFFFF).astype(np.int64)
    code = (col >> 27).astype(np.int64)
    sh = np.stack([code // 9 - 1, (code // 3) % 3 - 1, code % 3 - 1], 1).astype(np.float32)
    r = (pos[j] - pos[i]) + sh * np.asarray(s.box, np.float32)
    return int(((r * r).sum(1) < np.float32(s.r_cut) ** 2).sum())


if __name__ == "__main__":
    main()
