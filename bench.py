#!/usr/bin/env python
"""Benchmark: edges/s of one fused SO(2) convolution step (forward + backward +
double backward) on one MI355X.

Workload: the UMA/eSEN-like medium system -- 10,000 atoms at 0.08 atoms/A^3 in
a periodic cube, 6 A cutoff (~725k directed edges), lmax 4, mmax 2, C 128,
64 Gaussian radial basis functions, float32, weights ~ N(0, 1/C). Synthetic,
seeded (so2_synth). A step runs so2conv_fwd (keeping the differentiation
state), so2conv_bwd (all gradients, including weights and positions) and
so2conv_dbwd (the force-training pattern: directions on x, positions and rbf),
exactly as training on forces needs them (TrimSO(2) page, Appendix A.3).

The JSON line carries the live roofline of the dominant kernel (the
matrix-core GEMM of the per-order linears, timed with HIP events on its
stream) and the CPU oracle timed on the host cores on a bounded edge sample.

--config / --dtype select another workload of so2_synth (e.g. the
EquiformerV3-like high-degree system H with its bfloat16 features and
weights) for the same step; the default is the medium system in float32.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

def metric_name(lmax, channels, two_stage):
    stages = "fwd+bwd" if two_stage else "fwd+bwd+dbwd"
    return f"edges/sec {stages} SO(2) conv (lmax={lmax},C={channels}); HBM GB/s % of peak"


PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_BF16_MFMA_TFLOPS = 2500.0     # dense
PEAK_HBM_GBS = 8000.0
SPLIT_PRODUCTS = 6                 # bf16 MFMA products per float32 product of the split GEMMs
WORKLOADS = {"T": "tiny periodic radius graph", "S": "eSEN-like small periodic radius graph",
             "M": "UMA/eSEN-like medium periodic radius graph", "H": "EquiformerV3-like high-degree periodic radius graph",
             "X": "large clustered periodic radius graph", "P1": "EquiformerV3 captured-batch-sized radius graph",
             "P2": "uniform random K-target graph"}


def gemm_flops_per_edge(L, M, C):
    """F = 2 (MAC1 + MAC2): per-edge multiply-adds of the two per-order linears
    (input width 2C for the first, with its L*C gate columns)."""
    s = sum((L - m + 1) ** 2 for m in range(1, M + 1))
    mac1 = 2 * C * C * ((L + 1) * (2 * L + 1) + 4 * s)
    mac2 = C * C * ((L + 1) ** 2 + 4 * s)
    return 2.0 * (mac1 + mac2)


def host_cores():
    """Cores this process may run on: its CPU affinity, limited by a cgroup CPU
    quota when one is set (a container's share of the host)."""
    n = len(os.sched_getaffinity(0))
    try:
        quota, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if quota != "max":
            n = max(1, min(n, int(float(quota) / float(period))))
    except (OSError, ValueError):
        pass
    return n


def _sources_sha256():
    import hashlib
    csrc = os.path.join(ROOT, "so_graph_convolution_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp", ".cpp", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def measured_step_traffic(config, dtype, keep_bwd, ms_step):
    """HBM bytes of one whole step from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    record (copy-calibrated, every kernel of the step), if the record covers this
    workload and launch mix and every kernel source is unchanged since; else None."""
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", f"hbm_bytes_step_{config}_{dtype}.json")))
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != _sources_sha256() or bool(rec.get("backward_cotangents_kept")) != bool(keep_bwd):
        return None
    b = float(rec["step_bytes"])
    return {"counted_bytes_per_step": b, "GBps": b / (ms_step * 1e-3) / 1e9,
            "frac_of_peak": b / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, "peak_GBps": PEAK_HBM_GBS,
            "per_stage_bytes": rec.get("per_stage_bytes"), "source": rec.get("summary")}


def measured_gemm_traffic(config, dtype, keep_bwd, split):
    """HBM bytes per GEMM launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    counters (copy-calibrated) of the medium float32 step, or None for another
    workload, another launch mix (backward cotangents kept or not, split or
    float32 products) or if a GEMM source changed since."""
    import hashlib
    if config != "M" or dtype != "f32":
        return None
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "gemm_hbm_traffic_medium.json")))
        csrc = os.path.join(ROOT, "so_graph_convolution_amd", "csrc")
        src = b"".join(open(os.path.join(csrc, f), "rb").read()
                       for f in ("gemm.hip", "gemm.hpp", "gemm_x3.hip", "gemm_s3.hip", "gemm_dma.hpp", "gemm_tile.hpp"))
    except OSError:
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("kernel_source_sha256"):
        return None
    if bool(rec.get("backward_cotangents_kept")) != bool(keep_bwd) or bool(rec.get("split_products")) != bool(split):
        return None
    return rec["gemm_bytes_per_step"] / rec["gemm_launches_per_step"]


def cpu_baseline(d, n_edges_sample, seed=0, dbwd=True):
    """Time the float64 oracle (fwd, bwd and, with dbwd, the double backward) on a
    leading block of edges."""
    import numpy as np
    import torch
    from oracle import so2conv_oracle as O
    torch.set_num_threads(host_cores())
    inp = O.to_oracle_inputs(d)
    E = len(d["src"])
    n = min(n_edges_sample, E)
    edges = np.arange(n)
    t = lambda a: torch.tensor(a, dtype=torch.float64)  # noqa: E731
    gy = t(d["gy"])
    O.backward(inp, gy, chunk=2048, edges=np.arange(min(256, E)))       # warmup (thread pool, allocator)
    t0 = time.perf_counter()
    O.forward(inp, chunk=2048, edges=edges)
    O.backward(inp, gy, chunk=2048, edges=edges)
    if dbwd:
        O.double_backward(inp, gy, px=t(d["px"]), ppos=t(d["ppos"]), prbf=t(d["prbf"]), chunk=2048, edges=edges)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "edges/s", "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"first {n} of {E} edges of the same workload, {'fwd+bwd+dbwd' if dbwd else 'fwd+bwd'} in "
                      f"float64 (PyTorch CPU, autograd) after a 256-edge warmup, {dt:.1f} s; "
                      f"{len(os.sched_getaffinity(0))} cores in the process's affinity"}


def cpu_baseline_mole(d, m, n_edges_sample):
    """Time the float64 mixture oracle (fwd, bwd, dbwd) on a leading block of
    edges (the systems' edge ranges clipped to it)."""
    import numpy as np
    import torch
    from oracle import mole_oracle as MO
    from oracle import so2conv_oracle as O
    torch.set_num_threads(host_cores())
    base = O.to_oracle_inputs(d)
    E = len(d["src"])
    n = min(n_edges_sample, E)
    sp = np.minimum(m["sys_edge_ptr"], n).tolist()
    t = lambda a: torch.tensor(np.asarray(a), dtype=torch.float64)  # noqa: E731
    w1e, w2e, coef, gy = [t(w) for w in m["w1e"]], [t(w) for w in m["w2e"]], t(m["coef"]), t(d["gy"])
    t0 = time.perf_counter()
    MO.forward(base, w1e, w2e, coef, sp, chunk=2048)
    MO.backward(base, w1e, w2e, coef, sp, gy, chunk=2048)
    MO.double_backward(base, w1e, w2e, coef, sp, gy, px=t(d["px"]), ppos=t(d["ppos"]), prbf=t(d["prbf"]),
                       chunk=2048)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "edges/s", "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"first {n} of {E} edges of the same workload, fwd+bwd+dbwd in float64 "
                      f"(PyTorch CPU, autograd, mixture oracle), {dt:.1f} s"}


def bench_grid(args):
    """Node-to-node spherical projection (U = sum_l G_l X^(l) W_l A; Appendix B.4) at
    EquiformerV3's widths (lmax 4, C 128, FFN hidden 512) on the medium system's
    10,000 nodes, a 100-point grid: fwd + bwd + dbwd (all directions)."""
    import numpy as np
    import torch
    import so_graph_convolution_amd as K

    def progress(msg):
        print(f"[bench grid] {msg}", file=sys.stderr, flush=True)
    L, ci, ch, co, ng, N = 4, 128, 512, 512, 100, 10000
    d = (L + 1) ** 2
    rng = np.random.default_rng(7)
    host = dict(x=rng.normal(size=(N, d, ci)), G=rng.normal(size=(ng, d)) / np.sqrt(d),
                W=rng.normal(size=(L + 1, ci, ch)) / np.sqrt(ci), A=rng.normal(size=(ch, co)) / np.sqrt(ch),
                gU=rng.normal(size=(N, ng, co)), px=rng.normal(size=(N, d, ci)),
                pW=rng.normal(size=(L + 1, ci, ch)) / np.sqrt(ci), pA=rng.normal(size=(ch, co)) / np.sqrt(ch))
    g = {k: torch.tensor(v.astype(np.float32), device="cuda") for k, v in host.items()}
    cfg = K.GridConfig(L, ci, ch, co, ng)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(times=None):
        e = [ev() for _ in range(4)]
        e[0].record()
        K.so2grid_fwd(cfg, g["x"], g["G"], g["W"], g["A"])
        e[1].record()
        K.so2grid_bwd(cfg, g["x"], g["G"], g["W"], g["A"], g["gU"])
        e[2].record()
        K.so2grid_dbwd(cfg, g["x"], g["G"], g["W"], g["A"], g["gU"], px=g["px"], pW=g["pW"], pA=g["pA"])
        e[3].record()
        if times is not None:
            times.append(e)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    st = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([[a.elapsed_time(b) for a, b in zip(e[:-1], e[1:])] for e in st]).mean(0)
    # algorithmic HBM bytes of the forward: read x, G, W, A; write U
    fwd_bytes = 4.0 * (N * d * ci + ng * d + (L + 1) * ci * ch + ch * co + N * ng * co)
    out = {"metric": "nodes/sec fwd+bwd+dbwd spherical projection (lmax=4, c 128/512/512, 100-point grid)",
           "value": N * args.steps / wall, "unit": "nodes/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
           "dtype": "f32", "data": "synthetic",
           "config": {"workload": "EquiformerV3-width node-to-node spherical projection on 10,000 nodes",
                      "lmax": L, "c_in": ci, "c_h": ch, "c_out": co, "n_grid": ng, "n_nodes": N},
           "stage_ms": {"fwd": float(ms[0]), "bwd": float(ms[1]), "dbwd": float(ms[2])},
           "fwd_hbm": {"algorithmic_bytes": fwd_bytes, "GBs": fwd_bytes / (ms[0] * 1e-3) / 1e9,
                       "frac_of_8TBs": fwd_bytes / (ms[0] * 1e-3) / 8e12},
           "materialising_bytes_avoided": 4.0 * (N * d * ch + N * ng * ch) * 2}
    progress(f"{out['ms_per_step']:.2f} ms/step")
    if args.cpu_edges > 0:
        import oracle.grid_oracle as GO
        torch.set_num_threads(host_cores())
        n = 200
        r = {k: torch.tensor(v[:n] if k in ("x", "gU", "px") else v, dtype=torch.float64) for k, v in host.items()}
        t1 = time.perf_counter()
        GO.forward(r["x"], r["G"], r["W"], r["A"])
        GO.backward(r["x"], r["G"], r["W"], r["A"], r["gU"])
        GO.double_backward(r["x"], r["G"], r["W"], r["A"], r["gU"], px=r["px"], pW=r["pW"], pA=r["pA"])
        dt = time.perf_counter() - t1
        out["cpu_baseline"] = {"value": n / dt, "unit": "nodes/s", "cores": torch.get_num_threads(), "kind": "oracle",
                               "sample": f"first {n} of {N} nodes, fwd+bwd+dbwd in float64, {dt:.1f} s"}
    print(json.dumps(out), flush=True)


def bench_s2act(args):
    """Spherical-grid SwiGLU activation on edges (EquiformerV3's Edge -> Edge
    activation; Table 2, Appendix C.1 and Appendix B.4) at the high-degree
    system's size: 1,045,678 edges, 29 retained rows (lmax 6, mmax 2), C 128
    (U carries 2C), a 100-point grid; fwd + bwd + dbwd (both outputs)."""
    import numpy as np
    import torch
    import so_graph_convolution_amd as K

    def progress(msg):
        print(f"[bench s2act] {msg}", file=sys.stderr, flush=True)
    E, q, C, ng = 1045678, 29, 128, 100
    gen = torch.Generator(device="cuda").manual_seed(11)
    g = dict(U=torch.randn(E, q, 2 * C, device="cuda", generator=gen),
             gZ=torch.randn(E, q, C, device="cuda", generator=gen),
             pU=torch.randn(E, q, 2 * C, device="cuda", generator=gen),
             G=torch.randn(ng, q, device="cuda", generator=gen) / math.sqrt(q),
             P=torch.randn(q, ng, device="cuda", generator=gen) / math.sqrt(ng))
    cfg = K.S2Config(q, C, ng)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    progress(f"E={E} rows={q} C={C} n_grid={ng}")

    def step(times=None):
        e = [ev() for _ in range(4)]
        e[0].record()
        K.so2s2_fwd(cfg, g["U"], g["G"], g["P"])
        e[1].record()
        K.so2s2_bwd(cfg, g["U"], g["G"], g["P"], g["gZ"])
        e[2].record()
        K.so2s2_dbwd(cfg, g["U"], g["G"], g["P"], g["gZ"], g["pU"])
        e[3].record()
        if times is not None:
            times.append(e)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    st = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([[a.elapsed_time(b) for a, b in zip(e[:-1], e[1:])] for e in st]).mean(0)
    # contraction flops per (edge, channel, grid point) as the kernels compute
    # them (grid values recomputed, never stored): fwd 6q, bwd 10q, dbwd 16q
    units = float(E) * C * ng
    flops = {"fwd": 6 * q * units, "bwd": 10 * q * units, "dbwd": 16 * q * units}
    # the matrix cores see rows and grid points padded to whole 16x16x4 tiles:
    # 8 products of 2 x 16*ceil(q/16) x 16*ceil(ng/16) per dbwd column
    issued = 8 * 2 * (16 * -(-q // 16)) * (16 * -(-ng // 16)) * float(E) * C
    ach = flops["dbwd"] / (ms[2] * 1e-3) / 1e12
    out = {"metric": "edges/sec fwd+bwd+dbwd SwiGLU-S2 edge activation (lmax=6, mmax=2, C=128, 100-point grid)",
           "value": E * args.steps / wall, "unit": "edges/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": "SwiGLU-S2 on the edges of the EquiformerV3-like high-degree system",
                      "n_edges": E, "rows": q, "channels": C, "n_grid": ng},
           "stage_ms": {"fwd": float(ms[0]), "bwd": float(ms[1]), "dbwd": float(ms[2])},
           "roofline": {"bound": "mfma", "kernel": "s2_dbwd_kernel", "achieved": ach,
                        "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s", "frac": ach / PEAK_FP32_MFMA_TFLOPS,
                        "traffic": None, "flops_per_launch": flops["dbwd"], "flops_issued_per_launch": issued}}
    progress(f"{out['ms_per_step']:.2f} ms/step  stages {ms.round(2).tolist()}  dbwd {ach:.1f} TFLOP/s")
    if args.cpu_edges > 0:
        import oracle.s2act_oracle as SO
        torch.set_num_threads(host_cores())
        n, chunk = min(args.cpu_edges, 8192), 2048
        h = {k: v.double().cpu() for k, v in (("G", g["G"]), ("P", g["P"]))}
        t1 = time.perf_counter()
        for i in range(0, n, chunk):
            U, gZ, pU = (g[k][i:i + chunk].double().cpu() for k in ("U", "gZ", "pU"))
            SO.forward(U, h["G"], h["P"])
            SO.backward(U, h["G"], h["P"], gZ)
            SO.double_backward(U, h["G"], h["P"], gZ, pU)
        dt = time.perf_counter() - t1
        out["cpu_baseline"] = {"value": n / dt, "unit": "edges/s", "cores": torch.get_num_threads(), "kind": "oracle",
                               "sample": f"first {n} of {E} edges, fwd+bwd+dbwd in float64 (PyTorch CPU, autograd), "
                                         f"{chunk}-edge chunks, {dt:.1f} s"}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="M")
    ap.add_argument("--dtype", choices=("f32", "bf16"), default=None,
                    help="array dtype (default: the workload's own: f32 for M, bf16 for H and X)")
    ap.add_argument("--f32-native", action="store_true",
                    help="float32 per-order products on the float32 matrix cores (SO2_F32_NATIVE) instead of the "
                         "default bfloat16-piece products")
    ap.add_argument("--pos2", action="store_true",
                    help="the double backward also returns position derivatives (gpos2)")
    ap.add_argument("--op", choices=("conv", "grid", "mole", "s2act"), default="conv",
                    help="conv: the SO(2) convolution step (default); grid: the node-to-node spherical projection; "
                         "mole: the convolution with a system-dependent mixture of linear experts; "
                         "s2act: the spherical-grid SwiGLU activation on edges")
    ap.add_argument("--systems", type=int, default=16, help="systems of the batch (--op mole)")
    ap.add_argument("--experts", type=int, default=64, help="linear experts (--op mole; 64 for UMA)")
    ap.add_argument("--envelope", action="store_true",
                    help="per-edge cutoff envelope on the messages (with genv, and genv2 in the double backward)")
    ap.add_argument("--heads", type=int, default=1,
                    help="per-head attention weights on the messages (EquiformerV3: 8 heads), times the envelope")
    ap.add_argument("--act", choices=("gate", "swiglu_s2"), default="gate",
                    help="Edge -> Edge activation: the gate (eSEN/UMA) or the spherical-grid SwiGLU (EquiformerV3)")
    ap.add_argument("--n-grid", type=int, default=0,
                    help="grid points of --act swiglu_s2 (default 2(L+1) latitudes x (2M+3) longitudes)")
    ap.add_argument("--lmax", type=int, default=None, help="override the workload's lmax (sweeps)")
    ap.add_argument("--mmax", type=int, default=None, help="override the workload's mmax (sweeps)")
    ap.add_argument("--channels", type=int, default=None, help="override the workload's channels C (sweeps)")
    ap.add_argument("--n-atoms", type=int, default=None, help="override the workload's atom count (sweeps)")
    ap.add_argument("--k-targets", type=int, default=None,
                    help="override the targets per node of a K-target sweep graph (P2)")
    ap.add_argument("--cpu-edges", type=int, default=16384, help="edge sample of the CPU oracle baseline (0: skip)")
    ap.add_argument("--bounded-gib", type=float, default=32.0,
                    help="after the main line, time the same step with the workspace capped at this many GiB "
                         "(edge chunks), reported as bounded_memory (0: skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.ones(2 ** 28, device="cuda")          # 1 GiB of float32
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read_per_launch": src.numel() * 4, "copy_bytes_written_per_launch":
                          dst.numel() * 4, "launches": 3}), flush=True)
        return
    if args.op == "grid" and args.gpus == 1:
        bench_grid(args)
        return
    if args.op == "s2act" and args.gpus == 1:
        bench_s2act(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the convolution runs on a "
              "single MI355X, see the design notes on sharding)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import so2_synth
    import so_graph_convolution_amd as K

    def progress(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    cfg = so2_synth.CONFIGS[args.config]
    over = {k: v for k, v in (("lmax", args.lmax), ("mmax", args.mmax), ("channels", args.channels),
                              ("n_atoms", args.n_atoms), ("k_targets", args.k_targets)) if v is not None}
    if over:
        cfg = dataclasses.replace(cfg, **over)
    dtype = args.dtype or cfg.dtype
    if dtype == "bf16" and cfg.dtype != "bf16":
        cfg = dataclasses.replace(cfg, dtype="bf16")   # bf16-representable inputs
    s2 = args.act == "swiglu_s2"
    if s2:
        ng = args.n_grid or 2 * (cfg.lmax + 1) * (2 * cfg.mmax + 3)
        cfg = dataclasses.replace(cfg, act="swiglu_s2", n_grid=ng)
    d = so2_synth.make_inputs(cfg)
    progress(f"inputs ready: N={cfg.n_atoms} E={len(d['src'])}")
    E, N = len(d["src"]), cfg.n_atoms
    dev = torch.device("cuda:0")

    def t(a, dt=torch.float32):
        return torch.tensor(np.ascontiguousarray(a), dtype=dt, device=dev)

    ft = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = K.SO2Config(cfg.lmax, cfg.mmax, cfg.channels, cfg.n_rbf, dtype, heads=args.heads,
                     f32_native=args.f32_native, act=args.act,
                     grid=(t(d["grid_G"]), t(d["grid_P"])) if s2 else None)
    g = K.so2conv_graph_prepare(N, t(d["src"], torch.int32), t(d["dst"], torch.int32), t(d["shift"]))
    x, pos, rbf, w_rad = t(d["x"], ft), t(d["pos"]), t(d["rbf"]), t(d["w_rad"], ft)
    w1, w2 = [t(w, ft) for w in d["w1"]], [t(w, ft) for w in d["w2"]]
    gy, px, ppos, prbf = t(d["gy"], ft), t(d["px"], ft), t(d["ppos"]), t(d["prbf"])
    if args.heads > 1:
        args.envelope = True
        d["env"] = so2_synth.attention_weights(d, args.heads, seed=0) * so2_synth.cosine_envelope(d)[:, None]
    elif args.envelope:
        d["env"] = so2_synth.cosine_envelope(d)
    env = t(d["env"]) if args.envelope else None
    mole = args.op == "mole"
    if mole:   # the node range split into `systems` structures, each with its own coefficients
        mix_in = so2_synth.mixture_inputs(d, args.systems, args.experts, seed=0, bf16=dtype == "bf16")
        mix = K.Mixture(args.experts, mix_in["sys_edge_ptr"])
        w1e, w2e = [t(w, ft) for w in mix_in["w1e"]], [t(w, ft) for w in mix_in["w2e"]]
        coef = t(mix_in["coef"])
        progress(f"mixture: {args.systems} systems, {args.experts} experts")
    # the eSEN-like small and the large systems are specified as forward + backward
    two_stage = args.config in ("S", "X")
    db_need = ("gy", "x", "rbf", "w_rad", "w1", "w2") + (("pos",) if args.pos2 else ()) + \
        (("env",) if args.envelope else ())
    saved_b = K.so2conv_saved_bytes(kc, E)
    if mole:
        ws_b = max(K.so2mole_workspace_bytes(kc, mix, N, E, s, 0) for s in (0, 1, 2))
    else:
        ws_b = max(K.so2conv_workspace_bytes(kc, N, E, s) for s in (0, 1, 2))
    chunked = saved_b + ws_b > 200 * 2**30
    if chunked:   # workspace for chunks of about 256k edges (the library picks the chunk from its size)
        if mole:
            ws_b = max(K.so2mole_workspace_bytes(kc, mix, N, E, s, 262144) for s in (0, 1, 2))
        else:
            ws_b = max(K.so2conv_chunked_workspace_bytes(kc, N, E, s, 262144) for s in (0, 1, 2))
    # without room for the per-edge forward state (the large system), every
    # chunk recomputes it inside the workspace
    keep_state = saved_b + ws_b <= 200 * 2**30
    if not keep_state:
        saved_b = 0
    # the backward keeps its cotangents for the double backward of the same step
    # (one data-gradient product per linear less there) when memory allows
    sb_b = 0 if two_stage else K.so2conv_saved_bwd_bytes(kc, E)
    keep_bwd = not two_stage and keep_state and saved_b + ws_b + sb_b <= 230 * 2**30
    progress(f"saved state {saved_b / 2**30:.1f} GiB, workspace {ws_b / 2**30:.1f} GiB"
             + (" (edge chunks)" if chunked else "")
             + (f", backward cotangents kept {sb_b / 2**30:.1f} GiB" if keep_bwd else ""))
    saved = torch.empty(saved_b, dtype=torch.uint8, device=dev) if keep_state else None
    ws = torch.empty(ws_b, dtype=torch.uint8, device=dev)
    saved_bwd = torch.empty(sb_b, dtype=torch.uint8, device=dev) if keep_bwd else None
    args_c = (kc, g, x, pos, rbf, w_rad, w1, w2)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    args_m = (kc, g, mix, x, pos, rbf, w_rad, w1e, w2e, coef) if mole else None

    def step(times=None):
        e0, e1, e2, e3 = ev(), ev(), ev(), ev()
        e0.record()
        if mole:
            K.so2mole_fwd(*args_m, saved=saved, ws=ws, env=env)
            e1.record()
            K.so2mole_bwd(*args_m, saved, gy, ws=ws, env=env, saved_bwd=saved_bwd)
            e2.record()
            K.so2mole_dbwd(*args_m, saved, gy, px=px, ppos=ppos, prbf=prbf, ws=ws, env=env,
                           need=db_need + ("coef",), saved_bwd=saved_bwd)
        else:
            K.so2conv_fwd(*args_c, saved=saved, ws=ws, env=env)
            e1.record()
            K.so2conv_bwd(*args_c, saved, gy, ws=ws, env=env, saved_bwd=saved_bwd)
            e2.record()
            if not two_stage:
                K.so2conv_dbwd(*args_c, saved, gy, px=px, ppos=ppos, prbf=prbf, ws=ws, env=env, need=db_need,
                               saved_bwd=saved_bwd)
        e3.record()
        if times is not None:
            times.append((e0, e1, e2, e3))

    torch.cuda.reset_peak_memory_stats()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    progress("warmup done")
    K.so2conv_profile_reset()
    K.so2conv_profile_enable(True)
    stage = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(stage)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    K.so2conv_profile_enable(False)
    kinds = {0: "AB", 1: "ABt", 2: "AtB", 3: "ABt bf16", 4: "AtB bf16", 5: "AB complex", 6: "ABt complex",
             7: "AtB complex", 8: "AB pieces", 9: "ABt pieces", 10: "AtB pieces"}
    per_kind, raw = {}, {}
    for kind, name in kinds.items():
        n, ms, fl, by = K.so2conv_profile_read(kind)
        raw[kind] = (n, ms, fl, by)
        if n:
            per_kind[name] = {"launches": n, "avg_ms": ms / n, "algorithmic_tflops": fl / max(ms, 1e-9) / 1e9,
                              "algorithmic_bytes_per_launch": by / n}
    K.so2conv_profile_reset()
    # the dominant kernel: the per-order products (float32 through bfloat16 pieces,
    # SPLIT_PRODUCTS bf16 MFMA products per float32 product; float32 on the float32
    # matrix cores with SO2_F32_NATIVE; bfloat16), not the small radial products
    split = sum(raw[k][0] for k in (8, 9, 10)) > 0
    dom = (8, 9, 10) if split else ((3, 4) if dtype == "bf16" else (0, 1, 2, 5, 6, 7))
    n_l, gemm_ms, gemm_fl, gemm_by = (sum(raw[k][i] for k in dom) for i in range(4))
    st = np.array([[a.elapsed_time(b), b.elapsed_time(c), c.elapsed_time(e)] for a, b, c, e in stage])
    ms_step = wall * 1e3 / args.steps
    value = E * args.steps / wall
    F = gemm_flops_per_edge(cfg.lmax, cfg.mmax, cfg.channels)
    alg_tflops = gemm_fl / (gemm_ms * 1e-3) / 1e12
    executed = gemm_fl * (SPLIT_PRODUCTS if split else 1)
    achieved = executed / (gemm_ms * 1e-3) / 1e12
    peak = PEAK_BF16_MFMA_TFLOPS if (dtype == "bf16" or split) else PEAK_FP32_MFMA_TFLOPS
    if split:
        kname = ("gemm_s3_kernel (gemm_x3_kernel for gated launches): float32 per-order products (orders >= 1 "
                 "realified) with every operand the exact sum of three bfloat16 pieces, "
                 f"{SPLIT_PRODUCTS} bf16 MFMA products per float32 product")
    elif dtype == "bf16":
        kname = ("gemm_b3_kernel (A.B^T; gemm_b16_kernel for gated launches) and gemm_b16t_kernel (A^T.B weight "
                 "gradients): bf16 MFMA per-order linears")
    else:
        kname = ("gemm_f32_dma_kernel (order 0) and gemm_cplx_dma_kernel (orders >= 1, three real products per "
                 "complex one; fp32 MFMA)")
    kname += ", all launches of the timed steps"
    # Appendix B.5's intermediates of the separate-operation schedule (retained-order
    # layout, one stored copy each) and the per-edge forward state the fused path
    # keeps when it does not recompute: the memory a materialising implementation
    # would hold beyond the fused one
    qlm = sum(2 * min(l, cfg.mmax) + 1 for l in range(cfg.lmax + 1))
    dd_, C0, C1 = (cfg.lmax + 1) ** 2, 2 * cfg.channels, cfg.channels
    elem = 2 if dtype == "bf16" else 4
    mat_gib = elem * E * (dd_ * (C0 + C1) + qlm * (C0 + 2 * C1 + C1 + 2 * C1)) / 2**30
    out = {
        "metric": metric_name(cfg.lmax, cfg.channels, two_stage),
        "value": value,
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": f"{WORKLOADS.get(cfg.name, cfg.name)} ({cfg.name})", "n_atoms": N,
                   "n_edges": E, "lmax": cfg.lmax, "mmax": cfg.mmax, "channels": cfg.channels,
                   "n_rbf": cfg.n_rbf, "cutoff_A": cfg.rc, **({"k_targets": cfg.k_targets} if cfg.k_targets else {}),
                   "stages": ("fwd+bwd" if two_stage else "fwd+bwd+dbwd (force-training pattern)")
                   + (", dbwd with gpos2" if args.pos2 else "")
                   + (f", {args.heads}-head attention weights times the cutoff envelope" if args.heads > 1
                      else (", cutoff envelope" if args.envelope else ""))
                   + (f", mixture of {args.experts} linear experts over {args.systems} systems" if mole else "")
                   + (", float32 products on the float32 matrix cores" if args.f32_native and dtype == "f32" else "")
                   + (f", spherical-grid SwiGLU activation on {cfg.n_grid} grid points" if s2 else ""),
                   "edge_chunks": chunked, "forward_state_kept": keep_state, "backward_cotangents_kept": keep_bwd},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak,
                     "traffic": None if (mole or s2 or over) else measured_gemm_traffic(args.config, dtype, keep_bwd, split),
                     "algorithmic_bytes_per_launch": gemm_by / max(n_l, 1),
                     "kernel": kname,
                     "launches": n_l, "avg_launch_ms": gemm_ms / max(n_l, 1),
                     "executed_flops_per_step": executed / args.steps,
                     "algorithmic_flops_per_step": gemm_fl / args.steps,
                     "algorithmic_tflops": alg_tflops,
                     "algorithmic_frac_of_fp32_peak": alg_tflops / PEAK_FP32_MFMA_TFLOPS if dtype == "f32" else None,
                     "per_kind": per_kind},
        "stage_ms": {"fwd": float(st[:, 0].mean()), "bwd": float(st[:, 1].mean())} if two_stage else
        {"fwd": float(st[:, 0].mean()), "bwd": float(st[:, 1].mean()), "dbwd": float(st[:, 2].mean())},
        "step_gemm_share": gemm_ms / args.steps / ms_step,
        "peak_device_memory_GiB": torch.cuda.max_memory_allocated() / 2**30,
        "materialising_estimate_GiB": {"forward_state": K.so2conv_saved_bytes(kc, E) / 2**30,
                                       "separate_operation_intermediates": mat_gib},
        ("step_tflops_3F_equivalent" if two_stage else "step_tflops_8F_equivalent"):
            (3 if two_stage else 8) * F * E / (ms_step * 1e-3) / 1e12,
        "hbm": measured_step_traffic(args.config, dtype, keep_bwd, ms_step) if not (mole or args.envelope or s2 or over)
        else None,
    }
    progress(f"timed {args.steps} steps: {ms_step:.1f} ms/step")
    if args.bounded_gib > 0 and not mole and keep_state and not chunked:
        # the same step with the workspace capped (edge chunks), kept state and cotangents as above
        del ws
        torch.cuda.empty_cache()
        cap = args.bounded_gib * 2**30
        ce = 1 << max(12, int(math.log2(max(E, 4096))) + 1)
        while ce > 4096 and max(K.so2conv_chunked_workspace_bytes(kc, N, E, s_, ce) for s_ in (0, 1, 2)) > cap:
            ce //= 2
        ws = torch.empty(max(K.so2conv_chunked_workspace_bytes(kc, N, E, s_, ce) for s_ in (0, 1, 2)),
                         dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        step()
        torch.cuda.synchronize()
        nb = max(1, min(args.steps, 3))
        t0 = time.perf_counter()
        for _ in range(nb):
            step()
        torch.cuda.synchronize()
        wall_b = time.perf_counter() - t0
        out["bounded_memory"] = {
            "value": E * nb / wall_b, "unit": "edges/s", "ms_per_step": wall_b * 1e3 / nb, "steps": nb,
            "workspace_cap_GiB": args.bounded_gib, "workspace_GiB": ws.numel() / 2**30, "edge_chunk": ce,
            "peak_device_memory_GiB": torch.cuda.max_memory_allocated() / 2**30,
            "note": "same step, workspace for edge chunks within the cap; forward state and backward "
                    "cotangents kept as in the main line"}
        progress(f"bounded memory: {wall_b * 1e3 / nb:.1f} ms/step, chunk {ce} edges, peak "
                 f"{out['bounded_memory']['peak_device_memory_GiB']:.1f} GiB")
    if args.cpu_edges > 0:
        out["cpu_baseline"] = cpu_baseline_mole(d, mix_in, args.cpu_edges) if mole else \
            cpu_baseline(d, args.cpu_edges, dbwd=not two_stage)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
