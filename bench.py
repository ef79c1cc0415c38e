#!/usr/bin/env python3
"""Throughput of the chunkwise gated-delta-rule forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one gdn_chunk_fwd call (every kernel of the forward) over one batch
of synthetic inputs already resident in device memory, with L2 and the
Infinity Cache evicted before it (median of K such calls; back-to-back
"warm" calls are reported beside it).  Default workload: B=1, T=4096, H=16,
dk=dv=128, chunk 64, bf16 inputs, fp32 state.  Prints ONE JSON line with
tokens/s, the roofline position of the forward call (its algorithmic bytes
over the summed per-kernel device time from HIP events recorded by the
library on the launch stream) and the fp64 CPU oracle timed on this host's
cores as a baseline.

Other entry points (same JSON shape, their own metric string):
    --mode bwd      gdn_chunk_bwd alone      (default workload varlen_16k_dv256)
    --mode fwdbwd   forward + backward       (tokens / (t_fwd + t_bwd))
    --mode decode   gdn_decode_step in place (default workload decode_n256_h32)
    --mode product  gdn_chunk_fwd_product (Householder products, --nh steps)
    --mode tree     gdn_tree_verify + gdn_tree_commit (one speculative round)
    --mode decode_product  gdn_decode_step_product (--nh steps per token)
    --qk-l2norm     (forward) gdn_chunk_fwd_qknorm on q, k rows that are not
                    unit vectors (log-uniform row scales in [0.05, 20])
    --conv W        (forward) gdn_chunk_fwd_conv, short convolution of width W:
                    the workload's q, k, v are the projections

Algorithmic work per (token, head), chunk C:
    flops = 6 dk dv + C (3 dk + 2 dv) + C^2 / 3
    bytes = (2 dk + 2 dv) s_io + s_beta + s_gate      (+ state once per chain)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
PROFILES = os.path.join(ROOT, "profiles")


def algorithmic(B, T, H, dk, dv, C, s_io, s_gate, gate, nseq, s0, sfinal):
    th = B * T * H
    flops = th * (6 * dk * dv + C * (3 * dk + 2 * dv) + C * C / 3.0)
    gate_bytes = 0 if gate == "none" else (dk if gate == "channel" else 1) * s_gate
    byts = th * ((2 * dk + 2 * dv) * s_io + s_gate + gate_bytes)
    byts += nseq * H * dk * dv * 4 * ((1 if s0 else 0) + (1 if sfinal else 0))
    return flops, byts


def source_hash(files):
    """Hash of the kernel sources with // comments and blank lines removed,
    so a counter summary stays valid across comment-only edits."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


FWD_SOURCES = ["gated_delta_rule_79_amd/csrc/gdn_fwd.hip",
               "gated_delta_rule_79_amd/csrc/gdn_fwd_kernels.hpp",
               "gated_delta_rule_79_amd/csrc/gdn_chunk_common.hpp",
               "gated_delta_rule_79_amd/csrc/gdn_device.hpp"]
DECODE_SOURCES = ["gated_delta_rule_79_amd/csrc/gdn_decode.hip",
                  "gated_delta_rule_79_amd/csrc/gdn_device.hpp"]


def measured_traffic(workload, kernel, src_hash):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != src_hash:
        return None
    return d.get("bytes_per_launch")


def bwd_algorithmic(B, T, H, dk, dv, C, s_io, s_gate, gate, nseq):
    """Backward: flops = 2 x forward (matmul-backward convention, recompute not
    counted); bytes = read q, k, v, dO, beta, log-alpha, write dq, dk, dv and
    fp32 dbeta, dlog-alpha."""
    f_flops, _ = algorithmic(B, T, H, dk, dv, C, s_io, s_gate, gate, nseq, False, False)
    th = B * T * H
    gl = 0 if gate == "none" else (dk if gate == "channel" else 1)
    byts = th * ((2 * dk + 2 * dv) * s_io + dv * s_io + s_gate + gl * s_gate)  # reads
    byts += th * ((2 * dk + dv) * s_io + 4 + gl * 4)                          # writes
    return 2 * f_flops, byts


def decode_bytes(N, H, dk, dv, s_io):
    """Per step: fp32 state read and written once, q, k, v read, o written, and
    beta, log-alpha (fp32 or bf16; counted as 8 bytes)."""
    return N * H * (8 * dk * dv + (2 * dk + 2 * dv) * s_io + 8)


def host_cpu(max_workers=16):
    """Worker processes the CPU baseline may use (the cores this process may
    run on, at most ``max_workers``: the host's share for one GPU) and the
    CPU model string."""
    P = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return max(1, min(P, max_workers)), model


_ORACLE_JOB = None


def _oracle_unit(u):
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t = time.perf_counter()
        _ORACLE_JOB(u)
        return time.perf_counter() - t


def cpu_oracle_rate(job, units, work_per_unit, budget_s, what, unit="tokens/s"):
    """The oracle as it stands, run as ``job(u)`` over independent units
    (whole (sequence, head) chains, decode rows, trees) by P forked worker
    processes with one BLAS thread each; rounds over all units repeat until
    about ``budget_s`` seconds of wall clock.  Timed: the compute only (the
    pool is started and warmed first).  Call before the GPU is touched, so
    the workers hold no GPU state.  Returns the cpu_baseline record."""
    global _ORACLE_JOB
    import multiprocessing as mp
    units = list(units)
    P, model = host_cpu()
    P = min(P, len(units))
    _ORACLE_JOB = job
    try:
        with mp.get_context("fork").Pool(P) as pool:
            pool.map(_oracle_unit, units[:P], chunksize=1)        # warm the workers
            rounds, work, serial = 0, 0.0, 0.0
            t0 = time.perf_counter()
            while True:
                per = pool.map(_oracle_unit, units, chunksize=1)
                rounds += 1
                serial += sum(per)
                work += sum(work_per_unit(u) for u in units)
                if time.perf_counter() - t0 > budget_s:
                    break
            dt = time.perf_counter() - t0
    finally:
        _ORACLE_JOB = None
    return {"value": work / dt, "unit": unit, "cores": P, "kind": "oracle",
            "cpu_model": model,
            "single_worker_value": work / serial,
            "sample": f"{what}: {len(units)} units x {rounds} round(s) in {dt:.1f} s on "
                      f"{P} worker processes (one thread each) of {model}"}


def _chains(inp):
    """(batch row, first token, end token, state index) of every sequence."""
    B, T = inp.q.shape[:2]
    if inp.cu_seqlens is None:
        return [(b, 0, T, b) for b in range(B)]
    cu = inp.cu_seqlens.numpy()
    return [(0, int(cu[n]), int(cu[n + 1]), n) for n in range(len(cu) - 1)]


def cpu_baseline_bwd(inp, budget_s):
    """The oracle's adjoint on whole (sequence, head) chains of the workload
    (P workers); tokens/s of the whole workload."""
    import numpy as np
    import oracle
    f = inp.f64
    H, dk, dv = f["q"].shape[2], f["q"].shape[3], f["v"].shape[3]
    units = [(c, h) for c in _chains(inp) for h in range(H)]

    def job(u):
        (b, a, e, n), h = u
        sl = lambda x: None if x is None else x[b, a:e, h]
        m0 = np.zeros((dk, dv)) if f["s0"] is None else f["s0"][n, h]
        dm = None if f["ds_final"] is None else f["ds_final"][n, h]
        oracle.gdn_bwd_chain(sl(f["q"]), sl(f["k"]), sl(f["v"]), sl(f["beta"]),
                             sl(f["log_alpha"]), m0, sl(f["do"]), dm, inp.gate)

    return cpu_oracle_rate(job, units, lambda u: (u[0][2] - u[0][1]) / H, budget_s,
                           "oracle adjoint (backward) over every (sequence, head) chain")

def cpu_baseline_decode(inp, budget_s):
    """The oracle's decode step on every sequence (all heads per unit), P
    workers; tokens/s of the whole batch (one token per sequence)."""
    import oracle
    f = inp.f64
    N = f["q"].shape[0]

    def job(n):
        la = None if f["log_alpha"] is None else f["log_alpha"][n:n + 1, 0]
        oracle.gdn_decode(f["q"][n:n + 1, 0], f["k"][n:n + 1, 0], f["v"][n:n + 1, 0],
                          f["beta"][n:n + 1, 0], la, f["s0"][n:n + 1], inp.gate)

    return cpu_oracle_rate(job, range(N), lambda n: 1.0, budget_s,
                           "oracle decode step, one unit per sequence (all heads)")

def time_calls(fn, steps, warmup, cold_steps=0):
    """Median-free K-call timing with events on the current stream, plus an
    optional cold median (1 GiB write before each call)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        fn()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    cold = None
    if cold_steps > 0:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        times = []
        for _ in range(cold_steps):
            flush.fill_(1)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        times.sort()
        cold = times[len(times) // 2]
        del flush
    return ms, cold


def stage_pass(fn, steps):
    import torch
    import gated_delta_rule_79_amd as gdn
    gdn.stage_times(True)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    st = gdn.stage_times()
    gdn.stage_times(False)
    return {k: v[0] / v[1] for k, v in st.items()}


def product_algorithmic(B, T, H, dk, dv, C, nh, s_io):
    """Householder-product forward: nh steps per token.  Flops: per step the
    state products (4 dk dv) and the intra-chunk terms of the forward count,
    per token the output read 2 dk dv; bytes: q, o per token, k, v, beta
    per step, the gate per token and the fp32 final state."""
    th, sh = B * T * H, B * T * nh * H
    flops = sh * (4 * dk * dv + C * (3 * dk + 2 * dv) + C * C / 3.0) + th * 2 * dk * dv
    byts = (th * (dk + dv) * s_io + sh * (dk + dv) * s_io + sh * s_io + th * s_io
            + B * H * dk * dv * 4)
    return flops, byts


def cpu_baseline_product(inp, budget_s):
    """The fp64 oracle of the Householder-product forward on every
    (sequence, head) chain, P workers; tokens/s of the whole workload."""
    import oracle
    f = inp.f64
    B, T, H = f["q"].shape[:3]
    units = [(b, h) for b in range(B) for h in range(H)]

    def job(u):
        b, h = u
        bs, sl = slice(b, b + 1), slice(h, h + 1)
        la = None if f["log_alpha"] is None else f["log_alpha"][bs, :, sl]
        oracle.deltaproduct_fwd(f["q"][bs, :, sl], f["k"][bs, :, :, sl], f["v"][bs, :, :, sl],
                                f["beta"][bs, :, :, sl], la, None, inp.gate)

    return cpu_oracle_rate(job, units, lambda u: T / H, budget_s,
                           f"oracle Householder-product forward ({inp.k.shape[2]} steps per "
                           "token) over every (sequence, head) chain")

def main_product(args):
    """Householder-product forward (gdn_chunk_fwd_product) on B1 T4096 H16
    d128 bf16 with nh steps per token."""
    import torch
    import gated_delta_rule_79_amd as gdn
    from gated_delta_rule_79_amd import synth
    if torch.cuda.device_count() < 1:   # counts devices without initialising HIP
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    B, T, H, dk, dv, C, nh = 1, 4096, 16, 128, 128, 64, args.nh
    wl = f"product_t{T}_h{H}_nh{nh}"
    inp = synth.make_product_inputs(B, T, H, dk, dv, nh, dtype=torch.bfloat16,
                                    gate="scalar", chunk=C, seed=1006)
    cpu = None if args.no_cpu_baseline else cpu_baseline_product(inp, args.cpu_budget)
    d = inp.to("cuda")
    fn = lambda: gdn.chunk_fwd_product(d.q, d.k, d.v, d.beta, d.log_alpha, None, chunk=C)
    ms, cold = time_calls(fn, args.steps, args.warmup, args.cold_steps)
    per = stage_pass(fn, args.steps)
    flops, byts = product_algorithmic(B, T, H, dk, dv, C, nh, 2)
    dom = max(per, key=per.get)
    kernel = {"fwd_prep": "fwd_prep_sg_kernel", "fwd_scan": "fwd_scan_kernel",
              "fwd_trans": "fwd_trans_kernel", "fwd_combine": "fwd_combine_kernel",
              "chunk_map": "chunk_map_kernel"}.get(dom, dom)
    out = {
        "metric": f"tokens/sec gdn_chunk_fwd_product (T={T},H={H},d={dk},nh={nh} bf16); "
                  "% HBM roofline",
        "value": round(B * T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "cold_ms_per_step": None if cold is None else round(cold, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl, "B": B, "T": T, "H": H, "dk": dk, "dv": dv, "chunk": C,
                   "nh": nh, "gate": "scalar", "state": "fp32", "parallelism": "single GPU"},
        "roofline": {"bound": "hbm",
                     "achieved": round(byts / (per[dom] * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(byts / (per[dom] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None, "kernel": kernel,
                     "kernel_ms": {k: round(v, 5) for k, v in per.items()},
                     "alg_bytes_per_launch": int(byts), "alg_flops_per_launch": int(flops),
                     "path_frac_hbm": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "path_frac_mfma_bf16": round(flops / (ms * 1e-3) / 1e12 /
                                                  MFMA_BF16_PEAK_TFLOPS, 4)},
    }
    if cpu is not None:
        cpu["value"] = round(cpu["value"], 1)
    out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


def tree_depths(parent, n):
    """Root-path length of every node of dense trees parent [B, n]."""
    B = parent.shape[0]
    depth = [[0] * n for _ in range(B)]
    for b in range(B):
        for i in range(n):
            p = int(parent[b, i])
            depth[b][i] = 1 + (depth[b][p] if p >= 0 else 0)
    return depth


def tree_algorithmic(N, n, H, dk, dv, s_io, s_gate, path_nodes):
    """One speculative round over N trees of n nodes: verification reads the
    committed state once and every node's q, k, v, beta, log alpha and writes
    its output; the commit reads and writes the state once and reads k, v,
    beta, log alpha of the accepted paths' nodes.  Flops: the chunk form per
    node (the forward's count at chunk n) and 6 dk dv per committed step."""
    state = N * H * dk * dv * 4
    nodes = N * n * H
    v_bytes = state + nodes * ((2 * dk + 2 * dv) * s_io + 2 * s_gate)
    c_bytes = 2 * state + path_nodes * H * ((dk + dv) * s_io + 2 * s_gate)
    v_flops = nodes * (6 * dk * dv + n * (3 * dk + 2 * dv) + n * n / 3.0)
    c_flops = path_nodes * H * 6 * dk * dv
    return v_bytes, c_bytes, v_flops, c_flops


def cpu_baseline_tree(inp, parent, accepted, budget_s):
    """The fp64 oracle's verification and commit on every tree (all heads per
    unit), P workers; nodes/s."""
    import oracle
    f = inp.f64
    N, n = f["q"].shape[:2]
    par, acc = parent.numpy(), accepted.numpy()

    def job(m):
        sl = slice(m, m + 1)
        la = None if f["log_alpha"] is None else f["log_alpha"][sl]
        oracle.tree_fwd(f["q"][sl], f["k"][sl], f["v"][sl], f["beta"][sl], la,
                        par[sl], f["s0"][sl], inp.gate)
        oracle.tree_commit(f["k"][sl], f["v"][sl], f["beta"][sl], la, par[sl], acc[sl],
                           f["s0"][sl], inp.gate)

    return cpu_oracle_rate(job, range(N), lambda m: float(n), budget_s,
                           f"oracle verification and commit of every tree of {n} nodes",
                           unit="nodes/s")

def main_tree(args):
    """Speculative round on draft trees: gdn_tree_verify then gdn_tree_commit
    on 256 trees of 16 nodes, H32, d128, bf16 (the decode batch with a
    16-node draft tree per sequence)."""
    import torch
    import gated_delta_rule_79_amd as gdn
    from gated_delta_rule_79_amd import synth
    if torch.cuda.device_count() < 1:   # counts devices without initialising HIP
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    N, n, H, dk, dv = 256, 16, 32, 128, 128
    wl = f"tree_n{N}_h{H}_w{n}"
    inp, parent, accepted = synth.make_tree_inputs(N, n, H, dk, dv, dtype=torch.bfloat16,
                                                   gate="scalar", chunk=n, seed=1007,
                                                   s0_std=0.02)
    cpu = None if args.no_cpu_baseline else cpu_baseline_tree(inp, parent, accepted,
                                                              args.cpu_budget)
    d = inp.to("cuda")
    par, acc = parent.cuda(), accepted.cuda()
    state = d.s0.clone()
    ws = torch.empty(max(1, gdn.tree_verify_workspace(d.q, d.v, d.beta, d.log_alpha, chunk=n)),
                     dtype=torch.uint8, device="cuda")

    def fn():
        gdn.tree_verify(d.q, d.k, d.v, d.beta, d.log_alpha, par, state, chunk=n, workspace=ws)
        gdn.tree_commit(d.k, d.v, d.beta, d.log_alpha, par, acc, state, chunk=n)

    ms, cold = time_calls(fn, args.steps, args.warmup, args.cold_steps)
    per = stage_pass(fn, args.steps)
    depth = tree_depths(parent, n)
    path_nodes = sum(depth[m][int(accepted[m])] for m in range(N))
    vb, cb, vf, cf = tree_algorithmic(N, n, H, dk, dv, 2, 2, path_nodes)
    names = {"fwd_prep": "fwd_prep_sg_kernel", "fwd_scan": "fwd_scan_kernel",
             "tree_commit": "tree_commit_kernel"}
    # the kernels' own algorithmic bytes: the commit's state stream; the
    # scan reads the state, q and writes o; the prep reads k, v, beta, alpha
    own = {"tree_commit": cb,
           "fwd_scan": N * H * dk * dv * 4 + N * n * H * (dk + dv) * 2,
           "fwd_prep": N * n * H * ((dk + dv) * 2 + 4)}
    dom = max(per, key=per.get)
    ach = own[dom] / (per[dom] * 1e-3) / 1e9
    out = {
        "metric": f"nodes/sec gdn_tree_verify + gdn_tree_commit (N={N},n={n},H={H},d={dk} "
                  "bf16); % HBM roofline",
        "value": round(N * n / (ms * 1e-3), 1), "unit": "nodes/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "cold_ms_per_step": None if cold is None else round(cold, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl, "trees": N, "nodes": n, "H": H, "dk": dk, "dv": dv,
                   "chunk": n, "gate": "scalar", "accepted_path_nodes": path_nodes,
                   "state": "fp32", "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": names.get(dom, dom),
                     "kernel_ms": {k: round(v, 5) for k, v in per.items()},
                     "alg_bytes_per_launch": int(own[dom]),
                     "alg_bytes_per_step": int(vb + cb), "alg_flops_per_step": int(vf + cf),
                     "path_frac_hbm": round((vb + cb) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    if cpu is not None:
        cpu["value"] = round(cpu["value"], 1)
    out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


def main_decode_product(args):
    """Decode step with nh delta steps per token (gdn_decode_step_product) on
    the decode batch: N256 H32 d128 bf16, state fp32 in place."""
    import torch
    import gated_delta_rule_79_amd as gdn
    from gated_delta_rule_79_amd import synth
    if torch.cuda.device_count() < 1:   # counts devices without initialising HIP
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    N, H, dk, dv, nh = 256, 32, 128, 128, args.nh
    wl = f"decode_product_n{N}_h{H}_nh{nh}"
    inp = synth.make_product_inputs(N, 1, H, dk, dv, nh, dtype=torch.bfloat16,
                                    gate="scalar", chunk=16, seed=1008, s0_std=0.02)
    d = inp.to("cuda")
    q, k, v = d.q[:, 0].contiguous(), d.k[:, 0].contiguous(), d.v[:, 0].contiguous()
    beta, la = d.beta[:, 0].contiguous(), d.log_alpha[:, 0].contiguous()
    state = d.s0.clone()
    fn = lambda: gdn.decode_step_product(q, k, v, beta, la, state)
    ms, cold = time_calls(fn, args.steps, args.warmup, args.cold_steps)
    per = stage_pass(fn, args.steps)
    kms = per.get("decode", ms)
    # state read + written (fp32), q, o, and per step k, v, beta; the gate
    byts = N * H * (8 * dk * dv + (dk + dv) * 2 + nh * ((dk + dv) * 2 + 2) + 2)
    gbs = byts / (kms * 1e-3) / 1e9
    out = {
        "metric": f"tokens/sec gdn_decode_step_product (N={N},H={H},d={dk},nh={nh}); % HBM",
        "value": round(N / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "cold_ms_per_step": None if cold is None else round(cold, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl, "N": N, "H": H, "dk": dk, "dv": dv, "nh": nh,
                   "gate": "scalar", "state": "fp32", "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "decode_product_kernel",
                     "kernel_ms": {k2: round(v2, 5) for k2, v2 in per.items()},
                     "alg_bytes_per_launch": int(byts)},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def main_other(args):
    """bwd, fwdbwd and decode modes."""
    import torch
    import gated_delta_rule_79_amd as gdn
    from gated_delta_rule_79_amd import synth
    if torch.cuda.device_count() < 1:   # counts devices without initialising HIP
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    wl = args.workload or ("decode_n256_h32" if args.mode == "decode" else "varlen_16k_dv256")
    inp = synth.workload(wl, with_do=args.mode != "decode")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = (cpu_baseline_decode(inp, args.cpu_budget) if args.mode == "decode"
               else cpu_baseline_bwd(inp, args.cpu_budget))
    d = inp.to("cuda")
    B, T, H, dk = inp.q.shape
    dv = inp.v.shape[-1]
    C = inp.chunk
    s_io = 2 if inp.q.dtype == torch.bfloat16 else 4
    s_gate = 2 if inp.beta.dtype == torch.bfloat16 else 4
    nseq = B if inp.cu_seqlens is None else inp.cu_seqlens.numel() - 1
    cfg = {"workload": wl, "B": B, "T": T, "H": H, "dk": dk, "dv": dv, "chunk": C,
           "gate": inp.gate, "seed": inp.seed, "state": "fp32", "parallelism": "single GPU"}
    out = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if s_io == 2 else "f32",
           "data": "synthetic", "config": cfg}
    if args.mode == "decode":
        q, k, v = d.q[:, 0], d.k[:, 0], d.v[:, 0]
        beta = d.beta[:, 0]
        la = None if d.log_alpha is None else d.log_alpha[:, 0]
        state = d.s0.clone()
        fn = lambda: gdn.decode_step(q, k, v, beta, la, state)
        ms, cold = time_calls(fn, args.steps, args.warmup, args.cold_steps)
        per = stage_pass(fn, args.steps)
        kms = per.get("decode", ms)
        byts = decode_bytes(B, H, dk, dv, s_io)
        gbs = byts / (kms * 1e-3) / 1e9
        copy_gbs = copy_bandwidth()
        out.update({"metric": "tokens/sec gdn_decode_step (N=%d,H=%d,d=%d); %% HBM" % (B, H, dk),
                    "value": round(B / (ms * 1e-3), 1), "unit": "tokens/s",
                    "ms_per_step": round(ms, 5),
                    "cold_ms_per_step": None if cold is None else round(cold, 5),
                    "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                 "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                 "traffic": measured_traffic(
                                     wl, "decode_kernel", source_hash(DECODE_SOURCES)),
                                 "kernel": "decode_kernel",
                                 "kernel_ms": {k2: round(v2, 5) for k2, v2 in per.items()},
                                 "alg_bytes_per_launch": int(byts),
                                 "copy_GBps_measured": round(copy_gbs, 1),
                                 "frac_of_copy": round(gbs / copy_gbs, 4)}})
    else:
        plan = gdn.FwdPlan(d.q, d.k, d.v, d.beta, d.log_alpha, d.s0, chunk=C,
                           cu_seqlens=d.cu_seqlens)
        bwd = lambda: gdn.chunk_bwd(d.q, d.k, d.v, d.beta, d.log_alpha, d.s0, d.do,
                                    d.ds_final, chunk=C, cu_seqlens=d.cu_seqlens,
                                    need_ds0=d.s0 is not None)
        ms_b, cold_b = time_calls(bwd, args.steps, args.warmup, args.cold_steps)
        per = stage_pass(bwd, args.steps)
        bflops, bbytes = bwd_algorithmic(B, T, H, dk, dv, C, s_io, s_gate, inp.gate, nseq)
        tokens = B * T
        rf = {"bound": "mfma", "achieved": round(bflops / (ms_b * 1e-3) / 1e12, 2),
              "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
              "frac": round(bflops / (ms_b * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
              "traffic": None, "kernel": "gdn_chunk_bwd (all stages)",
              "kernel_ms": {k2: round(v2, 5) for k2, v2 in per.items()},
              "alg_flops_per_launch": int(bflops), "alg_bytes_per_launch": int(bbytes),
              "path_frac_hbm": round(bbytes / (ms_b * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if args.mode == "bwd":
            out.update({"metric": "tokens/sec gdn_chunk_bwd (%s); %% MFMA/HBM roofline" % wl,
                        "value": round(tokens / (ms_b * 1e-3), 1), "unit": "tokens/s",
                        "ms_per_step": round(ms_b, 5),
                        "cold_ms_per_step": None if cold_b is None else round(cold_b, 5),
                        "roofline": rf})
        else:
            ms_f, cold_f = time_calls(plan.run, args.steps, args.warmup, args.cold_steps)
            fflops, fbytes = algorithmic(B, T, H, dk, dv, C, s_io, s_gate, inp.gate, nseq,
                                         inp.s0 is not None, True)
            ms = ms_f + ms_b
            rf.update({"kernel": "gdn_chunk_fwd + gdn_chunk_bwd", "fwd_ms": round(ms_f, 5),
                       "bwd_ms": round(ms_b, 5),
                       "achieved": round((fflops + bflops) / (ms * 1e-3) / 1e12, 2),
                       "frac": round((fflops + bflops) / (ms * 1e-3) / 1e12 /
                                     MFMA_BF16_PEAK_TFLOPS, 4),
                       "alg_flops_per_launch": int(fflops + bflops),
                       "alg_bytes_per_launch": int(fbytes + bbytes),
                       "path_frac_hbm": round((fbytes + bbytes) / (ms * 1e-3) / 1e9 /
                                              HBM_PEAK_GBS, 4)})
            out.update({"metric": "tokens/sec gdn_chunk_fwd+bwd (%s); %% MFMA/HBM roofline" % wl,
                        "value": round(tokens / (ms * 1e-3), 1), "unit": "tokens/s",
                        "ms_per_step": round(ms, 5), "cold_ms_per_step": None,
                        "roofline": rf})
    if args.copy_calibration:
        copy_calibration()
    if cpu is not None:
        cpu["value"] = round(cpu["value"], 1)
    out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


def cache_evictor(nbytes=1 << 30):
    """A function that reads a 1 GiB device buffer: it evicts the inputs and
    the workspace of the previous call from L2 (4 MB per XCD) and the 256 MB
    Infinity Cache, leaving clean lines (a write would leave 256 MB of dirty
    lines whose write-back the next call would pay for)."""
    import torch
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")

    def evict():
        buf.max()
    return evict


def copy_calibration():
    """Device copies of known traffic for scaling memory counters: three of
    256 MiB (inside the 256 MB Infinity Cache) and three of 1 GiB (beyond
    it)."""
    import torch
    for n in (1 << 28, 1 << 30):
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(3)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst


def copy_bandwidth(nbytes=1 << 30, reps=10):
    """GB/s of the runtime's device-to-device copy of ``nbytes`` (read +
    written bytes over the median duration): the practical streaming
    ceiling of this GPU, measured in the same process."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(3)
    dst = torch.empty_like(src)
    dst.copy_(src)
    times = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    times.sort()
    del src, dst
    return 2 * nbytes / (times[len(times) // 2] * 1e-3) / 1e9


def cpu_baseline(inp, budget_s, qknorm=False, taps=None):
    """The fp64 oracle, as it stands, on every (sequence, head) chain of the
    workload, P workers; tokens/s of the whole workload.  qknorm: q and k rows
    go through the oracle's L2 normalisation first (timed); taps (wq, wk, wv,
    numpy fp64 [H, d, W]): q, k, v go through the oracle's convolution
    prologue first (timed)."""
    import numpy as np
    import oracle
    f = inp.f64
    H, dk, dv = f["q"].shape[2], f["q"].shape[3], f["v"].shape[3]
    units = [(c, h) for c in _chains(inp) for h in range(H)]

    def job(u):
        (b, a, e, n), h = u
        la = None if f["log_alpha"] is None else f["log_alpha"][b, a:e, h]
        m0 = np.zeros((dk, dv)) if f["s0"] is None else f["s0"][n, h]
        qc, kc, vc = f["q"][b, a:e, h], f["k"][b, a:e, h], f["v"][b, a:e, h]
        if qknorm:
            qc, kc = oracle.l2_normalize(qc), oracle.l2_normalize(kc)
        if taps is not None:   # one chain as a [1, len, 1, d] batch
            pro = lambda x, w, nz: oracle.conv_prologue(x[None, :, None], w[h][None], nz)[0, :, 0]
            qc, kc, vc = pro(qc, taps[0], True), pro(kc, taps[1], True), pro(vc, taps[2], False)
        oracle.gdn_fwd_chain(qc, kc, vc, f["beta"][b, a:e, h], la, m0, inp.gate)

    return cpu_oracle_rate(job, units, lambda u: (u[0][2] - u[0][1]) / H, budget_s,
                           "oracle token recurrence over every (sequence, head) chain")

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None,
                    help="synthetic workload (default: fwd_t4096_h16 for the forward)")
    ap.add_argument("--mode", default="fwd",
                    choices=("fwd", "bwd", "fwdbwd", "decode", "product", "tree",
                             "decode_product"))
    ap.add_argument("--nh", type=int, default=2,
                    help="delta steps per token for --mode product")
    ap.add_argument("--qk-l2norm", action="store_true",
                    help="forward with q and k L2-normalised inside the kernels")
    ap.add_argument("--conv", type=int, default=0,
                    help="(forward) gdn_chunk_fwd_conv with this short-convolution width: "
                         "the workload's q, k, v are the projections")
    ap.add_argument("--batch", type=int, default=0,
                    help="(forward) override the workload's batch size B")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="extra calls each preceded by a 1 GiB cache-flush write")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run device copies of 256 MiB and 1 GiB (kernels of known "
                         "traffic for scaling memory counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the gated delta rule path here runs on a "
              "single MI355X (heads and sequences shard with no communication; see "
              "the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.mode == "product":
        main_product(args)
        return
    if args.mode == "tree":
        main_tree(args)
        return
    if args.mode == "decode_product":
        main_decode_product(args)
        return
    if args.mode != "fwd":
        main_other(args)
        return
    if args.workload is None:
        args.workload = "fwd_t4096_h16"
    main_fwd(args)


def main_fwd(args):
    """The headline: gdn_chunk_fwd on B=1, T=4096, H=16, dk=dv=128, chunk 64,
    bf16 inputs, fp32 state (``--batch`` overrides B for the batch sweep).

    Timed region: K steps, each a 1 GiB read that evicts L2 and the 256 MB
    Infinity Cache (outside the events) followed by one forward call
    bracketed by HIP events on the call's stream; ``value`` is tokens over
    the median call.  The same K steps then run again with the library's
    per-kernel HIP events (kept out of the timed region: an event between
    kernels costs a few microseconds).  Back-to-back (warm) calls are timed
    last and reported as extra keys."""
    import torch
    import gated_delta_rule_79_amd as gdn
    from gated_delta_rule_79_amd import synth

    if torch.cuda.device_count() < 1:   # counts devices without initialising HIP
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    qkn = args.qk_l2norm
    over = {"raw_qk": (0.05, 20.0, 0.0)} if qkn else {}
    if args.batch:
        over["B"] = args.batch
    inp = synth.workload(args.workload, **over)
    B, T, H, dk = inp.q.shape
    dv = inp.v.shape[-1]
    C = inp.chunk
    nseq = B if inp.cu_seqlens is None else inp.cu_seqlens.numel() - 1
    wl = (args.workload + (f"_b{B}" if args.batch else "") + ("_qknorm" if qkn else "") +
          (f"_conv{args.conv}" if args.conv else ""))
    taps = synth.conv_taps(H, dk, dv, args.conv, inp.seed) if args.conv else None
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_budget, qknorm=qkn,
                           taps=None if taps is None else [t.double().numpy() for t in taps])
        cpu["value"] = round(cpu["value"], 1)
        cpu["single_worker_value"] = round(cpu["single_worker_value"], 1)

    d = inp.to("cuda")
    plan = gdn.FwdPlan(d.q, d.k, d.v, d.beta, d.log_alpha, d.s0, chunk=C,
                       cu_seqlens=d.cu_seqlens, qk_l2norm=qkn,
                       conv_taps=None if taps is None else [t.cuda() for t in taps])
    evict = cache_evictor()
    for _ in range(args.warmup):
        evict()
        plan.run()
    torch.cuda.synchronize()

    def cold_region(stages):
        """K steps: evict the caches, then one call between two events."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        if stages:
            gdn.stage_times(True)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for a, b in ev:
            evict()
            a.record()
            plan.run()
            b.record()
        torch.cuda.synchronize()
        t = time.perf_counter() - t
        st = None
        if stages:
            st = gdn.stage_times()
            gdn.stage_times(False)
        return sorted(a.elapsed_time(b) for a, b in ev), t, st

    # the timed region, then the same steps again with the library's HIP
    # events around every kernel (the per-kernel durations)
    times, t_host, _ = cold_region(False)
    cold_ms = times[len(times) // 2]
    _, _, st = cold_region(True)
    per_kernel = {k: v[0] / v[1] for k, v in st.items()}

    # warm: back-to-back calls, inputs and workspace resident in the caches
    warm_ms, _ = time_calls(plan.run, args.steps, 0)
    del evict

    if args.copy_calibration:
        copy_calibration()

    s_io = 2 if inp.q.dtype == torch.bfloat16 else 4
    s_gate = 2 if inp.beta.dtype == torch.bfloat16 else 4
    flops, byts = algorithmic(B, T, H, dk, dv, C, s_io, s_gate, inp.gate, nseq,
                              inp.s0 is not None, True)
    tokens = B * T
    path_ms = sum(per_kernel.values())
    prep_kernel = "fwd_prep_kernel" if inp.gate == "channel" else "fwd_prep_sg_kernel"
    names = {"fwd_prep": prep_kernel, "fwd_scan": "fwd_scan_kernel",
             "fwd_trans": "fwd_trans_kernel", "fwd_combine": "fwd_combine_kernel",
             "chunk_map": "chunk_map_kernel", "prologue": "prologue_kernel"}
    dom = max(per_kernel, key=per_kernel.get)
    src_hash = source_hash(FWD_SOURCES)
    traffic = None if (qkn or args.conv) else measured_traffic(wl, "fwd_call", src_hash)
    achieved = byts / (cold_ms * 1e-3) / 1e9
    roofline = {
        # the forward call as one unit: its algorithmic bytes over the median
        # call duration of the timed region (the per-kernel durations below
        # come from the second pass, where the events between kernels add a
        # few microseconds each)
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "kernel": "gdn_chunk_fwd (" + " + ".join(names.get(k, k) for k in per_kernel) + ")",
        "kernel_ms": {names.get(k, k): round(v, 5) for k, v in per_kernel.items()},
        "call_kernel_ms": round(path_ms, 5),
        "alg_bytes_per_launch": int(byts),
        "alg_flops_per_launch": int(flops),
        "frac_mfma_bf16": round(flops / (cold_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "dominant_kernel": names.get(dom, dom),
        "dominant_kernel_frac_if_alone": round(byts / (per_kernel[dom] * 1e-3) / 1e9 /
                                               HBM_PEAK_GBS, 4),
        "source_hash": src_hash,
    }
    out = {
        "metric": (f"tokens/sec gdn_chunk_fwd_conv (T={T},H={H},d={dk},W={args.conv}); "
                   "% HBM roofline" if args.conv else
                   "tokens/sec gdn_chunk_fwd_qknorm (T=4096,H=16,d=128 bf16); % HBM roofline"
                   if qkn else
                   "tokens/sec gdn_chunk_fwd (T=4096,H=16,d=128 bf16); % MFMA/HBM roofline"),
        "value": round(tokens / (cold_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(cold_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s_io == 2 else "f32",
        "data": "synthetic",
        "config": {"workload": wl, "B": B, "T": T, "H": H, "dk": dk, "dv": dv, "chunk": C,
                   "gate": inp.gate, "seed": inp.seed, "state": "fp32",
                   "timing": "median of K calls, each after a 1 GiB read that evicts L2 "
                             "and the Infinity Cache",
                   "parallelism": "single GPU"},
        "p10_ms": round(times[len(times) // 10], 5),
        "p90_ms": round(times[(len(times) * 9) // 10], 5),
        "warm_ms_per_step": round(warm_ms, 5),
        "warm_value": round(tokens / (warm_ms * 1e-3), 1),
        "timed_region_host_s": round(t_host, 3),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
