#!/usr/bin/env python
"""Benchmark of the on-the-fly equivariant attention layer on one MI355X.

One step is one pass of the whole hot path over the 100k-atom system: the
cell-list neighbour build (e2a_build_neighbors) and the fused layer
(e2a_attention_fwd: q/k prologue, weight packing, fused MFMA kernel).  Inputs
are resident in device memory before timing starts.  The headline value is
neighbour edges per second of the whole step; the fused kernel's own time,
measured with HIP events on the stream it runs on, gives the roofline block.
The fp64 oracle is timed on the host's cores on a bounded sample of
destination atoms as the CPU baseline.  The convolution stage (e2a_conv_fwd,
the same messages summed without attention) is timed separately and reported
in the breakdown, and so are the gradients.

The line checks itself: "parity" compares the timed step's output with the
oracle on seeded destinations (plus the first, last, highest- and
lowest-degree atoms) and the GPU neighbour list with the oracle's, entry by
entry; "breakdown.configs" times the layer on the other four workloads (the
64-atom system, the drug-like batch, the water box, the solvated protein)
with the same checks.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "neighbour edges/sec per attention layer (1 MI355X); achieved TFLOPS % of roofline"
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_mfma_large_traffic.txt")
KERNEL_SRC = os.path.join(ROOT, "so_graph_attention_amd", "csrc", "attention_mfma.hip")


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def flops_per_edge(L, C):
    """Algorithmic work per edge: SO(2) mix 2[(L+1)^2 + 4 sum_{m>=1} (L+1-m)^2] C^2,
    rotations in and out 4 sum_l (2l+1)^2 C, radial 2*8*(L+1) C, accumulate
    2 (L+1)^2 C, logits 2 C."""
    so2 = 2 * ((L + 1) ** 2 + 4 * sum((L + 1 - m) ** 2 for m in range(1, L + 1))) * C * C
    rot = 4 * sum((2 * l + 1) ** 2 for l in range(L + 1)) * C
    rad = 2 * 8 * (L + 1) * C
    accum = 2 * (L + 1) ** 2 * C
    return so2 + rot + rad + accum + 2 * C


def traffic_per_launch():
    """Measured HBM bytes per launch of the fused kernel from the committed
    rocprofv3 counter summary, or None when the kernel source changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        m = re.match(r"^\s*([a-z_]+)\s*:\s*(\S+)", line)
        if m:
            kv[m.group(1)] = m.group(2)
    import hashlib
    sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]
    if kv.get("kernel_source_sha") != sha or "hbm_bytes_per_launch" not in kv:
        return None
    return float(kv["hbm_bytes_per_launch"])


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, rp, col, seconds):
    """The oracle as it stands on a seeded sample of destination atoms, grown in
    batches of 32 until about `seconds` of CPU time have been spent."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    feat = w.as_f32("feat")
    args = (rp, col, feat, w.as_f32("w_q"), w.as_f32("w_k"), w.as_f32("w_rad"), w.as_f32("w_so2"),
            w.L, w.C, w.H, w.cutoff)
    order = np.random.default_rng(2024).permutation(w.n_atoms)
    done = 0
    edges = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds and done < w.n_atoms:
        dest = np.sort(order[done:done + 32])
        O.attention(w.pos, *args, box=w.box, dest=dest)
        edges += int((rp[dest + 1] - rp[dest]).sum())
        done += dest.size
    dt = time.perf_counter() - t0
    return {"value": edges / dt, "unit": "edges/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} seeded destination atoms ({edges} edges) of the same 100k-atom workload, "
                      f"{dt:.1f} s of fp64 NumPy on {threads} BLAS threads",
            "host": {"cpu_model": cpu_model(), "os_cpu_count": os.cpu_count()}}


def cpu_single_thread(name, seconds):
    """The oracle with one BLAS thread on a small workload (all of it, or a
    seeded sample of destinations grown in batches of 32 until about
    `seconds` have been spent)."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    from workloads import make_config
    w = make_config(name)
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    args = (rp, col, w.as_f32("feat"), w.as_f32("w_q"), w.as_f32("w_k"), w.as_f32("w_rad"), w.as_f32("w_so2"),
            w.L, w.C, w.H, w.cutoff)
    order = np.random.default_rng(2024).permutation(w.n_atoms)
    done = edges = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while done < w.n_atoms and (done == 0 or time.perf_counter() - t0 < seconds):
            dest = np.sort(order[done:done + 32])
            O.attention(w.pos, *args, box=w.box, dest=dest)
            edges += int((rp[dest + 1] - rp[dest]).sum())
            done += dest.size
        dt = time.perf_counter() - t0
    return {"workload": name, "value": edges / dt, "unit": "edges/s", "cores": 1,
            "sample": f"{done} of {w.n_atoms} destination atoms ({edges} edges), {dt:.1f} s"}


def backward_leg(B, torch, dev, w, pos, rp, col, feat, w_q, w_k, w_rad, w_so2, box):
    """The feature gradient (e2a_attention_bwd) on the same workload, from the
    forward's output and log-normaliser and a seeded cotangent; one warm-up
    and two timed calls with HIP events on the stream.  Algorithmic work: the
    message recomputed (query pass) plus its transpose (value pass), each the
    forward's per-edge work."""
    e = int(col.numel())
    out, lse = B.e2a_attention_fwd(pos, rp, col, feat, w_q, w_k, w_rad, w_so2, L=w.L, C=w.C, H=w.H,
                                   cutoff=w.cutoff, box=box, with_lse=True)
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    G = torch.randn(tuple(out.shape), generator=gen, device=dev, dtype=torch.float32)
    gfeat = torch.empty_like(out)
    ws = torch.empty(B.e2a_attention_bwd_workspace_bytes(w.n_atoms, e, w.L, w.C, w.H), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()

    def run():
        B.e2a_attention_bwd(pos, rp, col, feat, w_q, w_k, w_rad, w_so2, out, lse, G, L=w.L, C=w.C, H=w.H,
                            cutoff=w.cutoff, box=box, grad_feat=gfeat, workspace=ws)

    run()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(2):
        run()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / 2
    tflops = 2 * flops_per_edge(w.L, w.C) * e / (ms * 1e-3) / 1e12
    return {"backward_ms": ms, "backward_edges_per_s": e / (ms * 1e-3), "backward_tflops": tflops,
            "backward_frac_of_bf16_peak": tflops / PEAK_BF16_TFLOPS,
            "backward_kernels": "e2a_attention_bwd: delta, query pass, value pass (fused MFMA kernel modes), "
                                "l = 0 terms"}


def sample_dest(rp, n_sample, seed):
    """Seeded destinations plus the first, last, highest- and lowest-degree atoms."""
    n = rp.size - 1
    deg = np.diff(rp)
    pick = set(np.random.default_rng(seed).choice(n, size=min(n, n_sample), replace=False).tolist())
    pick |= {0, n - 1, int(np.argmax(deg)), int(np.argmin(deg))}
    return np.array(sorted(pick), dtype=np.int64)


def parity_check(w, rp_gpu, col_gpu, out, lse, n_sample=64, seed=11):
    """The GPU's neighbour list against the oracle's (bit for bit) and its
    output and log-normaliser against the oracle's on sampled destinations."""
    import oracle as O
    rp_o, col_o = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    exact = bool(np.array_equal(rp_gpu, rp_o) and np.array_equal(col_gpu, col_o))
    dest = sample_dest(rp_o, n_sample, seed) if n_sample < w.n_atoms else np.arange(w.n_atoms)
    want, want_lse = O.attention(w.pos, rp_o, col_o, w.as_f32("feat"), w.as_f32("w_q"), w.as_f32("w_k"),
                                 w.as_f32("w_rad"), w.as_f32("w_so2"), w.L, w.C, w.H, w.cutoff, box=w.box, dest=dest)
    got = out[dest].astype(np.float64)
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    fin = np.isfinite(want_lse)
    lse_err = float(np.max(np.abs(lse[dest][fin] - want_lse[fin]))) if fin.any() else 0.0
    tol = 2e-2 if w.dtype == "bf16" else 1e-5
    return {"rel_l2": rel, "tol": tol, "ok": bool(exact and rel <= tol), "n_dest": int(dest.size),
            "lse_max_abs_err": lse_err, "neighbours_bit_exact": exact,
            "sample": "all destinations" if dest.size == w.n_atoms else
                      f"{dest.size} destinations: {n_sample} seeded (seed {seed}) plus first, last, "
                      f"highest- and lowest-degree atoms"}


def config_leg(B, torch, dev, name, iters=10):
    """One more workload: the neighbour build and the layer, timed with HIP
    events (median over `iters` calls after warm-up), checked like the
    headline step."""
    from workloads import make_config
    w = make_config(name)
    box = None if w.box is None else w.box.tolist()

    def stored(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    pos = torch.from_numpy(w.pos).to(dev)
    batch = None if w.batch is None else torch.from_numpy(w.batch.astype(np.int32)).to(dev)
    feat, w_q, w_k, w_rad, w_so2 = (stored(getattr(w, n)) for n in ("feat", "w_q", "w_k", "w_rad", "w_so2"))
    stream = torch.cuda.current_stream()
    rp, col = B.e2a_build_neighbors(pos, w.cutoff, box=box, batch=batch)
    e = int(col.numel())
    dtype_code = B.E2A_DTYPE_BF16 if w.dtype == "bf16" else B.E2A_DTYPE_F32
    out = torch.empty((w.n_atoms, (w.L + 1) ** 2, w.C), dtype=torch.float32, device=dev)
    lse = torch.empty((w.n_atoms, w.H), dtype=torch.float32, device=dev)
    ws = torch.empty(B.e2a_attention_workspace_bytes(w.n_atoms, w.L, w.C, w.H, dtype_code), dtype=torch.uint8,
                     device=dev)

    def call():
        B.e2a_attention_fwd(pos, rp, col, feat, w_q, w_k, w_rad, w_so2, L=w.L, C=w.C, H=w.H, cutoff=w.cutoff,
                            box=box, out=out, out_lse=lse, workspace=ws)

    def nb():
        B.e2a_build_neighbors(pos, w.cutoff, box=box, batch=batch, capacity=e)

    for _ in range(3):
        call()
        nb()
    ts, tn = [], []
    for _ in range(iters):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        nb()
        ev[1].record(stream)
        call()
        ev[2].record(stream)
        torch.cuda.synchronize()
        tn.append(ev[0].elapsed_time(ev[1]))
        ts.append(ev[1].elapsed_time(ev[2]))
    ms = float(np.median(ts))
    f = flops_per_edge(w.L, w.C)
    tflops = f * e / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    res = {"workload": f"{name}: {w.n_atoms} atoms, "
                       + ("periodic box %.4g A" % w.box[0] if w.box is not None else "open boundaries")
                       + f", cutoff {w.cutoff:g} A, L={w.L}, C={w.C}, H={w.H}, {w.dtype} storage",
           "n_atoms": w.n_atoms, "n_edges": e, "neighbors_ms": float(np.median(tn)), "attention_ms": ms,
           "edges_per_s": e / (ms * 1e-3), "step_edges_per_s": e / ((ms + float(np.median(tn))) * 1e-3),
           "tflops": tflops, "peak": peak, "frac": tflops / peak,
           "kernel": "MFMA (bf16 operands)" if w.dtype == "bf16" else "scalar fp32 (VALU)"}
    res["parity"] = parity_check(w, rp.cpu().numpy(), col.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy())
    return res


def block_leg(B, torch, dev, w, pos, rp, col, box, attn_ms):
    """One block around the layer (e2a_block_fwd) and two stacked blocks on
    the same workload, each block with its own seeded weights: one warm-up
    and three timed calls, HIP events on the stream."""
    from workloads import make_block_weights
    h = torch.from_numpy(np.ascontiguousarray(w.as_f32("feat"))).to(dev)

    def dev_w(bw):
        out = {}
        for k, v in bw.items():
            if v.dtype == np.uint16:
                out[k] = torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).to(dev)
            else:
                out[k] = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(dev)
        return out

    bws = [dev_w(make_block_weights(w, i)) for i in range(2)]
    dtype_code = B.E2A_DTYPE_BF16 if w.dtype == "bf16" else B.E2A_DTYPE_F32
    ws = torch.empty(B.e2a_block_workspace_bytes(w.n_atoms, w.L, w.C, w.H, dtype_code), dtype=torch.uint8,
                     device=dev)
    x1 = torch.empty_like(h)
    x2 = torch.empty_like(h)
    stream = torch.cuda.current_stream()

    def one():
        B.e2a_block_fwd(pos, rp, col, h, bws[0], L=w.L, C=w.C, H=w.H, cutoff=w.cutoff, box=box, out=x1,
                        workspace=ws)

    def two():
        one()
        B.e2a_block_fwd(pos, rp, col, x1, bws[1], L=w.L, C=w.C, H=w.H, cutoff=w.cutoff, box=box, out=x2,
                        workspace=ws)

    res = {}
    for name, fn in (("block_ms", one), ("two_blocks_ms", two)):
        fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(3):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        res[name] = ev[0].elapsed_time(ev[1]) / 3
    res["block_nodewise_ms"] = res["block_ms"] - attn_ms
    if w.dtype == "bf16":
        # node-wise arrays once each, as the bf16 block moves them: Norm1 (h in
        # fp32, bf16 out), projection (layer output and h in, h1 out, fp32),
        # gate logits (h1's degree-0 rows in, z out), first FFN product (h1 and
        # z in, bf16 activations out), second (activations and h1 in, fp32 out)
        nkc = w.n_atoms * (w.L + 1) ** 2 * w.C
        nc = w.n_atoms * w.C
        alg = nkc * (6 + 12 + 6 + 10) + nc * (4 + 8 * w.L)
        res["block_nodewise_alg_bytes"] = alg
        res["block_nodewise_hbm_frac"] = alg / (res["block_nodewise_ms"] * 1e-3) / (PEAK_HBM_GBS * 1e9)
    res["block_finite"] = bool(torch.isfinite(x2).all())
    res["block_kernels"] = ("e2a_block_fwd: per-degree RMS norm, the fused layer, per-degree projection + residual "
                            "(bf16 MFMA GEMM), gated FFN (bf16 MFMA GEMMs with the second norm folded into the "
                            "products that read it and the gate into the first one's epilogue) + residual; "
                            "block_nodewise_ms is the block's time less the standalone layer call's")
    return res


def algorithmic_bytes(w, n_edges):
    """HBM bytes of one layer call with every array touched once: the node
    features (storage precision) in and the fp32 output out, the CSR graph,
    positions, q and k (fp32), and the weights."""
    s = 2 if w.dtype == "bf16" else 4
    n, K, C, L = w.n_atoms, (w.L + 1) ** 2, w.C, w.L
    so2 = sum((1 if m == 0 else 2) * ((L + 1 - m) * C) ** 2 for m in range(L + 1))
    weights = (so2 + 2 * C * C + 8 * (L + 1) * C) * s
    return n * K * C * (s + 4) + 4 * n_edges + 8 * (n + 1) + 12 * n + 8 * n * C + weights


def so2_flops_per_edge(L, C):
    """The SO(2) mix alone: 2[(L+1)^2 + 4 sum_{m>=1} (L+1-m)^2] C^2 per edge."""
    return 2 * ((L + 1) ** 2 + 4 * sum((L + 1 - m) ** 2 for m in range(1, L + 1))) * C * C


def forces_leg(B, torch, dev, w, pos, rp, col, feat, w_q, w_k, w_rad, w_so2, box):
    """What forces from an energy built on the layer need from one cotangent:
    dL/dh (for the layers below) and dL/dx (e2a_attention_bwd_weights with
    the position output); one warm-up and two timed calls."""
    e = int(col.numel())
    out, lse = B.e2a_attention_fwd(pos, rp, col, feat, w_q, w_k, w_rad, w_so2, L=w.L, C=w.C, H=w.H,
                                   cutoff=w.cutoff, box=box, with_lse=True)
    gen = torch.Generator(device=dev)
    gen.manual_seed(9)
    G = torch.randn(tuple(out.shape), generator=gen, device=dev, dtype=torch.float32)
    ws = torch.empty(B.e2a_attention_bwd_weights_workspace_bytes(w.n_atoms, e, w.L, w.C, w.H), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()

    def run():
        return B.e2a_attention_bwd_weights(pos, rp, col, feat, w_q, w_k, w_rad, w_so2, out, lse, G, L=w.L, C=w.C,
                                           H=w.H, cutoff=w.cutoff, box=box, weights=(), pos_grad=True, workspace=ws)

    run()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(2):
        res = run()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / 2
    return {"forces_ms": ms, "forces_edges_per_s": e / (ms * 1e-3),
            "forces_finite": all(bool(torch.isfinite(v).all()) for v in res.values()),
            "forces_kernels": "e2a_attention_bwd_weights: dL/dh and dL/dx (per-edge batches: SO2(x) and "
                              "SO2^T(dy) on the matrix cores, Wigner tangents per edge)"}


def training_backward_leg(B, torch, dev, w, pos, rp, col, feat, w_q, w_k, w_rad, w_so2, box):
    """Everything training the layer needs from one cotangent
    (e2a_attention_bwd_weights: dL/dh and the gradients of W_q, W_k, W_rad,
    W_so2); one warm-up and two timed calls.  Algorithmic work: the feature
    gradient's two passes plus, for the weights, the SO(2) mix of the rotated
    features (for dW_rad) and the weight products, each the size of the
    forward's mix."""
    e = int(col.numel())
    out, lse = B.e2a_attention_fwd(pos, rp, col, feat, w_q, w_k, w_rad, w_so2, L=w.L, C=w.C, H=w.H,
                                   cutoff=w.cutoff, box=box, with_lse=True)
    gen = torch.Generator(device=dev)
    gen.manual_seed(8)
    G = torch.randn(tuple(out.shape), generator=gen, device=dev, dtype=torch.float32)
    ws = torch.empty(B.e2a_attention_bwd_weights_workspace_bytes(w.n_atoms, e, w.L, w.C, w.H), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()

    def run():
        return B.e2a_attention_bwd_weights(pos, rp, col, feat, w_q, w_k, w_rad, w_so2, out, lse, G, L=w.L, C=w.C,
                                           H=w.H, cutoff=w.cutoff, box=box, workspace=ws)

    run()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(2):
        res = run()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / 2
    finite = all(bool(torch.isfinite(v).all()) for v in res.values())
    flops = (2 * flops_per_edge(w.L, w.C) + 2 * so2_flops_per_edge(w.L, w.C)) * e
    tflops = flops / (ms * 1e-3) / 1e12
    return {"train_backward_ms": ms, "train_backward_tflops": tflops,
            "train_backward_frac_of_bf16_peak": tflops / PEAK_BF16_TFLOPS, "train_backward_finite": finite,
            "train_backward_kernels": "e2a_attention_bwd_weights: dL/dh and dW_q, dW_k, dW_rad, dW_so2 "
                                      "(per-edge batches of 262144, GEMMs on the matrix cores)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="large")
    ap.add_argument("--variant", default="auto", choices=["auto", "mfma", "reference"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the other four workloads")
    ap.add_argument("--no-block", action="store_true", help="skip the block around the layer")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import so_graph_attention_amd.e2a as B
    from workloads import make_config

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    progress(f"generating workload {args.config}")
    w = make_config(args.config)
    box = None if w.box is None else w.box.tolist()

    def stored(name):
        a = getattr(w, name)
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    pos = torch.from_numpy(w.pos).to(dev)
    batch = None if w.batch is None else torch.from_numpy(w.batch.astype(np.int32)).to(dev)
    feat, w_q, w_k, w_rad, w_so2 = (stored(n) for n in ("feat", "w_q", "w_k", "w_rad", "w_so2"))
    n = w.n_atoms
    K = (w.L + 1) ** 2
    dtype_code = B.E2A_DTYPE_BF16 if w.dtype == "bf16" else B.E2A_DTYPE_F32
    out = torch.empty((n, K, w.C), dtype=torch.float32, device=dev)
    ws = torch.empty(B.e2a_attention_workspace_bytes(n, w.L, w.C, w.H, dtype_code), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    rp, col = B.e2a_build_neighbors(pos, w.cutoff, box=box, batch=batch)
    n_edges = int(col.numel())
    progress(f"{n} atoms, {n_edges} edges; warmup {args.warmup}")

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        r, c = B.e2a_build_neighbors(pos, w.cutoff, box=box, batch=batch, capacity=n_edges)
        if ev is not None:
            ev[1].record(stream)
        B.e2a_attention_fwd(pos, r, c, feat, w_q, w_k, w_rad, w_so2, L=w.L, C=w.C, H=w.H, cutoff=w.cutoff,
                            box=box, variant=args.variant, out=out, workspace=ws)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    progress(f"timing {args.steps} steps")
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    nb_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    attn_all = [e[1].elapsed_time(e[2]) for e in events]
    attn_ms = float(np.mean(attn_all))
    attn_med = float(np.median(attn_all))
    progress(f"step {ms_step:.3f} ms (neighbours {nb_ms:.3f} ms, attention {attn_ms:.3f} ms)")

    # self-check of the timed step: its output (and one more call's
    # log-normaliser) against the oracle, its neighbour list bit for bit
    progress("parity of the timed step against the oracle")
    lse = torch.empty((n, w.H), dtype=torch.float32, device=dev)
    out_chk = torch.empty_like(out)
    torch.cuda.reset_peak_memory_stats(dev)
    held = torch.cuda.memory_allocated(dev)
    B.e2a_attention_fwd(pos, rp, col, feat, w_q, w_k, w_rad, w_so2, L=w.L, C=w.C, H=w.H, cutoff=w.cutoff, box=box,
                        variant=args.variant, out=out_chk, out_lse=lse, workspace=ws)
    torch.cuda.synchronize()
    peak_delta = torch.cuda.max_memory_allocated(dev) - held
    same = bool(torch.equal(out_chk, out))
    parity = parity_check(w, rp.cpu().numpy(), col.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy())
    parity["launches_bit_identical"] = same
    progress(f"rel-L2 {parity['rel_l2']:.2e} on {parity['n_dest']} destinations, neighbours bit-exact "
             f"{parity['neighbours_bit_exact']}")
    memory = {"workspace_bytes": int(ws.numel()), "out_bytes": int(out.numel() * 4),
              "allocated_during_call_bytes": int(peak_delta),
              "edge_materialised_bytes": int(n_edges * K * w.C * 4),
              "note": "the library allocates nothing; its scratch is the caller's O(N) workspace, against "
                      "E x (L+1)^2 x C fp32 values for one materialised per-edge message tensor"}

    # the convolution stage (same messages, no attention weights), timed on
    # its own after the steps; it is not part of the headline step
    conv_out = torch.empty_like(out)

    def conv():
        B.e2a_conv_fwd(pos, rp, col, feat, w_rad, w_so2, L=w.L, C=w.C, H=w.H, cutoff=w.cutoff, box=box,
                       variant=args.variant, out=conv_out, workspace=ws)

    for _ in range(2):
        conv()
    cev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    cev[0].record(stream)
    for _ in range(args.steps):
        conv()
    cev[1].record(stream)
    torch.cuda.synchronize()
    conv_ms = cev[0].elapsed_time(cev[1]) / args.steps
    progress(f"convolution {conv_ms:.3f} ms")

    f_edge = flops_per_edge(w.L, w.C)

    bwd = None
    if not args.no_backward:
        progress("timing the feature gradient")
        bwd = backward_leg(B, torch, dev, w, pos, rp, col, feat, w_q, w_k, w_rad, w_so2, box)
        progress(f"feature gradient {bwd['backward_ms']:.1f} ms")
        progress("timing the training backward (feature and weight gradients)")
        bwd.update(training_backward_leg(B, torch, dev, w, pos, rp, col, feat, w_q, w_k, w_rad, w_so2, box))
        progress(f"training backward {bwd['train_backward_ms']:.1f} ms")
        progress("timing the forces (feature and position gradients)")
        bwd.update(forces_leg(B, torch, dev, w, pos, rp, col, feat, w_q, w_k, w_rad, w_so2, box))
        progress(f"forces {bwd['forces_ms']:.1f} ms")

    achieved = f_edge * n_edges / (attn_ms * 1e-3) / 1e12
    # the committed byte counters were taken on the 100k-atom workload
    traffic = traffic_per_launch() if args.config == "large" else None
    alg_bytes = algorithmic_bytes(w, n_edges)
    result = {
        "metric": METRIC,
        "value": n_edges / (ms_step * 1e-3),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {n} atoms, "
                               + ("periodic box %.3g A" % w.box[0] if w.box is not None else "open boundaries")
                               + f", cutoff {w.cutoff:g} A, L={w.L}, C={w.C}, H={w.H}, {w.dtype} storage",
                   "n_atoms": n, "n_edges": n_edges, "L": w.L, "C": w.C, "H": w.H,
                   "variant": args.variant},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "kernel": "e2a_attention_fwd (fused MFMA kernel + q/k prologue + weight pack)",
                     "flop_per_edge": f_edge},
        "breakdown": {"neighbors_ms": nb_ms, "attention_ms": attn_ms, "attention_ms_median": attn_med,
                      "attention_alg_bytes": alg_bytes,
                      "attention_alg_hbm_frac": alg_bytes / (attn_ms * 1e-3) / (PEAK_HBM_GBS * 1e9),
                      "attention_measured_hbm_frac": (None if traffic is None else
                                                      traffic / (attn_ms * 1e-3) / (PEAK_HBM_GBS * 1e9)),
                      "attention_edges_per_s": n_edges / (attn_ms * 1e-3),
                      "conv_ms": conv_ms, "conv_edges_per_s": n_edges / (conv_ms * 1e-3),
                      "conv_tflops": (f_edge - 2 * w.C) * n_edges / (conv_ms * 1e-3) / 1e12},
    }
    if bwd is not None:
        result["breakdown"].update(bwd)
    if not args.no_block:
        progress("timing one block and two stacked blocks")
        result["breakdown"].update(block_leg(B, torch, dev, w, pos, rp, col, box, attn_ms))
        progress(f"block {result['breakdown']['block_ms']:.1f} ms, two blocks "
                 f"{result['breakdown']['two_blocks_ms']:.1f} ms")
    result["parity"] = parity
    result["breakdown"]["memory"] = memory
    if not args.no_configs:
        result["breakdown"]["configs"] = {}
        for name in ("tiny", "drug", "water", "protein"):
            progress(f"workload {name}")
            r = config_leg(B, torch, dev, name)
            progress(f"{name}: {r['attention_ms']:.3f} ms, {r['frac']:.3f} of peak, rel-L2 "
                     f"{r['parity']['rel_l2']:.2e}, neighbours bit-exact {r['parity']['neighbours_bit_exact']}")
            result["breakdown"]["configs"][name] = r
    if not args.no_cpu_baseline:
        progress(f"oracle CPU baseline (~{args.cpu_seconds:.0f} s)")
        rp_h = rp.cpu().numpy()
        col_h = col.cpu().numpy()
        result["cpu_baseline"] = cpu_baseline(w, rp_h, col_h, args.cpu_seconds)
        progress("oracle single-thread runs (tiny, drug)")
        result["cpu_baseline"]["single_thread"] = [cpu_single_thread("tiny", 2.0),
                                                   cpu_single_thread("drug", 5.0)]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
