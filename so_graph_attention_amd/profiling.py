"""Small programs to run under rocprofv3.

  python -m so_graph_attention_amd.profiling attention [--config large] [--iters 2]
      the fused layer on one workload, `iters` launches after one warm-up;
  python -m so_graph_attention_amd.profiling block [--config large] [--iters 2]
      one block around the layer (e2a_block_fwd) on one workload;
  python -m so_graph_attention_amd.profiling gradients [--config large] [--iters 2] [--forces]
      e2a_attention_bwd_weights on one workload: dL/dh and every weight
      gradient (training), or with --forces dL/dh and dL/dx;
  python -m so_graph_attention_amd.profiling neighbors [--config large] [--iters 10]
      the neighbour build (e2a_build_neighbors) on one workload, `iters`
      calls after one warm-up, each with the edge capacity it needs;
  python -m so_graph_attention_amd.profiling copy [--mib 1024] [--iters 2]
      a plain device-to-device copy of known size, whose FETCH_SIZE /
      WRITE_SIZE readings calibrate the byte counters of the layer's run.

Each prints what it ran and exits; none reads the oracle.
"""
import argparse
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def run_attention(config: str, iters: int, variant: str):
    import torch

    import so_graph_attention_amd.e2a as B
    from workloads import make_config

    dev = torch.device("cuda:0")
    w = make_config(config)

    def stored(name):
        a = getattr(w, name)
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    pos = torch.from_numpy(w.pos).to(dev)
    box = None if w.box is None else w.box.tolist()
    batch = None if w.batch is None else torch.from_numpy(w.batch.astype(np.int32)).to(dev)
    rp, col = B.e2a_build_neighbors(pos, w.cutoff, box=box, batch=batch)
    tensors = [stored(n) for n in ("feat", "w_q", "w_k", "w_rad", "w_so2")]
    out = None
    for _ in range(iters + 1):
        out = B.e2a_attention_fwd(pos, rp, col, *tensors, L=w.L, C=w.C, H=w.H, cutoff=w.cutoff, box=box,
                                  variant=variant, out=out)
    torch.cuda.synchronize()
    print(f"attention {config}: {w.n_atoms} atoms, {col.numel()} edges, {iters + 1} launches", flush=True)


def run_block(config: str, iters: int):
    import torch

    import so_graph_attention_amd.e2a as B
    from workloads import make_block_weights, make_config

    dev = torch.device("cuda:0")
    w = make_config(config)

    def stored(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    pos = torch.from_numpy(w.pos).to(dev)
    box = None if w.box is None else w.box.tolist()
    batch = None if w.batch is None else torch.from_numpy(w.batch.astype(np.int32)).to(dev)
    rp, col = B.e2a_build_neighbors(pos, w.cutoff, box=box, batch=batch)
    bw = {k: stored(v) for k, v in make_block_weights(w).items()}
    h = torch.from_numpy(np.ascontiguousarray(w.as_f32("feat"))).to(dev)
    out = torch.empty_like(h)
    for _ in range(iters + 1):
        B.e2a_block_fwd(pos, rp, col, h, bw, L=w.L, C=w.C, H=w.H, cutoff=w.cutoff, box=box, out=out)
    torch.cuda.synchronize()
    print(f"block {config}: {w.n_atoms} atoms, {col.numel()} edges, {iters + 1} calls", flush=True)


def run_gradients(config: str, iters: int, forces: bool):
    import torch

    import so_graph_attention_amd.e2a as B
    from workloads import make_config

    dev = torch.device("cuda:0")
    w = make_config(config)

    def stored(name):
        a = getattr(w, name)
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    pos = torch.from_numpy(w.pos).to(dev)
    box = None if w.box is None else w.box.tolist()
    batch = None if w.batch is None else torch.from_numpy(w.batch.astype(np.int32)).to(dev)
    rp, col = B.e2a_build_neighbors(pos, w.cutoff, box=box, batch=batch)
    feat, w_q, w_k, w_rad, w_so2 = [stored(n) for n in ("feat", "w_q", "w_k", "w_rad", "w_so2")]
    out, lse = B.e2a_attention_fwd(pos, rp, col, feat, w_q, w_k, w_rad, w_so2, L=w.L, C=w.C, H=w.H,
                                   cutoff=w.cutoff, box=box, with_lse=True)
    gen = torch.Generator(device=dev)
    gen.manual_seed(8)
    G = torch.randn(tuple(out.shape), generator=gen, device=dev, dtype=torch.float32)
    ws = torch.empty(B.e2a_attention_bwd_weights_workspace_bytes(w.n_atoms, col.numel(), w.L, w.C, w.H),
                     dtype=torch.uint8, device=dev)
    kw = dict(weights=(), pos_grad=True) if forces else {}
    for _ in range(iters + 1):
        B.e2a_attention_bwd_weights(pos, rp, col, feat, w_q, w_k, w_rad, w_so2, out, lse, G, L=w.L, C=w.C, H=w.H,
                                    cutoff=w.cutoff, box=box, workspace=ws, **kw)
    torch.cuda.synchronize()
    what = "forces" if forces else "training"
    print(f"gradients ({what}) {config}: {w.n_atoms} atoms, {col.numel()} edges, {iters + 1} calls", flush=True)


def run_neighbors(config: str, iters: int):
    import torch

    import so_graph_attention_amd.e2a as B
    from workloads import make_config

    dev = torch.device("cuda:0")
    w = make_config(config)
    pos = torch.from_numpy(w.pos).to(dev)
    box = None if w.box is None else w.box.tolist()
    batch = None if w.batch is None else torch.from_numpy(w.batch.astype(np.int32)).to(dev)
    rp, col = B.e2a_build_neighbors(pos, w.cutoff, box=box, batch=batch)
    for _ in range(iters):
        B.e2a_build_neighbors(pos, w.cutoff, box=box, batch=batch, capacity=col.numel())
    torch.cuda.synchronize()
    print(f"neighbors {config}: {w.n_atoms} atoms, {col.numel()} edges, {iters + 1} builds", flush=True)


def run_copy(mib: int, iters: int):
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(iters + 1):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy: {mib} MiB x {iters + 1}", flush=True)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("attention")
    a.add_argument("--config", default="large")
    a.add_argument("--iters", type=int, default=2)
    a.add_argument("--variant", default="auto")
    b = sub.add_parser("block")
    b.add_argument("--config", default="large")
    b.add_argument("--iters", type=int, default=2)
    g = sub.add_parser("gradients")
    g.add_argument("--config", default="large")
    g.add_argument("--iters", type=int, default=2)
    g.add_argument("--forces", action="store_true")
    nb = sub.add_parser("neighbors")
    nb.add_argument("--config", default="large")
    nb.add_argument("--iters", type=int, default=10)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--iters", type=int, default=2)
    args = ap.parse_args()
    if args.what == "attention":
        run_attention(args.config, args.iters, args.variant)
    elif args.what == "block":
        run_block(args.config, args.iters)
    elif args.what == "neighbors":
        run_neighbors(args.config, args.iters)
    elif args.what == "gradients":
        run_gradients(args.config, args.iters, args.forces)
    else:
        run_copy(args.mib, args.iters)


if __name__ == "__main__":
    main()
