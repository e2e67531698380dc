"""Small programs to run under rocprofv3.

  python -m so_graph_attention_amd.profiling attention [--config large] [--iters 2]
      the fused layer on one workload, `iters` launches after one warm-up;
  python -m so_graph_attention_amd.profiling copy [--mib 1024] [--iters 2]
      a plain device-to-device copy of known size, whose FETCH_SIZE /
      WRITE_SIZE readings calibrate the byte counters of the layer's run.

Both print what they ran and exit; neither reads the oracle.
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
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--iters", type=int, default=2)
    args = ap.parse_args()
    if args.what == "attention":
        run_attention(args.config, args.iters, args.variant)
    else:
        run_copy(args.mib, args.iters)


if __name__ == "__main__":
    main()
