"""Helpers shared by the GPU tests: move a workload to the device, sample
destinations, compare with the oracle."""
import sys

import numpy as np
import torch

import oracle as O


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_tensor(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def stored_tensor(w, name, dev):
    a = getattr(w, name)
    if a.dtype == np.uint16:
        return bf16_tensor(a, dev)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def to_device(w, dev="cuda:0"):
    d = {"pos": torch.from_numpy(np.ascontiguousarray(w.pos)).to(dev),
         "batch": None if w.batch is None else torch.from_numpy(np.ascontiguousarray(w.batch, dtype=np.int32)).to(dev)}
    for n in ("feat", "w_q", "w_k", "w_rad", "w_so2"):
        d[n] = stored_tensor(w, n, dev)
    return d


def sample_dest(rp, n_sample, seed):
    n = rp.size - 1
    deg = np.diff(rp)
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(n, size=min(n, n_sample), replace=False).tolist())
    pick |= {0, n - 1, int(np.argmax(deg)), int(np.argmin(deg))}
    return np.array(sorted(pick), dtype=np.int64)


def oracle_out(w, rp, col, dest):
    return O.attention(w.pos, rp, col, w.as_f32("feat"), w.as_f32("w_q"), w.as_f32("w_k"), w.as_f32("w_rad"),
                       w.as_f32("w_so2"), w.L, w.C, w.H, w.cutoff, box=w.box, dest=dest)


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
