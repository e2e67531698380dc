"""Weights packed once (e2a_pack_so2_weights) and a destination order given
by the caller (e2a_destination_order) give the plain call's result bit for
bit; another order gives a result within the bf16 bound of the oracle (the
order only decides which atoms share edge tiles)."""
import numpy as np
import pytest
import torch

import oracle as O
from workloads import make_block_weights, make_config

from gpu_util import log, oracle_out, rel_l2, sample_dest, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import so_graph_attention_amd.e2a as mod
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return mod


@pytest.fixture(scope="module")
def drug(B):
    w = make_config("drug")
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    d = to_device(w)
    d["row_ptr"] = torch.from_numpy(rp).cuda()
    d["col"] = torch.from_numpy(col).cuda()
    return w, rp, col, d


def fwd(B, w, d, **kw):
    out, lse = B.e2a_attention_fwd(d["pos"], d["row_ptr"], d["col"], d["feat"], d["w_q"], d["w_k"], d["w_rad"],
                                   d["w_so2"], L=w.L, C=w.C, H=w.H, cutoff=w.cutoff, with_lse=True, **kw)
    torch.cuda.synchronize()
    return out, lse


def test_prepacked_and_given_order_bit_identical(B, drug):
    log("[prepacked] drug-like: packed image and caller order")
    w, rp, col, d = drug
    base, base_lse = fwd(B, w, d)
    packed = B.e2a_pack_so2_weights(d["w_so2"], L=w.L, C=w.C)
    order = B.e2a_destination_order(d["pos"])
    torch.cuda.synchronize()
    o = order.cpu().numpy()
    assert np.array_equal(np.sort(o), np.arange(w.n_atoms))
    out, lse = fwd(B, w, d, w_so2_packed=packed, order=order)
    assert torch.equal(out, base) and torch.equal(lse, base_lse)
    conv_a = B.e2a_conv_fwd(d["pos"], d["row_ptr"], d["col"], d["feat"], d["w_rad"], d["w_so2"], L=w.L, C=w.C,
                            cutoff=w.cutoff)
    conv_b = B.e2a_conv_fwd(d["pos"], d["row_ptr"], d["col"], d["feat"], d["w_rad"], d["w_so2"], L=w.L, C=w.C,
                            cutoff=w.cutoff, w_so2_packed=packed, order=order)
    torch.cuda.synchronize()
    assert torch.equal(conv_a, conv_b)


def test_other_order_within_bound(B, drug):
    log("[prepacked] drug-like: reversed atom order")
    w, rp, col, d = drug
    order = torch.arange(w.n_atoms - 1, -1, -1, dtype=torch.int32, device="cuda")
    out, _ = fwd(B, w, d, order=order)
    dest = sample_dest(rp, 64, 13)
    want, _ = oracle_out(w, rp, col, dest)
    err = rel_l2(out.cpu().numpy()[dest], want)
    log(f"[prepacked] rel-L2 {err:.3e}")
    assert err <= 2e-2


def test_block_with_packed_and_order(B):
    w = make_config("tiny", L=3, C=128, H=8, dtype="bf16")
    rp, col = O.neighbor_list(w.pos, w.cutoff)
    d = to_device(w)
    d["row_ptr"] = torch.from_numpy(rp).cuda()
    d["col"] = torch.from_numpy(col).cuda()
    bw = {k: torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).cuda()
          for k, v in make_block_weights(w).items()}
    h = torch.from_numpy(np.ascontiguousarray(w.as_f32("feat"))).cuda()
    a = B.e2a_block_fwd(d["pos"], d["row_ptr"], d["col"], h, bw, L=w.L, C=w.C, H=w.H, cutoff=w.cutoff)
    b = B.e2a_block_fwd(d["pos"], d["row_ptr"], d["col"], h, bw, L=w.L, C=w.C, H=w.H, cutoff=w.cutoff,
                        w_so2_packed=B.e2a_pack_so2_weights(bw["w_so2"], L=w.L, C=w.C),
                        order=B.e2a_destination_order(d["pos"]))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def morton_order_cpu(pos):
    """The documented default order, in numpy fp32: cells of a 64^3 grid over
    the bounding box, the Morton code of the cell (x in bit 0 of each bit
    triple), stably sorted so that ties keep the atom index order."""
    p = np.ascontiguousarray(pos, dtype=np.float32)
    lo, hi = p.min(axis=0), p.max(axis=0)
    ext = np.maximum(hi - lo, np.float32(1e-6))
    f = (p - lo) / ext * np.float32(64)
    c = np.clip(f, np.float32(0), np.float32(63)).astype(np.uint32)
    key = np.zeros(len(p), dtype=np.uint32)
    for b in range(6):
        for d in range(3):
            key |= ((c[:, d] >> b) & 1) << (3 * b + d)
    return np.argsort(key, kind="stable").astype(np.int32)


@pytest.mark.parametrize("case", ["drug", "one", "five", "one_block_plus", "clustered", "n70k", "n200k"])
def test_destination_order_is_the_stable_morton_order(B, case):
    """The fused order (keys with the first digit counts, the second counts
    taken in the first scatter, one-launch scans up to 65,536 entries and the
    three-launch scan beyond) against the same order computed on the host;
    the clustered case has many atoms per cell, so ties decide most of it."""
    rng = np.random.default_rng(7)
    if case == "drug":
        pos = make_config("drug").pos
    elif case == "clustered":
        pos = (rng.integers(0, 4, size=(5000, 3)) * 2.0).astype(np.float32)
    else:
        n = {"one": 1, "five": 5, "one_block_plus": 1025, "n70k": 70000, "n200k": 200000}[case]
        pos = rng.uniform(-20.0, 35.0, size=(n, 3)).astype(np.float32)
    log(f"[order] {case}: {len(pos)} atoms")
    got = B.e2a_destination_order(torch.from_numpy(np.ascontiguousarray(pos)).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), morton_order_cpu(pos))
