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
