"""GPU convolution stage (the per-edge messages summed with no attention
weights, e2a_conv_fwd) vs the fp64 oracle's ``convolution``, element by
element on the same seeded inputs.

Tolerances (relative L2 over the compared outputs), as for the attention
layer: 1e-5 for the fp32 reference kernel, 2e-2 for the bf16 MFMA kernel
(bf16 operands, fp32 accumulation)."""
import numpy as np
import pytest
import torch

import oracle as O
from workloads import make_config
from workloads.generators import isolated_atom_variant

from gpu_util import log, rel_l2, sample_dest, to_device

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


@pytest.fixture(scope="module")
def B():
    import so_graph_attention_amd.e2a as mod
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return mod


def setup(w):
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    d = to_device(w)
    d["row_ptr"] = torch.from_numpy(rp).cuda()
    d["col"] = torch.from_numpy(col).cuda()
    return rp, col, d


def conv_gpu(B, w, d, variant):
    out = B.e2a_conv_fwd(d["pos"], d["row_ptr"], d["col"], d["feat"], d["w_rad"], d["w_so2"], L=w.L, C=w.C,
                         H=w.H, cutoff=w.cutoff, box=None if w.box is None else w.box.tolist(), variant=variant)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def conv_oracle(w, rp, col, dest=None):
    return O.convolution(w.pos, rp, col, w.as_f32("feat"), w.as_f32("w_rad"), w.as_f32("w_so2"), w.L, w.C,
                         w.cutoff, box=w.box, dest=dest)


def test_conv_tiny_fp32_full_output(B):
    log("[conv] tiny fp32 full")
    w = make_config("tiny")
    rp, col, d = setup(w)
    out = conv_gpu(B, w, d, "auto")
    err = rel_l2(out, conv_oracle(w, rp, col))
    log(f"[conv] tiny rel-L2 {err:.3e}")
    assert err <= TOL_F32


@pytest.mark.parametrize("L,C,H", [(0, 8, 2), (3, 32, 4)])
def test_conv_reference_kernel_bf16_shapes(B, L, C, H):
    log(f"[conv] reference tiny-geometry L={L} C={C} H={H} bf16")
    w = make_config("tiny", L=L, C=C, H=H, dtype="bf16")
    rp, col, d = setup(w)
    out = conv_gpu(B, w, d, "reference")
    err = rel_l2(out, conv_oracle(w, rp, col))
    log(f"[conv] rel-L2 {err:.3e}")
    assert err <= TOL_F32


@pytest.mark.parametrize("L", [1, 2, 4])
def test_conv_mfma_tiny_geometry_full_output(B, L):
    """C = 128, H = 8, bf16, every output of a 64-atom system plus one atom
    with no neighbours (its output must be exactly zero)."""
    log(f"[conv] mfma tiny-geometry L={L}")
    w = isolated_atom_variant(make_config("tiny", L=L, C=128, H=8, dtype="bf16"))
    rp, col, d = setup(w)
    assert rp[-1] == rp[-2]
    out = conv_gpu(B, w, d, "mfma")
    want = conv_oracle(w, rp, col)
    err = rel_l2(out, want)
    log(f"[conv] mfma L={L} rel-L2 {err:.3e}")
    assert np.all(np.isfinite(out))
    assert np.all(out[-1] == 0)
    assert err <= TOL_BF16


@pytest.mark.parametrize("name", ["drug", "large"])
def test_conv_mfma_full_configs_sampled(B, name):
    log(f"[conv] mfma {name}")
    w = make_config(name)
    rp, col, d = setup(w)
    out = conv_gpu(B, w, d, "auto")
    assert np.all(np.isfinite(out))
    dest = sample_dest(rp, 48, seed=13)
    err = rel_l2(out[dest], conv_oracle(w, rp, col, dest))
    log(f"[conv] mfma {name} rel-L2 {err:.3e} on {dest.size} atoms")
    assert err <= TOL_BF16


def test_conv_then_attention_share_a_workspace(B):
    """The convolution writes no state the attention call depends on: the
    same workspace serves both, in either order, with unchanged results."""
    log("[conv] shared workspace")
    w = make_config("drug")
    rp, col, d = setup(w)
    n, K = w.n_atoms, (w.L + 1) ** 2
    ws = torch.empty(B.e2a_attention_workspace_bytes(n, w.L, w.C, w.H, B.E2A_DTYPE_BF16), dtype=torch.uint8,
                     device="cuda")
    box = None if w.box is None else w.box.tolist()
    args = (d["pos"], d["row_ptr"], d["col"], d["feat"])
    a1 = B.e2a_attention_fwd(*args, d["w_q"], d["w_k"], d["w_rad"], d["w_so2"], L=w.L, C=w.C, H=w.H,
                             cutoff=w.cutoff, box=box, workspace=ws).clone()
    c1 = B.e2a_conv_fwd(*args, d["w_rad"], d["w_so2"], L=w.L, C=w.C, H=w.H, cutoff=w.cutoff, box=box,
                        workspace=ws).clone()
    a2 = B.e2a_attention_fwd(*args, d["w_q"], d["w_k"], d["w_rad"], d["w_so2"], L=w.L, C=w.C, H=w.H,
                             cutoff=w.cutoff, box=box, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2)
    assert c1.shape == (n, K, w.C) and bool(torch.isfinite(c1).all())
