"""GPU feature gradient (e2a_attention_bwd) vs the fp64 oracle's
``attention_backward`` on the same seeded inputs and the same seeded
cotangent.

The backward reads the forward's output o and log-normaliser.  Most tests take
them from the fp32 scalar forward, so that the comparison measures the
backward kernels (fp32 throughout): relative L2 <= 1e-5, the forward's fp32
bound (ds = alpha (dalpha - delta) subtracts two sums of the same size, but
the measured error stays below 1e-6).  One test takes o and lse from the bf16
MFMA forward (whose outputs are within 2e-2 of the oracle's) and holds the
gradient to 2e-2.  The matrix-core backward (bf16 operands, fp32 accumulation)
is held to 2e-2 against the oracle, on full outputs of 64-atom systems and on
samples of the drug-like and 100k-atom workloads."""
import numpy as np
import pytest
import torch

import oracle as O
from workloads import make_config

from gpu_util import log, rel_l2, sample_dest, to_device

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


@pytest.fixture(scope="module")
def B():
    import so_graph_attention_amd.e2a as mod
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return mod


def setup(w, seed=99):
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    d = to_device(w)
    d["row_ptr"] = torch.from_numpy(rp).cuda()
    d["col"] = torch.from_numpy(col).cuda()
    G = np.random.default_rng(seed).standard_normal((w.n_atoms, (w.L + 1) ** 2, w.C)).astype(np.float32)
    d["G"] = torch.from_numpy(G).cuda()
    return rp, col, d, G


def gpu_grad(B, w, d, fwd_variant="reference", bwd_variant="reference"):
    box = None if w.box is None else w.box.tolist()
    out, lse = B.e2a_attention_fwd(d["pos"], d["row_ptr"], d["col"], d["feat"], d["w_q"], d["w_k"], d["w_rad"],
                                   d["w_so2"], L=w.L, C=w.C, H=w.H, cutoff=w.cutoff, box=box, variant=fwd_variant,
                                   with_lse=True)
    g = B.e2a_attention_bwd(d["pos"], d["row_ptr"], d["col"], d["feat"], d["w_q"], d["w_k"], d["w_rad"],
                            d["w_so2"], out, lse, d["G"], L=w.L, C=w.C, H=w.H, cutoff=w.cutoff, box=box,
                            variant=bwd_variant)
    torch.cuda.synchronize()
    return g.cpu().numpy()


def oracle_grad(w, rp, col, G, dest=None):
    return O.attention_backward(w.pos, rp, col, w.as_f32("feat"), w.as_f32("w_q"), w.as_f32("w_k"),
                                w.as_f32("w_rad"), w.as_f32("w_so2"), w.L, w.C, w.H, w.cutoff, G, box=w.box,
                                dest=dest)


@pytest.mark.parametrize("L,C,H,dtype", [(1, 16, 1, "f32"), (1, 16, 2, "f32"), (0, 8, 2, "f32"),
                                         (2, 24, 3, "bf16"), (3, 32, 4, "f32"), (4, 32, 8, "bf16")])
def test_bwd_tiny_geometry_full(B, L, C, H, dtype):
    log(f"[bwd] tiny geometry L={L} C={C} H={H} {dtype}")
    w = make_config("tiny", L=L, C=C, H=H, dtype=dtype)
    rp, col, d, G = setup(w)
    got = gpu_grad(B, w, d)
    err = rel_l2(got, oracle_grad(w, rp, col, G))
    log(f"[bwd] rel-L2 {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= TOL_F32


def test_bwd_small_periodic_box(B):
    """120 atoms in an 11 A periodic box (about 47 neighbours each; minimum
    image on every edge frame)."""
    from workloads.generators import _rsa_periodic, _to_f32_periodic
    log("[bwd] periodic")
    rng = np.random.default_rng(1414)
    box = np.full(3, 11.0)
    pos = _to_f32_periodic(_rsa_periodic(rng, 120, 11.0, 0.9), box)
    w = make_config("tiny", L=2, C=16, H=2, geometry=(pos, box.astype(np.float32), None, {}))
    rp, col, d, G = setup(w)
    got = gpu_grad(B, w, d)
    err = rel_l2(got, oracle_grad(w, rp, col, G))
    log(f"[bwd] periodic rel-L2 {err:.3e}")
    assert err <= TOL_F32


def test_bwd_drug_sampled(B):
    """The drug-like batch (L = 3, C = 128, H = 8, bf16 storage): seeded sample
    of atoms, backward on the fp32 forward's outputs."""
    log("[bwd] drug sampled")
    w = make_config("drug")
    rp, col, d, G = setup(w)
    got = gpu_grad(B, w, d)
    dest = sample_dest(rp, 40, seed=21)
    err = rel_l2(got[dest], oracle_grad(w, rp, col, G, dest))
    log(f"[bwd] drug rel-L2 {err:.3e} on {dest.size} atoms")
    assert err <= TOL_F32


def test_bwd_after_mfma_forward(B):
    """The same, with o and lse from the bf16 MFMA forward."""
    log("[bwd] drug after the MFMA forward")
    w = make_config("drug")
    rp, col, d, G = setup(w)
    got = gpu_grad(B, w, d, fwd_variant="mfma", bwd_variant="reference")
    dest = sample_dest(rp, 40, seed=22)
    err = rel_l2(got[dest], oracle_grad(w, rp, col, G, dest))
    log(f"[bwd] drug (MFMA forward) rel-L2 {err:.3e}")
    assert err <= TOL_BF16


def test_bwd_isolated_atom_and_determinism(B):
    """An atom with no neighbours gets the gradient of its l = 0 block only
    through nothing (it is no one's neighbour and has no edges): zero.  Two
    launches give bit-identical gradients."""
    from workloads.generators import isolated_atom_variant
    log("[bwd] isolated atom, determinism")
    w = isolated_atom_variant(make_config("tiny", L=2, C=16, H=2))
    rp, col, d, G = setup(w)
    assert rp[-1] == rp[-2]
    g1 = gpu_grad(B, w, d)
    g2 = gpu_grad(B, w, d)
    assert np.array_equal(g1, g2)
    assert np.all(g1[-1] == 0)
    assert rel_l2(g1, oracle_grad(w, rp, col, G)) <= TOL_F32


@pytest.mark.parametrize("L", [1, 2, 3, 4])
def test_bwd_mfma_tiny_geometry_full(B, L):
    """Matrix-core passes, C = 128, H = 8, bf16: every row of the gradient of
    a 64-atom system, against the oracle and against the scalar kernels."""
    log(f"[bwd] mfma tiny geometry L={L}")
    w = make_config("tiny", L=L, C=128, H=8, dtype="bf16")
    rp, col, d, G = setup(w)
    got = gpu_grad(B, w, d, fwd_variant="mfma", bwd_variant="mfma")
    ref = gpu_grad(B, w, d, fwd_variant="mfma", bwd_variant="reference")
    want = oracle_grad(w, rp, col, G)
    err = rel_l2(got, want)
    # the l = 0 block alone carries the logit path (dq W_q^T + dk W_k^T)
    err0 = rel_l2(got[:, 0], want[:, 0])
    log(f"[bwd] mfma L={L} rel-L2 {err:.3e} (l = 0 block {err0:.3e}), vs scalar {rel_l2(got, ref):.3e}")
    assert np.all(np.isfinite(got))
    assert err <= TOL_BF16 and err0 <= TOL_BF16
    assert rel_l2(got, ref) <= TOL_BF16


@pytest.mark.parametrize("name", ["drug", "large"])
def test_bwd_mfma_configs_sampled(B, name):
    log(f"[bwd] mfma {name}")
    w = make_config(name)
    rp, col, d, G = setup(w)
    got = gpu_grad(B, w, d, fwd_variant="mfma", bwd_variant="mfma")
    assert np.all(np.isfinite(got))
    dest = sample_dest(rp, 24, seed=23)
    err = rel_l2(got[dest], oracle_grad(w, rp, col, G, dest))
    log(f"[bwd] mfma {name} rel-L2 {err:.3e} on {dest.size} atoms")
    assert err <= TOL_BF16


def test_bwd_mfma_deterministic(B):
    log("[bwd] mfma determinism")
    w = make_config("drug")
    rp, col, d, G = setup(w)
    g1 = gpu_grad(B, w, d, fwd_variant="mfma", bwd_variant="mfma")
    g2 = gpu_grad(B, w, d, fwd_variant="mfma", bwd_variant="mfma")
    assert np.array_equal(g1, g2)


@pytest.mark.parametrize("scale", [2.0 ** -20, 2.0 ** 20])
def test_bwd_mfma_cotangent_power_of_two(B, scale):
    """The matrix-core passes normalise the cotangent by powers of two (per
    atom for the query pass's fp16 copy, by its global maximum in the value
    pass), so every rounding sees the same significands and a cotangent
    scaled by 2^-20 or 2^20 gives exactly the scaled gradient."""
    log(f"[bwd] mfma cotangent x {scale:g}")
    w = make_config("tiny", L=4, C=128, H=8, dtype="bf16")
    rp, col, d, G = setup(w)
    g1 = gpu_grad(B, w, d, fwd_variant="mfma", bwd_variant="mfma")
    d["G"] = d["G"] * scale
    g2 = gpu_grad(B, w, d, fwd_variant="mfma", bwd_variant="mfma")
    assert np.array_equal(g2, g1 * np.float32(scale))


@pytest.mark.parametrize("scale", [1e-7, 1e6])
def test_bwd_mfma_cotangent_magnitude(B, scale):
    """Cotangents whose fp16 images would be subnormal (1e-7) or overflow
    (1e6) without the normalisation keep the bf16 bound against the oracle."""
    log(f"[bwd] mfma cotangent magnitude {scale:g}")
    w = make_config("tiny", L=3, C=128, H=8, dtype="bf16")
    rp, col, d, G = setup(w)
    Gs = (G.astype(np.float64) * scale).astype(np.float32)
    d["G"] = torch.from_numpy(Gs).cuda()
    got = gpu_grad(B, w, d, fwd_variant="mfma", bwd_variant="mfma")
    err = rel_l2(got, oracle_grad(w, rp, col, Gs))
    log(f"[bwd] mfma cotangent x {scale:g}: rel-L2 {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= TOL_BF16
