"""GPU edge cases against the fp64 oracle: edges exactly along the frame's
poles and axes, input magnitudes far from one, atoms at one point, a
zero-length edge in a hand-made graph, and more heads than the scalar
kernel has softmax threads.

Tolerances as elsewhere: relative L2 <= 1e-5 for fp32 storage (scalar
kernels), <= 2e-2 for bf16 storage on the matrix cores.  Scaling a weight by
a power of two must scale the matrix-core output by exactly that power (every
operand keeps fp32's exponent range)."""
import numpy as np
import pytest
import torch

import oracle as O
from workloads import axis_lattice_geometry, coincident_geometry, f32_to_bf16_bits, make_config

from gpu_util import bf16_tensor, log, rel_l2, to_device

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


@pytest.fixture(scope="module")
def B():
    import so_graph_attention_amd.e2a as mod
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return mod


def graph(w, d=None):
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    d = to_device(w) if d is None else d
    d["row_ptr"] = torch.from_numpy(rp).cuda()
    d["col"] = torch.from_numpy(col).cuda()
    return rp, col, d


def fwd(B, w, d, variant):
    out, lse = B.e2a_attention_fwd(d["pos"], d["row_ptr"], d["col"], d["feat"], d["w_q"], d["w_k"], d["w_rad"],
                                   d["w_so2"], L=w.L, C=w.C, H=w.H, cutoff=w.cutoff,
                                   box=None if w.box is None else w.box.tolist(), variant=variant, with_lse=True)
    torch.cuda.synchronize()
    return out, lse


def oracle_fwd(w, rp, col, feat=None, w_so2=None, w_rad=None):
    return O.attention(w.pos, rp, col, w.as_f32("feat") if feat is None else feat, w.as_f32("w_q"),
                       w.as_f32("w_k"), w.as_f32("w_rad") if w_rad is None else w_rad,
                       w.as_f32("w_so2") if w_so2 is None else w_so2, w.L, w.C, w.H, w.cutoff, box=w.box)


# ------------------------------------------------------------ poles, axes ---
@pytest.mark.parametrize("L", [1, 2, 3, 4])
def test_axis_lattice_mfma_forward_conv_backward(B, L):
    """A cubic lattice: 576 of its 3216 edges lie exactly along +-x, +-y or
    +-z, so the frame's pole branch (r_hat = +-z, phi undefined) and the
    recursion at axis directions run on the device."""
    log(f"[edge] axis lattice L={L} mfma")
    w = make_config("tiny", L=L, C=128, H=8, dtype="bf16", geometry=axis_lattice_geometry())
    rp, col, d = graph(w)
    out, lse = fwd(B, w, d, "mfma")
    want, want_lse = oracle_fwd(w, rp, col)
    err = rel_l2(out.cpu().numpy(), want)
    log(f"[edge] forward rel-L2 {err:.3e}")
    assert err <= TOL_BF16
    assert np.max(np.abs(lse.cpu().numpy() - want_lse)) <= 1e-3
    conv = B.e2a_conv_fwd(d["pos"], d["row_ptr"], d["col"], d["feat"], d["w_rad"], d["w_so2"], L=L, C=w.C, H=w.H,
                          cutoff=w.cutoff, variant="mfma")
    torch.cuda.synchronize()
    cwant = O.convolution(w.pos, rp, col, w.as_f32("feat"), w.as_f32("w_rad"), w.as_f32("w_so2"), L, w.C,
                          w.cutoff)
    cerr = rel_l2(conv.cpu().numpy(), cwant)
    log(f"[edge] convolution rel-L2 {cerr:.3e}")
    assert cerr <= TOL_BF16
    G = np.random.default_rng(7).standard_normal((w.n_atoms, (L + 1) ** 2, w.C)).astype(np.float32)
    g = B.e2a_attention_bwd(d["pos"], d["row_ptr"], d["col"], d["feat"], d["w_q"], d["w_k"], d["w_rad"],
                            d["w_so2"], out, lse, torch.from_numpy(G).cuda(), L=L, C=w.C, H=w.H, cutoff=w.cutoff,
                            variant="mfma")
    torch.cuda.synchronize()
    gwant = O.attention_backward(w.pos, rp, col, w.as_f32("feat"), w.as_f32("w_q"), w.as_f32("w_k"),
                                 w.as_f32("w_rad"), w.as_f32("w_so2"), L, w.C, w.H, w.cutoff, G)
    gerr = rel_l2(g.cpu().numpy(), gwant)
    log(f"[edge] feature gradient rel-L2 {gerr:.3e}")
    assert gerr <= TOL_BF16


@pytest.mark.parametrize("L", [1, 2, 3, 4])
def test_axis_lattice_reference_kernels_fp32(B, L):
    log(f"[edge] axis lattice L={L} reference fp32")
    w = make_config("tiny", L=L, C=16, H=2, dtype="f32", geometry=axis_lattice_geometry())
    rp, col, d = graph(w)
    out, lse = fwd(B, w, d, "reference")
    want, want_lse = oracle_fwd(w, rp, col)
    err = rel_l2(out.cpu().numpy(), want)
    log(f"[edge] rel-L2 {err:.3e}")
    assert err <= TOL_F32
    G = np.random.default_rng(8).standard_normal((w.n_atoms, (L + 1) ** 2, w.C)).astype(np.float32)
    g = B.e2a_attention_bwd(d["pos"], d["row_ptr"], d["col"], d["feat"], d["w_q"], d["w_k"], d["w_rad"],
                            d["w_so2"], out, lse, torch.from_numpy(G).cuda(), L=L, C=w.C, H=w.H, cutoff=w.cutoff,
                            variant="reference")
    torch.cuda.synchronize()
    gwant = O.attention_backward(w.pos, rp, col, w.as_f32("feat"), w.as_f32("w_q"), w.as_f32("w_k"),
                                 w.as_f32("w_rad"), w.as_f32("w_so2"), L, w.C, w.H, w.cutoff, G)
    gerr = rel_l2(g.cpu().numpy(), gwant)
    log(f"[edge] feature gradient rel-L2 {gerr:.3e}")
    assert gerr <= TOL_F32


def test_axis_lattice_position_gradient(B):
    """dL/dx on the lattice (edges along the axes, where the frame's angles
    are singular) against the oracle's central differences, sampled atoms."""
    log("[edge] axis lattice position gradient L=2 fp32")
    w = make_config("tiny", L=2, C=16, H=2, dtype="f32", geometry=axis_lattice_geometry())
    rp, col, d = graph(w)
    out, lse = fwd(B, w, d, "reference")
    G = np.random.default_rng(9).standard_normal((w.n_atoms, 9, w.C)).astype(np.float32)
    res = B.e2a_attention_bwd_weights(d["pos"], d["row_ptr"], d["col"], d["feat"], d["w_q"], d["w_k"], d["w_rad"],
                                      d["w_so2"], out, lse, torch.from_numpy(G).cuda(), L=2, C=w.C, H=w.H,
                                      cutoff=w.cutoff, variant="reference", feat_grad=False, weights=(),
                                      pos_grad=True)
    torch.cuda.synchronize()
    atoms = np.array([0, 5, 21, 42, 63])
    want = O.attention_position_backward(w.pos, rp, col, w.as_f32("feat"), w.as_f32("w_q"), w.as_f32("w_k"),
                                         w.as_f32("w_rad"), w.as_f32("w_so2"), 2, w.C, w.H, w.cutoff, G,
                                         atoms=atoms)
    err = rel_l2(res["pos"].cpu().numpy()[atoms], want)
    log(f"[edge] position gradient rel-L2 {err:.3e}")
    assert err <= TOL_F32


# --------------------------------------------------------------- magnitudes -
@pytest.fixture(scope="module")
def mag_case(B):
    w = make_config("tiny", L=4, C=128, H=8, dtype="bf16")
    rp, col, d = graph(w)
    return w, rp, col, d


@pytest.mark.parametrize("which", ["w_so2", "w_rad"])
@pytest.mark.parametrize("k", [20, -20])
def test_mfma_weight_power_of_two_scales_output_exactly(B, mag_case, which, k):
    """A weight scaled by 2^k scales the output by exactly 2^k: the SO(2)
    product, the radial product, the alpha*rho*y operand and the rotate-out
    keep fp32's exponent range (bf16 operands, fp32 sums)."""
    log(f"[edge] {which} x 2^{k}")
    w, rp, col, d = mag_case
    base, _ = fwd(B, w, d, "mfma")
    d2 = dict(d)
    d2[which] = d[which] * (2.0 ** k)
    scaled, _ = fwd(B, w, d2, "mfma")
    got = scaled.cpu().numpy()
    assert np.all(np.isfinite(got))
    assert np.array_equal(got, base.cpu().numpy() * np.float32(2.0 ** k))


@pytest.mark.parametrize("scale", [1e-6, 1e5])
def test_mfma_feature_magnitudes(B, mag_case, scale):
    """Features of degree >= 1 scaled by 1e-6 or 1e5 (rounded to bf16 again;
    the oracle reads the same rounded values) stay within the bf16 bound."""
    log(f"[edge] l >= 1 features x {scale:g}")
    w, rp, col, d = mag_case
    f = w.as_f32("feat").copy()
    f[:, 1:, :] *= np.float32(scale)
    bits = f32_to_bf16_bits(f)
    d2 = dict(d)
    d2["feat"] = bf16_tensor(bits, "cuda:0")
    out, _ = fwd(B, w, d2, "mfma")
    want, _ = oracle_fwd(w, rp, col, feat=(bits.astype(np.uint32) << 16).view(np.float32))
    got = out.cpu().numpy()
    err_hi = rel_l2(got[:, 1:], want[:, 1:])
    err_0 = rel_l2(got[:, :1], want[:, :1])
    log(f"[edge] rel-L2 l >= 1 {err_hi:.3e}, l = 0 {err_0:.3e}")
    assert err_hi <= TOL_BF16 and err_0 <= TOL_BF16


# --------------------------------------------------------- coincident atoms -
def test_neighbours_skip_coincident_atoms(B):
    """Atoms at one point are not each other's neighbours; the GPU list equals
    the oracle's bit for bit (which a brute-force pin checks on the CPU)."""
    log("[edge] coincident atoms: neighbour build")
    w = make_config("tiny", geometry=coincident_geometry(np.random.default_rng(3)))
    rp, col = O.neighbor_list(w.pos, w.cutoff)
    grp, gcol = B.e2a_build_neighbors(torch.from_numpy(w.pos).cuda(), w.cutoff)
    torch.cuda.synchronize()
    assert np.array_equal(grp.cpu().numpy(), rp) and np.array_equal(gcol.cpu().numpy(), col)
    dup = w.meta["duplicated"]
    for t, a in enumerate(dup):
        b = 64 + t
        assert b not in col[rp[a]:rp[a + 1]] and a not in col[rp[b]:rp[b + 1]]


@pytest.mark.parametrize("variant,L,C,H,dtype,tol", [("reference", 2, 16, 2, "f32", TOL_F32),
                                                      ("mfma", 3, 128, 8, "bf16", TOL_BF16)])
def test_zero_length_edge_in_a_given_graph(B, variant, L, C, H, dtype, tol):
    """A caller-built graph may pair two atoms at one point: that edge takes
    the identity frame (r_hat = z), as the oracle reads it; every output stays
    finite, including the other destination sharing the edge chunk."""
    log(f"[edge] zero-length edge, {variant}")
    w = make_config("tiny", L=L, C=C, H=H, dtype=dtype, geometry=coincident_geometry(np.random.default_rng(4)))
    rp, col = O.neighbor_list(w.pos, w.cutoff)
    a, b = w.meta["duplicated"][0], 64
    # insert the edges (a, b) and (b, a) into the sorted rows
    src = np.repeat(np.arange(w.n_atoms), np.diff(rp)).tolist() + [a, b]
    dst = col.tolist() + [b, a]
    order = np.lexsort((np.array(dst), np.array(src)))
    src = np.array(src)[order]
    col2 = np.array(dst, dtype=np.int32)[order]
    rp2 = np.zeros(w.n_atoms + 1, dtype=np.int64)
    np.cumsum(np.bincount(src, minlength=w.n_atoms), out=rp2[1:])
    d = to_device(w)
    d["row_ptr"] = torch.from_numpy(rp2).cuda()
    d["col"] = torch.from_numpy(col2).cuda()
    out, lse = fwd(B, w, d, variant)
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(lse.cpu().numpy()[np.diff(rp2) > 0]))
    want, _ = oracle_fwd(w, rp2, col2)
    err = rel_l2(got, want)
    log(f"[edge] rel-L2 {err:.3e}")
    assert err <= tol
    assert rel_l2(got[[a, b]], want[[a, b]]) <= tol


# ------------------------------------------------------------- many heads ---
def test_reference_kernel_more_heads_than_threads(B):
    """H = 256 heads (one channel each) on the scalar kernel: every head's
    online softmax runs (threads take the heads in turn)."""
    log("[edge] reference H=256")
    w = make_config("tiny", L=0, C=256, H=256, dtype="f32")
    rp, col, d = graph(w)
    out, lse = fwd(B, w, d, "reference")
    want, want_lse = oracle_fwd(w, rp, col)
    err = rel_l2(out.cpu().numpy(), want)
    log(f"[edge] rel-L2 {err:.3e}")
    assert err <= TOL_F32
    assert np.max(np.abs(lse.cpu().numpy() - want_lse)) <= 1e-4
