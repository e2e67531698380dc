"""Pins of the oracle's block around the layer (CPU only): the per-degree
norm against PyTorch's RMS norm, the scalar path of the gated FFN against
PyTorch's SiLU, and the block's rotation equivariance, permutation
equivariance, residual identity at zero output weights, and invariance of
the norm's statistics under rotation.  The pages print none of the block;
these are the facts its reading must satisfy."""
import numpy as np
import pytest
import torch

import oracle as O
from workloads import block_weights_f32, make_block_weights, make_config

from test_oracle_pins import random_rotation


def rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300)


@pytest.fixture(scope="module")
def small():
    w = make_config("tiny", L=2, C=8, H=2, dtype="f32")
    rp, col = O.neighbor_list(w.pos, w.cutoff)
    bw = block_weights_f32(make_block_weights(w))
    return w, rp, col, bw


def test_degree_norm_equals_library_rms_norm():
    """Each degree's (2l+1) x C block normalised as one vector by
    torch.nn.functional.rms_norm, with the gain repeated over m."""
    rng = np.random.default_rng(1)
    L, C = 3, 5
    h = rng.standard_normal((7, (L + 1) ** 2, C)) * rng.uniform(0.01, 100, size=(7, 1, 1))
    g = rng.standard_normal((L + 1, C))
    got = O.degree_rms_norm(h, g, L)
    for l in range(L + 1):
        blk = torch.from_numpy(h[:, l * l:(l + 1) ** 2, :].reshape(7, -1))
        wt = torch.from_numpy(np.tile(g[l], 2 * l + 1))
        want = torch.nn.functional.rms_norm(blk, (blk.shape[1],), weight=wt, eps=O.NORM_EPS).numpy()
        assert rel(got[:, l * l:(l + 1) ** 2, :].reshape(7, -1), want) < 1e-13, l


def test_degree_norm_rotation_and_scale():
    """The per-degree statistics do not change under a rotation (so the norm
    commutes with D(R)); scaling a degree by s > 0 leaves it unchanged up to
    eps."""
    rng = np.random.default_rng(2)
    L, C = 3, 4
    h = rng.standard_normal((5, (L + 1) ** 2, C))
    g = rng.standard_normal((L + 1, C))
    R = random_rotation(rng)
    Dh = np.empty_like(h)
    for l in range(L + 1):
        Dh[:, l * l:(l + 1) ** 2, :] = np.einsum("mn,anc->amc", O.wigner_d(l, R), h[:, l * l:(l + 1) ** 2, :])
    a = O.degree_rms_norm(Dh, g, L)
    b = O.degree_rms_norm(h, g, L)
    for l in range(L + 1):
        Db = np.einsum("mn,anc->amc", O.wigner_d(l, R), b[:, l * l:(l + 1) ** 2, :])
        assert rel(a[:, l * l:(l + 1) ** 2, :], Db) < 1e-13
    # only eps breaks scale invariance: its relative weight is eps / mean(h^2)
    assert rel(O.degree_rms_norm(1e3 * h, g, L), b) < 2 * O.NORM_EPS / np.min(np.mean(h * h, axis=(1, 2)))
    assert rel(O.degree_rms_norm(1e3 * h, g, L), O.degree_rms_norm(1e6 * h, g, L)) < 1e-12


def test_gated_ffn_scalar_path_is_silu_mlp():
    """With only scalars (l >= 1 zero) the FFN is SiLU(n0 W1[0]) W2[0] on l = 0
    (torch's SiLU) and exactly zero on every l >= 1."""
    rng = np.random.default_rng(3)
    L, C = 2, 6
    n = np.zeros((4, (L + 1) ** 2, C))
    n[:, 0, :] = rng.standard_normal((4, C))
    w1 = rng.standard_normal((L + 1, C, C))
    w2 = rng.standard_normal((L + 1, C, C))
    wg = rng.standard_normal((C, L * C))
    f = O.gated_ffn(n, w1, wg, w2, L, C)
    want = torch.nn.functional.silu(torch.from_numpy(n[:, 0, :] @ w1[0])).numpy() @ w2[0]
    assert rel(f[:, 0, :], want) < 1e-13
    assert np.all(f[:, 1:, :] == 0.0)


def test_gated_ffn_gate_saturation():
    """A gate logit of +1e3 passes u through (sigmoid = 1 in fp64), -1e3 blocks it."""
    rng = np.random.default_rng(4)
    L, C = 1, 3
    n = rng.standard_normal((2, 4, C))
    w1 = rng.standard_normal((2, C, C))
    w2 = rng.standard_normal((2, C, C))
    n[:, 0, :] = 1.0
    wg = np.full((C, C), 1e3)
    f_open = O.gated_ffn(n, w1, wg, w2, L, C)
    assert rel(f_open[:, 1:, :], (n[:, 1:, :] @ w1[1]) @ w2[1]) < 1e-13
    f_shut = O.gated_ffn(n, w1, -wg, w2, L, C)
    assert np.max(np.abs(f_shut[:, 1:, :])) < 1e-300


def test_block_rotation_equivariance(small):
    """block(R x + t, D(R) h) = D(R) block(x, h) on an open system."""
    w, rp, col, bw = small
    rng = np.random.default_rng(5)
    h = w.as_f32("feat").astype(np.float64)
    R = random_rotation(rng)
    t = rng.standard_normal(3)
    pos2 = w.pos.astype(np.float64) @ R.T + t
    Dh = np.empty_like(h)
    for l in range(w.L + 1):
        Dh[:, l * l:(l + 1) ** 2, :] = np.einsum("mn,anc->amc", O.wigner_d(l, R), h[:, l * l:(l + 1) ** 2, :])
    a = O.block(pos2, rp, col, Dh, bw, w.L, w.C, w.H, w.cutoff)
    b = O.block(w.pos, rp, col, h, bw, w.L, w.C, w.H, w.cutoff)
    Db = np.empty_like(b)
    for l in range(w.L + 1):
        Db[:, l * l:(l + 1) ** 2, :] = np.einsum("mn,anc->amc", O.wigner_d(l, R), b[:, l * l:(l + 1) ** 2, :])
    assert rel(a, Db) < 1e-11


def test_block_permutation(small):
    w, rp, col, bw = small
    rng = np.random.default_rng(6)
    perm = rng.permutation(w.n_atoms)
    inv = np.argsort(perm)
    pos2 = w.pos[perm]
    h = w.as_f32("feat").astype(np.float64)
    rp2, col2 = O.neighbor_list(pos2, w.cutoff)
    a = O.block(pos2, rp2, col2, h[perm], bw, w.L, w.C, w.H, w.cutoff)
    b = O.block(w.pos, rp, col, h, bw, w.L, w.C, w.H, w.cutoff)
    assert rel(a[inv], b) < 1e-12


def test_block_residual_identity_at_zero_weights(small):
    """W_o = 0 and W_2 = 0: both residual branches vanish and the block returns
    its input exactly."""
    w, rp, col, bw = small
    z = dict(bw)
    z["w_o"] = np.zeros_like(bw["w_o"])
    z["w_2"] = np.zeros_like(bw["w_2"])
    h = w.as_f32("feat").astype(np.float64)
    assert np.array_equal(O.block(w.pos, rp, col, h, z, w.L, w.C, w.H, w.cutoff), h)


def test_block_dest_subset_equals_full(small):
    w, rp, col, bw = small
    h = w.as_f32("feat").astype(np.float64)
    full = O.block(w.pos, rp, col, h, bw, w.L, w.C, w.H, w.cutoff)
    dest = np.array([3, 17, 40, 63])
    assert rel(O.block(w.pos, rp, col, h, bw, w.L, w.C, w.H, w.cutoff, dest=dest), full[dest]) < 1e-14
