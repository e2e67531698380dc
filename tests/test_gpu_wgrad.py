"""GPU weight and position gradients (e2a_attention_bwd_weights) vs the fp64
oracle's attention_weight_backward and attention_position_backward on the
same seeded inputs and cotangent.

The backward reads the forward's log-normaliser; these tests take it from
the fp32 scalar forward (except where named), so that the comparison
measures the weight-gradient kernels.  fp32 storage: relative L2 <= 1e-5 per
weight (fp32 GEMMs).  bf16 storage: <= 2e-2 (bf16 operands on the matrix
cores, fp32 sums).  The weight gradients are sums over every edge, so the
full-size workloads cannot be sampled by rows as dL/dh is; there the
cotangent is nonzero on a seeded sample of destinations only, which makes
every other edge's terms vanish, while the GPU still runs all edges (and all
batches of 65536)."""
import numpy as np
import pytest
import torch

import oracle as O
from workloads import make_config

from gpu_util import log, rel_l2, sample_dest, to_device

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2
NAMES = ("w_q", "w_k", "w_rad", "w_so2")


@pytest.fixture(scope="module")
def B():
    import so_graph_attention_amd.e2a as mod
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return mod


def setup(w, seed=77, keep=None):
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    d = to_device(w)
    d["row_ptr"] = torch.from_numpy(rp).cuda()
    d["col"] = torch.from_numpy(col).cuda()
    G = np.random.default_rng(seed).standard_normal((w.n_atoms, (w.L + 1) ** 2, w.C)).astype(np.float32)
    if keep is not None:
        G[np.setdiff1d(np.arange(w.n_atoms), keep)] = 0.0
    d["G"] = torch.from_numpy(G).cuda()
    return rp, col, d, G


def forward(B, w, d, variant="reference"):
    box = None if w.box is None else w.box.tolist()
    return B.e2a_attention_fwd(d["pos"], d["row_ptr"], d["col"], d["feat"], d["w_q"], d["w_k"], d["w_rad"],
                               d["w_so2"], L=w.L, C=w.C, H=w.H, cutoff=w.cutoff, box=box, variant=variant,
                               with_lse=True)


def gpu_wgrad(B, w, d, out, lse, variant="auto", **kw):
    box = None if w.box is None else w.box.tolist()
    res = B.e2a_attention_bwd_weights(d["pos"], d["row_ptr"], d["col"], d["feat"], d["w_q"], d["w_k"], d["w_rad"],
                                      d["w_so2"], out, lse, d["G"], L=w.L, C=w.C, H=w.H, cutoff=w.cutoff, box=box,
                                      variant=variant, **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in res.items()}


def oracle_wgrad(w, rp, col, G, centres=None):
    return O.attention_weight_backward(w.pos, rp, col, w.as_f32("feat"), w.as_f32("w_q"), w.as_f32("w_k"),
                                       w.as_f32("w_rad"), w.as_f32("w_so2"), w.L, w.C, w.H, w.cutoff, G, box=w.box,
                                       centres=centres)


def check(got, want, tol, tag):
    for name in NAMES:
        err = rel_l2(got[name].reshape(want[name].shape), want[name])
        log(f"[wgrad] {tag} {name}: rel-L2 {err:.3e}")
        assert np.all(np.isfinite(got[name])), name
        assert err <= tol, (name, err)


@pytest.mark.parametrize("L,C,H", [(0, 8, 2), (1, 16, 2), (2, 16, 2), (3, 8, 1), (4, 8, 2)])
def test_wgrad_f32_tiny_full(B, L, C, H):
    """fp32 storage, every weight of a 64-atom system; dL/dh from the same
    call equals e2a_attention_bwd's."""
    log(f"[wgrad] f32 tiny L={L} C={C} H={H}")
    w = make_config("tiny", L=L, C=C, H=H)
    rp, col, d, G = setup(w)
    out, lse = forward(B, w, d)
    got = gpu_wgrad(B, w, d, out, lse, variant="reference")
    check(got, oracle_wgrad(w, rp, col, G), TOL_F32, f"f32 L={L}")
    feat = B.e2a_attention_bwd(d["pos"], d["row_ptr"], d["col"], d["feat"], d["w_q"], d["w_k"], d["w_rad"],
                               d["w_so2"], out, lse, d["G"], L=w.L, C=w.C, H=w.H, cutoff=w.cutoff,
                               variant="reference")
    torch.cuda.synchronize()
    assert np.array_equal(got["feat"], feat.cpu().numpy())


def test_wgrad_f32_periodic_box(B):
    log("[wgrad] f32 periodic box")
    rng = np.random.default_rng(1516)
    box = np.full(3, 9.0, dtype=np.float32)
    pts = []
    while len(pts) < 90:   # random points at least 0.9 apart (minimum image)
        p = rng.random(3) * 9.0
        if all(np.linalg.norm((p - q + 4.5) % 9.0 - 4.5) >= 0.9 for q in pts):
            pts.append(p)
    pos = np.array(pts, dtype=np.float32)
    w = make_config("tiny", L=2, C=8, H=2, geometry=(pos, box, None, {}))
    rp, col, d, G = setup(w)
    out, lse = forward(B, w, d)
    got = gpu_wgrad(B, w, d, out, lse, variant="reference", feat_grad=False)
    check(got, oracle_wgrad(w, rp, col, G), TOL_F32, "f32 periodic")


@pytest.mark.parametrize("L", [1, 2, 3, 4])
def test_wgrad_bf16_tiny_full(B, L):
    """bf16 storage, C = 128, H = 8: the matrix-core GEMMs (and the
    matrix-core query pass for ds), every weight of a 64-atom system."""
    log(f"[wgrad] bf16 tiny L={L}")
    w = make_config("tiny", L=L, C=128, H=8, dtype="bf16")
    rp, col, d, G = setup(w)
    out, lse = forward(B, w, d)
    got = gpu_wgrad(B, w, d, out, lse)
    check(got, oracle_wgrad(w, rp, col, G), TOL_BF16, f"bf16 L={L}")


@pytest.mark.parametrize("L,C,H", [(2, 12, 3), (3, 24, 3)])
def test_wgrad_bf16_off_matrix_core_shapes(B, L, C, H):
    """bf16 storage with C not a multiple of 32 (the scalar layer kernels,
    the generic GEMM for y and dx, the scalar force kernel): C = 12 has
    blocks of 12 (L + 1 - m) channels, some not a multiple of 8, which must
    take the element-by-element GEMM paths; C = 24 runs the weight products
    as complex pairs with ragged tiles.  Every weight gradient and every
    position gradient against the oracle."""
    log(f"[wgrad] bf16 L={L} C={C} H={H}")
    w = make_config("tiny", L=L, C=C, H=H, dtype="bf16")
    rp, col, d, G = setup(w, seed=83)
    out, lse = forward(B, w, d)
    got = gpu_wgrad(B, w, d, out, lse, pos_grad=True)
    check(got, oracle_wgrad(w, rp, col, G), TOL_BF16, f"bf16 L={L} C={C}")
    check_pos(got["pos"], oracle_pos(w, rp, col, G), TOL_BF16, f"bf16 L={L} C={C}")


def test_wgrad_bf16_drug_sparse_cotangent(B):
    """The drug-like workload (347k edges: 6 batches), with the MFMA forward's
    log-normaliser; G nonzero on 24 sampled destinations."""
    log("[wgrad] bf16 drug, sparse cotangent")
    w = make_config("drug")
    rp0, _ = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    keep = sample_dest(rp0, 24, seed=31)
    rp, col, d, G = setup(w, keep=keep)
    out, lse = forward(B, w, d, variant="mfma")
    got = gpu_wgrad(B, w, d, out, lse, feat_grad=False)
    check(got, oracle_wgrad(w, rp, col, G, centres=keep), TOL_BF16, "bf16 drug")


def test_wgrad_deterministic_and_partial_requests(B):
    """Two calls are bit-identical, and asking for some outputs only (which
    skips the query pass when neither dL/dh nor W_q, W_k is wanted) gives the
    same values as the full call; dW_rad from the edge batches (with the
    positions) agrees with the fused kernel's radial pass."""
    log("[wgrad] determinism and partial requests")
    w = make_config("tiny", L=3, C=128, H=8, dtype="bf16")
    rp, col, d, G = setup(w)
    out, lse = forward(B, w, d)
    full = gpu_wgrad(B, w, d, out, lse)
    again = gpu_wgrad(B, w, d, out, lse)
    for name in full:
        assert np.array_equal(full[name], again[name]), name
    part = gpu_wgrad(B, w, d, out, lse, feat_grad=False, weights=("w_rad", "w_so2"))
    assert set(part) == {"w_rad", "w_so2"}
    for name in part:
        assert np.array_equal(part[name], full[name]), name
    qk = gpu_wgrad(B, w, d, out, lse, feat_grad=False, weights=("w_k",))
    assert np.array_equal(qk["w_k"], full["w_k"])
    # with the positions asked for, dW_rad still comes from the fused kernel's
    # radial pass; the scalar build takes it from the edge batches (drho from
    # y and the dyhat the gather keeps): the same gradient to the bf16 bound
    withpos = gpu_wgrad(B, w, d, out, lse, feat_grad=False, weights=("w_rad",), pos_grad=True)
    assert np.array_equal(withpos["w_rad"], full["w_rad"])
    batches = gpu_wgrad(B, w, d, out, lse, variant="reference", feat_grad=False, weights=("w_rad",),
                        pos_grad=True)
    err = rel_l2(batches["w_rad"], full["w_rad"])
    log(f"[wgrad] w_rad batches vs radial pass: rel-L2 {err:.3e}")
    assert err <= TOL_BF16


def oracle_pos(w, rp, col, G, atoms=None):
    return O.attention_position_backward(w.pos, rp, col, w.as_f32("feat"), w.as_f32("w_q"), w.as_f32("w_k"),
                                         w.as_f32("w_rad"), w.as_f32("w_so2"), w.L, w.C, w.H, w.cutoff, G,
                                         box=w.box, atoms=atoms)


def check_pos(got, want, tol, tag):
    err = rel_l2(got, want)
    log(f"[wgrad] {tag} positions: rel-L2 {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= tol, err


@pytest.mark.parametrize("L,C,H", [(0, 8, 2), (1, 8, 2), (2, 8, 2), (4, 8, 1)])
def test_pos_f32_tiny_full(B, L, C, H):
    """fp32 storage: every atom's position gradient of a 64-atom system
    against the oracle's central differences (graph held fixed)."""
    log(f"[wgrad] positions f32 tiny L={L}")
    w = make_config("tiny", L=L, C=C, H=H)
    rp, col, d, G = setup(w, seed=78)
    out, lse = forward(B, w, d)
    got = gpu_wgrad(B, w, d, out, lse, variant="reference", feat_grad=False, weights=(), pos_grad=True)
    check_pos(got["pos"], oracle_pos(w, rp, col, G), TOL_F32, f"f32 L={L}")


def test_pos_f32_periodic_box(B):
    log("[wgrad] positions f32 periodic box")
    rng = np.random.default_rng(1517)
    box = np.full(3, 9.0, dtype=np.float32)
    pts = []
    while len(pts) < 90:
        p = rng.random(3) * 9.0
        if all(np.linalg.norm((p - q + 4.5) % 9.0 - 4.5) >= 0.9 for q in pts):
            pts.append(p)
    w = make_config("tiny", L=2, C=8, H=2, geometry=(np.array(pts, dtype=np.float32), box, None, {}))
    rp, col, d, G = setup(w, seed=79)
    out, lse = forward(B, w, d)
    got = gpu_wgrad(B, w, d, out, lse, variant="reference", feat_grad=False, weights=(), pos_grad=True)
    atoms = np.arange(0, 90, 6)
    check_pos(got["pos"][atoms], oracle_pos(w, rp, col, G, atoms), TOL_F32, "f32 periodic")


@pytest.mark.parametrize("L", [2, 4])
def test_pos_bf16_tiny_sampled(B, L):
    """bf16 storage, C = 128, H = 8 (matrix-core GEMMs), on 16 atoms."""
    log(f"[wgrad] positions bf16 tiny L={L}")
    w = make_config("tiny", L=L, C=128, H=8, dtype="bf16")
    rp, col, d, G = setup(w, seed=80)
    out, lse = forward(B, w, d)
    got = gpu_wgrad(B, w, d, out, lse, feat_grad=False, weights=(), pos_grad=True)
    atoms = np.arange(0, 64, 4)
    check_pos(got["pos"][atoms], oracle_pos(w, rp, col, G, atoms), TOL_BF16, f"bf16 L={L}")


def test_pos_bf16_drug_sparse_cotangent(B):
    """The drug-like workload (all its edges and batches on the GPU) with the
    cotangent on 8 sampled destinations; the oracle's differences at those
    atoms and at one neighbour of each."""
    log("[wgrad] positions bf16 drug, sparse cotangent")
    w = make_config("drug")
    rp0, col0 = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    keep = sample_dest(rp0, 8, seed=32)
    rp, col, d, G = setup(w, keep=keep)
    out, lse = forward(B, w, d, variant="mfma")
    got = gpu_wgrad(B, w, d, out, lse, feat_grad=False, weights=("w_so2",), pos_grad=True)
    nbr = np.array([col[rp[i]] for i in keep if rp[i + 1] > rp[i]], dtype=np.int64)
    atoms = np.unique(np.concatenate([keep, nbr]))
    check_pos(got["pos"][atoms], oracle_pos(w, rp, col, G, atoms), TOL_BF16, "bf16 drug")


def test_pos_deterministic_and_with_weights(B):
    """Position gradients are bit-identical across calls and do not change
    when the weight gradients are asked for in the same call."""
    log("[wgrad] positions determinism")
    w = make_config("tiny", L=3, C=128, H=8, dtype="bf16")
    rp, col, d, G = setup(w, seed=81)
    out, lse = forward(B, w, d)
    a = gpu_wgrad(B, w, d, out, lse, feat_grad=False, weights=(), pos_grad=True)
    b = gpu_wgrad(B, w, d, out, lse, pos_grad=True)
    assert np.array_equal(a["pos"], b["pos"])
    # the scalar kernels with fp32 storage, where dW_rad comes from the edge
    # batches: the same positions with and without it
    w = make_config("tiny", L=2, C=16, H=2)
    rp, col, d, G = setup(w, seed=85)
    out, lse = forward(B, w, d)
    a = gpu_wgrad(B, w, d, out, lse, variant="reference", feat_grad=False, weights=(), pos_grad=True)
    b = gpu_wgrad(B, w, d, out, lse, variant="reference", pos_grad=True)
    c = gpu_wgrad(B, w, d, out, lse, variant="reference", pos_grad=True)
    assert np.array_equal(a["pos"], b["pos"]) and np.array_equal(b["pos"], c["pos"])


def test_wgrad_no_edges_and_isolated_atom(B):
    """Atoms farther apart than the cutoff: no edges, so every weight and
    position gradient is zero.  Then one atom set apart from a small cluster:
    its position gradient is exactly zero and the rest match the oracle."""
    log("[wgrad] no edges, isolated atom")
    far = np.array([[1.0, 1.0, 1.0], [20.0, 1.0, 1.0], [1.0, 20.0, 1.0]], dtype=np.float32)
    w = make_config("tiny", L=2, C=8, H=2, geometry=(far, None, None, {}))
    rp, col, d, G = setup(w, seed=82)
    assert col.size == 0
    out, lse = forward(B, w, d)
    got = gpu_wgrad(B, w, d, out, lse, variant="reference", pos_grad=True)
    for name, v in got.items():
        assert np.all(v == 0), name
    rng = np.random.default_rng(83)
    cluster = (rng.random((12, 3)) * 4.0).astype(np.float32)
    pos = np.concatenate([cluster, np.array([[40.0, 40.0, 40.0]], dtype=np.float32)])
    w = make_config("tiny", L=2, C=8, H=2, geometry=(pos, None, None, {}))
    rp, col, d, G = setup(w, seed=84)
    assert rp[-1] == rp[-2]   # the last atom has no neighbours
    out, lse = forward(B, w, d)
    got = gpu_wgrad(B, w, d, out, lse, variant="reference", feat_grad=False, pos_grad=True)
    assert np.all(got["pos"][-1] == 0)
    check_pos(got["pos"], oracle_pos(w, rp, col, G), TOL_F32, "f32 cluster + isolated atom")
    check(got, oracle_wgrad(w, rp, col, G), TOL_F32, "f32 cluster + isolated atom")


def oracle_feat(w, rp, col, G, dest=None):
    return O.attention_backward(w.pos, rp, col, w.as_f32("feat"), w.as_f32("w_q"), w.as_f32("w_k"),
                                w.as_f32("w_rad"), w.as_f32("w_so2"), w.L, w.C, w.H, w.cutoff, G, box=w.box,
                                dest=dest)


def check_forces_call(B, w, d, out, lse, got, want_feat, rows, tag):
    """dL/dh of a forces call (positions, no weight but W_so2): against the
    oracle on `rows`; rows l >= 1 (the value pass) equal e2a_attention_bwd's
    bit for bit, row 0 (through the softmax gradient, here formed from the
    edge batches) within the bf16 bound of it."""
    box = None if w.box is None else w.box.tolist()
    err = rel_l2(got["feat"][rows], want_feat)
    log(f"[wgrad] {tag} forces call dL/dh: rel-L2 {err:.3e} against the oracle")
    assert np.all(np.isfinite(got["feat"])) and err <= TOL_BF16, err
    ref = B.e2a_attention_bwd(d["pos"], d["row_ptr"], d["col"], d["feat"], d["w_q"], d["w_k"], d["w_rad"],
                              d["w_so2"], out, lse, d["G"], L=w.L, C=w.C, H=w.H, cutoff=w.cutoff, box=box)
    torch.cuda.synchronize()
    ref = ref.cpu().numpy()
    assert np.array_equal(got["feat"][:, 1:], ref[:, 1:])
    err0 = rel_l2(got["feat"][:, 0], ref[:, 0])
    log(f"[wgrad] {tag} forces call dL/dh row 0: rel-L2 {err0:.3e} against e2a_attention_bwd")
    assert err0 <= TOL_BF16, err0


@pytest.mark.parametrize("L", [1, 4])
def test_forces_call_softmax_gradient_from_batches(B, L):
    """dL/dh with the positions and no weight gradient (bf16, C = 128,
    H = 8): the softmax gradient comes from the batches' y and dy instead of
    a query pass.  Every atom of a 64-atom system; the positions equal those
    of the call without dL/dh, bit for bit."""
    log(f"[wgrad] forces call bf16 tiny L={L}")
    w = make_config("tiny", L=L, C=128, H=8, dtype="bf16")
    rp, col, d, G = setup(w, seed=86)
    out, lse = forward(B, w, d)
    got = gpu_wgrad(B, w, d, out, lse, weights=(), pos_grad=True)
    check_forces_call(B, w, d, out, lse, got, oracle_feat(w, rp, col, G), slice(None), f"L={L}")
    pos_only = gpu_wgrad(B, w, d, out, lse, feat_grad=False, weights=(), pos_grad=True)
    assert np.array_equal(got["pos"], pos_only["pos"])
    with_so2 = gpu_wgrad(B, w, d, out, lse, weights=("w_so2",), pos_grad=True)
    assert np.array_equal(with_so2["feat"], got["feat"]) and np.array_equal(with_so2["pos"], got["pos"])


def test_forces_call_drug_sampled(B):
    """The same on the drug-like workload (347k edges, 2 batches), with the
    MFMA forward's log-normaliser: dL/dh on 24 sampled atoms against the
    oracle."""
    log("[wgrad] forces call bf16 drug")
    w = make_config("drug")
    rp, col, d, G = setup(w, seed=87)
    out, lse = forward(B, w, d, variant="mfma")
    got = gpu_wgrad(B, w, d, out, lse, weights=(), pos_grad=True)
    dest = sample_dest(rp, 24, seed=24)
    check_forces_call(B, w, d, out, lse, got, oracle_feat(w, rp, col, G, dest), dest, "drug")
