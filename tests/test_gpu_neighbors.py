"""GPU neighbour build vs the oracle's fp32 radius graph: bit-exact CSR."""
import numpy as np
import pytest
import torch

import oracle as O
from workloads import make_config
from workloads.generators import isolated_atom_variant

from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import so_graph_attention_amd.e2a as mod
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return mod


def gpu_csr(B, w, **kw):
    pos = torch.from_numpy(np.ascontiguousarray(w.pos)).cuda()
    batch = None if w.batch is None else torch.from_numpy(w.batch.astype(np.int32)).cuda()
    rp, col = B.e2a_build_neighbors(pos, w.cutoff, box=None if w.box is None else w.box.tolist(), batch=batch, **kw)
    torch.cuda.synchronize()
    return rp.cpu().numpy(), col.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "drug", "drug_origin", "water", "protein", "large"])
def test_neighbors_bit_exact(B, name):
    log(f"[neighbors] {name}")
    w = make_config(name, C=4, H=1, L=0)
    rp_o, col_o = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    rp_g, col_g = gpu_csr(B, w)
    log(f"[neighbors] {name}: E oracle {col_o.size} gpu {col_g.size}")
    assert np.array_equal(rp_g, rp_o)
    assert np.array_equal(col_g, col_o)


def test_neighbors_capacity_retry(B):
    log("[neighbors] capacity")
    w = make_config("tiny", C=4, H=1, L=0)
    rp_o, col_o = O.neighbor_list(w.pos, w.cutoff)
    pos = torch.from_numpy(w.pos).cuda()
    with pytest.raises(B.E2AError) as ei:
        B.e2a_build_neighbors(pos, w.cutoff, capacity=10)
    assert ei.value.status == B.E2A_ERR_CAPACITY
    rp, col = B.e2a_build_neighbors(pos, w.cutoff)   # binding retries with the reported count
    assert np.array_equal(col.cpu().numpy(), col_o)


def test_neighbors_edge_cases(B):
    log("[neighbors] edge cases")
    # empty system
    rp, col = B.e2a_build_neighbors(torch.zeros((0, 3), device="cuda"), 5.0)
    assert rp.cpu().tolist() == [0] and col.numel() == 0
    # one atom, and an isolated atom
    rp, col = B.e2a_build_neighbors(torch.zeros((1, 3), device="cuda"), 5.0)
    assert rp.cpu().tolist() == [0, 0]
    w = isolated_atom_variant(make_config("tiny", C=4, H=1, L=0))
    rp_o, col_o = O.neighbor_list(w.pos, w.cutoff)
    rp_g, col_g = gpu_csr(B, w)
    assert np.array_equal(rp_g, rp_o) and np.array_equal(col_g, col_o) and rp_g[-1] == rp_g[-2]
    # periodic coordinate outside [0, box)
    pos = torch.tensor([[1.0, 1.0, 1.0], [25.0, 1.0, 1.0]], device="cuda")
    with pytest.raises(B.E2AError) as ei:
        B.e2a_build_neighbors(pos, 5.0, box=[20.0, 20.0, 20.0])
    assert ei.value.status == B.E2A_ERR_INVALID_ARG
    with pytest.raises(B.E2AError) as ei:
        B.e2a_build_neighbors(pos, 5.0, box=[9.0, 40.0, 40.0])
    assert ei.value.status == B.E2A_ERR_BOX_TOO_SMALL
    # non-finite coordinate
    pos = torch.tensor([[1.0, float("nan"), 1.0], [2.0, 1.0, 1.0]], device="cuda")
    with pytest.raises(B.E2AError):
        B.e2a_build_neighbors(pos, 5.0)
    # a periodic box checks its coordinates with the edge count (one wait on
    # the device): non-finite, negative and too-large coordinates are refused
    # there, and the next call is unaffected
    for bad in ([[1.0, float("nan"), 1.0], [2.0, 1.0, 1.0]], [[1.0, -0.5, 1.0], [2.0, 1.0, 1.0]],
                [[1.0, 1.0, 1.0], [2.0, 1.0, float("inf")]]):
        with pytest.raises(B.E2AError) as ei:
            B.e2a_build_neighbors(torch.tensor(bad, device="cuda"), 5.0, box=[20.0, 20.0, 20.0])
        assert ei.value.status == B.E2A_ERR_INVALID_ARG
    rp, col = B.e2a_build_neighbors(torch.tensor([[1.0, 1.0, 1.0], [19.0, 1.0, 1.0]], device="cuda"), 5.0,
                                    box=[20.0, 20.0, 20.0])
    assert rp.cpu().tolist() == [0, 1, 2] and col.cpu().tolist() == [1, 0]


def test_neighbors_open_grid_extreme_extent(B):
    """Open boundaries size the cell grid on the device: an extent of 1e7
    cutoffs is clamped before the integer conversion and the grid coarsened
    to the workspace's cells; the one close pair is still found, bit-exact
    against the oracle."""
    pos = np.array([[0.0, 0.0, 0.0], [1.5, 0.5, -0.5], [5.0e7, 0.0, 0.0], [-5.0e7, 3.0e7, 1.0e7],
                    [2.0e7, -4.0e7, 2.5e7]], dtype=np.float32)
    rp_o, col_o = O.neighbor_list_bruteforce(pos, 5.0)
    rp, col = B.e2a_build_neighbors(torch.from_numpy(pos).cuda(), 5.0)
    assert np.array_equal(rp.cpu().numpy(), rp_o) and np.array_equal(col.cpu().numpy(), col_o)
    assert rp.cpu().tolist() == [0, 1, 2, 2, 2, 2]


@pytest.mark.parametrize("side", [10.5, 14.0, 16.0])
def test_neighbors_small_periodic_boxes(B, side):
    """Boxes of 2-3 cutoffs give 1 or 2 cells per axis: the stencil must not
    visit a cell twice."""
    log(f"[neighbors] small box {side}")
    rng = np.random.default_rng(int(side * 10))
    n = int(0.1 * side ** 3)
    pos = rng.uniform(0, side, (n, 3)).astype(np.float32)
    pos[pos >= np.float32(side)] = 0
    box = np.full(3, side, dtype=np.float32)
    rp_o, col_o = O.neighbor_list_bruteforce(pos, 5.0, box)
    rp, col = B.e2a_build_neighbors(torch.from_numpy(pos).cuda(), 5.0, box=box.tolist())
    assert np.array_equal(rp.cpu().numpy(), rp_o) and np.array_equal(col.cpu().numpy(), col_o)


def dense_cluster(deg, seed):
    """deg + 1 atoms within a ball of radius 2.4 A (every pair closer than a
    5 A cutoff: each has exactly deg neighbours) plus 40 atoms far away."""
    rng = np.random.default_rng(seed)
    v = rng.normal(size=(deg + 1, 3))
    v *= 2.4 * rng.random((deg + 1, 1)) ** (1 / 3) / np.linalg.norm(v, axis=1, keepdims=True)
    far = rng.uniform(0, 60, (40, 3)) + np.array([30.0, 0.0, 0.0])
    return np.concatenate([v + 10.0, far]).astype(np.float32)


@pytest.mark.parametrize("deg", [256, 300])
def test_neighbors_long_rows(B, deg):
    """Rows of exactly 256 fill the per-wave row buffer of the fast fill;
    longer rows take the LDS bitonic path."""
    log(f"[neighbors] long rows {deg}")
    pos = dense_cluster(deg, seed=deg)
    rp_o, col_o = O.neighbor_list(pos, 5.0)
    assert np.diff(rp_o).max() == deg
    rp, col = B.e2a_build_neighbors(torch.from_numpy(pos).cuda(), 5.0)
    assert np.array_equal(rp.cpu().numpy(), rp_o) and np.array_equal(col.cpu().numpy(), col_o)


def test_neighbors_row_limit(B):
    """4096 neighbours, the documented maximum, fill the general path's LDS
    sort buffer exactly and come out bit-exact; 4097 are refused with
    E2A_ERR_UNSUPPORTED (from the count pass, before any row is filled)."""
    log("[neighbors] row limit 4096 / 4097")
    pos = dense_cluster(4096, seed=41)
    rp_o, col_o = O.neighbor_list(pos, 5.0)
    assert np.diff(rp_o).max() == 4096
    rp, col = B.e2a_build_neighbors(torch.from_numpy(pos).cuda(), 5.0)
    assert np.array_equal(rp.cpu().numpy(), rp_o) and np.array_equal(col.cpu().numpy(), col_o)
    pos = dense_cluster(4097, seed=42)
    with pytest.raises(B.E2AError) as ei:
        B.e2a_build_neighbors(torch.from_numpy(pos).cuda(), 5.0)
    assert ei.value.status == B.E2A_ERR_UNSUPPORTED
