"""GPU fused attention vs the fp64 oracle (element by element on the same
seeded inputs).

Tolerances (relative L2 over the compared outputs): 1e-5 for fp32 storage and
for the fp32 reference kernel on bf16 inputs; 2e-2 for the bf16 MFMA kernel
(bf16 operands, fp32 accumulation).  Full-size configs run the whole layer on
the GPU and compare a seeded sample of destinations (plus the first, last,
highest- and lowest-degree atoms), which the oracle computes one by one."""
import numpy as np
import pytest
import torch

import oracle as O
from workloads import make_config
from workloads.generators import isolated_atom_variant

from gpu_util import log, oracle_out, rel_l2, sample_dest, to_device

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


@pytest.fixture(scope="module")
def B():
    import so_graph_attention_amd.e2a as mod
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return mod


_cache = {}


def setup(B, name, **kw):
    key = (name, tuple(sorted(kw.items())))
    if key not in _cache:
        w = make_config(name, **kw)
        rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
        d = to_device(w)
        d["row_ptr"] = torch.from_numpy(rp).cuda()
        d["col"] = torch.from_numpy(col).cuda()
        _cache.clear()
        _cache[key] = (w, rp, col, d)
    return _cache[key]


def run_gpu(B, w, d, variant):
    out, lse = B.e2a_attention_fwd(d["pos"], d["row_ptr"], d["col"], d["feat"], d["w_q"], d["w_k"], d["w_rad"],
                                   d["w_so2"], L=w.L, C=w.C, H=w.H, cutoff=w.cutoff,
                                   box=None if w.box is None else w.box.tolist(), variant=variant, with_lse=True)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def test_tiny_fp32_full_output(B):
    log("[attn] tiny fp32 full")
    w, rp, col, d = setup(B, "tiny")
    out, lse = run_gpu(B, w, d, "auto")
    want, want_lse = oracle_out(w, rp, col, None)
    err = rel_l2(out, want)
    log(f"[attn] tiny rel-L2 {err:.3e}")
    assert err <= TOL_F32
    assert np.max(np.abs(lse - want_lse)) <= 1e-5


@pytest.mark.parametrize("L,C,H", [(0, 8, 2), (2, 24, 3), (3, 32, 4), (4, 32, 8), (1, 160, 5)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_reference_kernel_small_shapes(B, L, C, H, dtype):
    log(f"[attn] reference tiny-geometry L={L} C={C} H={H} {dtype}")
    w, rp, col, d = setup(B, "tiny", L=L, C=C, H=H, dtype=dtype)
    out, lse = run_gpu(B, w, d, "reference")
    want, want_lse = oracle_out(w, rp, col, None)
    err = rel_l2(out, want)
    log(f"[attn] rel-L2 {err:.3e}")
    assert err <= TOL_F32
    assert np.max(np.abs(lse - want_lse)) <= 1e-4


def test_empty_rows_are_zero(B):
    log("[attn] isolated atom")
    w = isolated_atom_variant(make_config("tiny"))
    rp, col = O.neighbor_list(w.pos, w.cutoff)
    d = to_device(w)
    d["row_ptr"] = torch.from_numpy(rp).cuda()
    d["col"] = torch.from_numpy(col).cuda()
    out, lse = run_gpu(B, w, d, "auto")
    assert np.all(out[-1] == 0) and np.all(np.isneginf(lse[-1]))
    want, _ = oracle_out(w, rp, col, None)
    assert rel_l2(out, want) <= TOL_F32


@pytest.mark.parametrize("name", ["drug", "water"])
def test_reference_kernel_bf16_configs_sampled(B, name):
    log(f"[attn] reference {name}")
    w, rp, col, d = setup(B, name)
    out, _ = run_gpu(B, w, d, "reference")
    dest = sample_dest(rp, 48, seed=7)
    want, _ = oracle_out(w, rp, col, dest)
    err = rel_l2(out[dest], want)
    log(f"[attn] reference {name} rel-L2 {err:.3e} on {dest.size} atoms")
    assert err <= TOL_F32


@pytest.mark.parametrize("L", [1, 2, 3, 4])
def test_mfma_kernel_tiny_geometry_full_output(B, L):
    """C = 128, H = 8, bf16: every output of a 64-atom system (rows of 11-36
    neighbours: one or two 32-edge chunks with ragged tails)."""
    log(f"[attn] mfma tiny-geometry L={L}")
    w, rp, col, d = setup(B, "tiny", L=L, C=128, H=8, dtype="bf16")
    out, lse = run_gpu(B, w, d, "mfma")
    want, want_lse = oracle_out(w, rp, col, None)
    err = rel_l2(out, want)
    log(f"[attn] mfma L={L} rel-L2 {err:.3e}")
    assert np.all(np.isfinite(out))
    assert err <= TOL_BF16
    assert np.max(np.abs(lse - want_lse)) <= 1e-4


@pytest.mark.parametrize("name", ["drug", "drug_origin", "water", "protein", "large"])
def test_mfma_kernel_full_configs_sampled(B, name):
    log(f"[attn] mfma {name}")
    w, rp, col, d = setup(B, name)
    out, lse = run_gpu(B, w, d, "auto")
    assert np.all(np.isfinite(out))
    dest = sample_dest(rp, 64, seed=11)
    want, want_lse = oracle_out(w, rp, col, dest)
    err = rel_l2(out[dest], want)
    log(f"[attn] mfma {name} rel-L2 {err:.3e} on {dest.size} atoms")
    assert err <= TOL_BF16
    assert np.max(np.abs(lse[dest] - want_lse)) <= 1e-4


def cluster_geometry(sizes, cutoff, seed):
    """Separated tight clusters: every atom of a cluster of size g has exactly
    g - 1 neighbours (all pairs closer than the cutoff, clusters 3 cutoffs
    apart), so the degrees of the system are chosen directly."""
    rng = np.random.default_rng(seed)
    pos = []
    for c, g in enumerate(sizes):
        centre = np.array([3.0 * cutoff * c, 0.5 * cutoff * (c % 3), 0.0])
        v = rng.normal(size=(g, 3))
        v *= (cutoff / 3.2) * rng.random((g, 1)) ** (1 / 3) / np.linalg.norm(v, axis=1, keepdims=True)
        pos.append(centre + v)
    pos = np.concatenate(pos).astype(np.float32)
    return pos, None, None, {"clusters": list(sizes)}


@pytest.mark.parametrize("L", [1, 4])
def test_mfma_kernel_chunk_packing_degrees(B, L):
    """Degrees 0 (several isolated atoms in a row), 1, 2, 4, 8, 16, 31, 32,
    33 and 64: chunks that end inside an atom, hold two atoms, finish both,
    or are filled exactly; every output compared."""
    sizes = [1, 1, 1, 2, 3, 5, 9, 17, 1, 32, 33, 34, 2, 65, 1]
    cutoff = float(np.float32(5.0))
    geom = cluster_geometry(sizes, cutoff, seed=21)
    w = make_config("tiny", L=L, C=128, H=8, dtype="bf16", geometry=geom)
    w.cutoff = cutoff
    log(f"[attn] mfma chunk packing L={L}: {w.n_atoms} atoms")
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    deg = np.diff(rp)
    assert sorted(set(deg.tolist())) == sorted({g - 1 for g in sizes})
    d = to_device(w)
    d["row_ptr"] = torch.from_numpy(rp).cuda()
    d["col"] = torch.from_numpy(col).cuda()
    out, lse = run_gpu(B, w, d, "mfma")
    want, want_lse = oracle_out(w, rp, col, None)
    assert np.all(np.isfinite(out))
    iso = deg == 0
    assert np.all(out[iso] == 0) and np.all(np.isneginf(lse[iso]))
    err = rel_l2(out, want)
    log(f"[attn] mfma chunk packing L={L} rel-L2 {err:.3e}")
    assert err <= TOL_BF16
    assert np.max(np.abs(lse[~iso] - want_lse[~iso])) <= 1e-4


def test_mfma_kernel_balanced_deal_full_output(B):
    """A system whose mean degree is above the 32-edge chunk (clusters of 33
    to 60 atoms), so destinations are dealt to workgroups by degree in
    rounds: several rounds, both directions and a ragged last round.  Every
    output is compared with the oracle, and a second launch must agree bit
    for bit."""
    rng = np.random.default_rng(5)
    sizes = [int(g) for g in rng.integers(33, 61, size=20)]
    cutoff = float(np.float32(5.0))
    geom = cluster_geometry(sizes, cutoff, seed=23)
    w = make_config("tiny", L=4, C=128, H=8, dtype="bf16", geometry=geom)
    w.cutoff = cutoff
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    assert col.size >= 32 * w.n_atoms
    log(f"[attn] mfma balanced deal: {w.n_atoms} atoms, {col.size} edges")
    d = to_device(w)
    d["row_ptr"] = torch.from_numpy(rp).cuda()
    d["col"] = torch.from_numpy(col).cuda()
    out, lse = run_gpu(B, w, d, "mfma")
    out2, lse2 = run_gpu(B, w, d, "mfma")
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    want, want_lse = oracle_out(w, rp, col, None)
    err = rel_l2(out, want)
    log(f"[attn] mfma balanced deal rel-L2 {err:.3e}")
    assert np.all(np.isfinite(out))
    assert err <= TOL_BF16
    assert np.max(np.abs(lse - want_lse)) <= 1e-4


@pytest.mark.parametrize("name", ["drug", "protein"])
def test_mfma_kernel_is_deterministic(B, name):
    """Two launches on the same inputs give bit-identical outputs: the spatial
    order of destinations (which decides how atoms share edge chunks, and so
    the fp32 summation order) must not depend on timing."""
    log(f"[attn] mfma determinism {name}")
    w, rp, col, d = setup(B, name)
    out0, lse0 = run_gpu(B, w, d, "auto")
    out1, lse1 = run_gpu(B, w, d, "auto")
    assert np.array_equal(out0, out1)
    assert np.array_equal(lse0, lse1)


def test_mfma_kernel_graph_capture_replays(B):
    """The layer enqueues only kernels (no memset/copy nodes, no host sync),
    so it can be recorded into a HIP graph.  Three replays, with eager work
    and synchronisation between them, each match the eager result bitwise."""
    log("[attn] mfma graph capture, drug")
    w, rp, col, d = setup(B, "drug")
    n, K = w.n_atoms, (w.L + 1) ** 2
    args = (d["pos"], d["row_ptr"], d["col"], d["feat"], d["w_q"], d["w_k"], d["w_rad"], d["w_so2"])
    kw = dict(L=w.L, C=w.C, H=w.H, cutoff=w.cutoff, box=None if w.box is None else w.box.tolist())
    eager, eager_lse = B.e2a_attention_fwd(*args, **kw, with_lse=True)
    torch.cuda.synchronize()
    eager, eager_lse = eager.cpu().numpy(), eager_lse.cpu().numpy()
    out = torch.empty((n, K, w.C), dtype=torch.float32, device="cuda")
    lse = torch.empty((n, w.H), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.e2a_attention_workspace_bytes(n, w.L, w.C, w.H, B.E2A_DTYPE_BF16), dtype=torch.uint8,
                     device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on the capture stream
        B.e2a_attention_fwd(*args, **kw, out=out, out_lse=lse, workspace=ws, with_lse=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.e2a_attention_fwd(*args, **kw, out=out, out_lse=lse, workspace=ws, with_lse=True)
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager), f"replay {rep}"
        assert np.array_equal(lse.cpu().numpy(), eager_lse), f"replay {rep}"


def test_mfma_kernel_long_rows(B):
    """Destinations with 300 neighbours (about ten 32-edge chunks each),
    L = 1, sampled destinations against the oracle."""
    from test_gpu_neighbors import dense_cluster
    log("[attn] mfma long rows")
    geom = (dense_cluster(300, seed=5), None, None, {"cluster": 300})
    w = make_config("tiny", L=1, C=128, H=8, dtype="bf16", geometry=geom)
    w.cutoff = float(np.float32(5.0))
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    d = to_device(w)
    d["row_ptr"] = torch.from_numpy(rp).cuda()
    d["col"] = torch.from_numpy(col).cuda()
    out, lse = run_gpu(B, w, d, "mfma")
    dest = np.array([0, 1, 77, 150, 299, 300, 301, 320, 340])
    want, want_lse = oracle_out(w, rp, col, dest)
    err = rel_l2(out[dest], want)
    log(f"[attn] mfma long rows rel-L2 {err:.3e}")
    assert np.all(np.isfinite(out))
    assert err <= TOL_BF16
    iso = np.diff(rp)[dest] == 0
    assert np.all(np.isneginf(lse[dest][iso])) and np.all(np.isneginf(want_lse[iso]))
    assert np.max(np.abs(lse[dest][~iso] - want_lse[~iso])) <= 1e-4


def test_mfma_kernel_rows_at_the_limit(B):
    """Destinations with 4096 neighbours (the neighbour build's maximum row,
    128 full 32-edge chunks each), L = 1; sampled destinations against the
    oracle, attention and convolution."""
    from test_gpu_neighbors import dense_cluster
    log("[attn] mfma rows of 4096")
    geom = (dense_cluster(4096, seed=43), None, None, {"cluster": 4096})
    w = make_config("tiny", L=1, C=128, H=8, dtype="bf16", geometry=geom)
    w.cutoff = float(np.float32(5.0))
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    assert np.diff(rp).max() == 4096
    d = to_device(w)
    d["row_ptr"] = torch.from_numpy(rp).cuda()
    d["col"] = torch.from_numpy(col).cuda()
    out, lse = run_gpu(B, w, d, "mfma")
    dest = np.array([0, 2048, 4096, 4097, 4120])
    want, want_lse = oracle_out(w, rp, col, dest)
    err = rel_l2(out[dest], want)
    log(f"[attn] mfma 4096-row rel-L2 {err:.3e}")
    assert np.all(np.isfinite(out))
    assert err <= TOL_BF16
    iso = np.diff(rp)[dest] == 0
    assert np.max(np.abs(lse[dest][~iso] - want_lse[~iso])) <= 1e-4
    conv = B.e2a_conv_fwd(d["pos"], d["row_ptr"], d["col"], d["feat"], d["w_rad"], d["w_so2"], L=w.L, C=w.C,
                          H=w.H, cutoff=w.cutoff, variant="mfma")
    torch.cuda.synchronize()
    cwant = O.convolution(w.pos, rp, col, w.as_f32("feat"), w.as_f32("w_rad"), w.as_f32("w_so2"), w.L, w.C,
                          w.cutoff, dest=dest)
    cerr = rel_l2(conv.cpu().numpy()[dest], cwant)
    log(f"[conv] mfma 4096-row rel-L2 {cerr:.3e}")
    assert cerr <= TOL_BF16
