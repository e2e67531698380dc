"""GPU block around the layer (e2a_block_fwd: Norm1, the fused layer,
projection and residual, Norm2, gated FFN and residual) against the oracle's
``block`` on the same seeded inputs and weights; two stacked blocks against
the oracle's composition.

Tolerances: 1e-5 relative L2 for fp32 storage (scalar kernels, fp32 GEMMs),
2e-2 for bf16 storage (the norm outputs and gated activations are stored in
bf16, the products take bf16 operands on the matrix cores, sums are fp32)."""
import numpy as np
import pytest
import torch

import oracle as O
from workloads import block_weights_f32, make_block_weights, make_config
from workloads.generators import isolated_atom_variant

from gpu_util import log, rel_l2, sample_dest, stored_tensor, to_device

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


@pytest.fixture(scope="module")
def B():
    import so_graph_attention_amd.e2a as mod
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return mod


def bw_device(bw):
    out = {}
    for k, v in bw.items():
        if v.dtype == np.uint16:
            out[k] = torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).cuda()
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).cuda()
    return out


def setup(w):
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    d = to_device(w)
    d["row_ptr"] = torch.from_numpy(rp).cuda()
    d["col"] = torch.from_numpy(col).cuda()
    h = w.as_f32("feat")
    d["h"] = torch.from_numpy(np.ascontiguousarray(h)).cuda()
    return rp, col, d, h


def gpu_block(B, w, d, h_dev, bwd, variant="auto"):
    out = B.e2a_block_fwd(d["pos"], d["row_ptr"], d["col"], h_dev, bwd, L=w.L, C=w.C, H=w.H, cutoff=w.cutoff,
                          box=None if w.box is None else w.box.tolist(), variant=variant)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("L,C,H,dtype,variant,tol", [
    (1, 16, 1, "f32", "auto", TOL_F32), (0, 8, 2, "f32", "auto", TOL_F32), (3, 16, 2, "f32", "auto", TOL_F32),
    (2, 24, 3, "bf16", "reference", TOL_BF16), (1, 128, 8, "bf16", "mfma", TOL_BF16),
    (4, 128, 8, "bf16", "mfma", TOL_BF16),
    # degree 0 only on the matrix-core GEMMs (the gate is SiLU alone), and
    # bf16 with C above the matrix-core GEMM's 128 (fp32 node-wise products)
    (0, 32, 2, "bf16", "auto", TOL_BF16), (1, 160, 5, "bf16", "reference", TOL_BF16)])
def test_block_tiny_full(B, L, C, H, dtype, variant, tol):
    log(f"[block] tiny L={L} C={C} H={H} {dtype} {variant}")
    w = isolated_atom_variant(make_config("tiny", L=L, C=C, H=H, dtype=dtype))
    rp, col, d, h = setup(w)
    bw = make_block_weights(w)
    got = gpu_block(B, w, d, d["h"], bw_device(bw), variant).cpu().numpy()
    want = O.block(w.pos, rp, col, h, block_weights_f32(bw), L, C, H, w.cutoff)
    err = rel_l2(got, want)
    log(f"[block] rel-L2 {err:.3e}")
    assert err <= tol
    # the atom without neighbours: its attention output is zero, the rest runs
    assert rel_l2(got[-1], want[-1]) <= tol


@pytest.mark.parametrize("name", ["drug", "large"])
def test_block_workload_sampled(B, name):
    log(f"[block] {name} sampled")
    w = make_config(name)
    rp, col, d, h = setup(w)
    bw = make_block_weights(w)
    got = gpu_block(B, w, d, d["h"], bw_device(bw)).cpu().numpy()
    dest = sample_dest(rp, 48, 31)
    want = O.block(w.pos, rp, col, h, block_weights_f32(bw), w.L, w.C, w.H, w.cutoff, box=w.box, dest=dest)
    err = rel_l2(got[dest], want)
    log(f"[block] rel-L2 {err:.3e} on {dest.size} atoms")
    assert err <= TOL_BF16


@pytest.mark.parametrize("name,kw,tol", [("tiny", dict(L=2, C=16, H=2, dtype="f32"), TOL_F32),
                                         ("tiny", dict(L=3, C=128, H=8, dtype="bf16"), TOL_BF16)])
def test_two_stacked_blocks(B, name, kw, tol):
    """Two blocks with their own weights (block 1 draws its own attention
    weights), the second reading the first's output in place."""
    log(f"[block] two blocks {name} {kw}")
    w = make_config(name, **kw)
    rp, col, d, h = setup(w)
    bws = [make_block_weights(w, i) for i in range(2)]
    x = d["h"].clone()
    for bw in bws:
        out = B.e2a_block_fwd(d["pos"], d["row_ptr"], d["col"], x, bw_device(bw), L=w.L, C=w.C, H=w.H,
                              cutoff=w.cutoff, out=x)
    torch.cuda.synchronize()
    want = h.astype(np.float64)
    for bw in bws:
        want = O.block(w.pos, rp, col, want, block_weights_f32(bw), w.L, w.C, w.H, w.cutoff)
    err = rel_l2(out.cpu().numpy(), want)
    log(f"[block] rel-L2 {err:.3e}")
    assert err <= tol


def test_block_deterministic_and_residual_identity(B):
    """Two calls give bit-identical outputs; zero output weights (W_o, W_2)
    return the input bit for bit."""
    w = make_config("tiny", L=2, C=128, H=8, dtype="bf16")
    rp, col, d, h = setup(w)
    bw = bw_device(make_block_weights(w))
    a = gpu_block(B, w, d, d["h"], bw)
    b = gpu_block(B, w, d, d["h"], bw)
    assert torch.equal(a, b)
    z = dict(bw)
    z["w_o"] = torch.zeros_like(bw["w_o"])
    z["w_2"] = torch.zeros_like(bw["w_2"])
    assert torch.equal(gpu_block(B, w, d, d["h"], z), d["h"])


def test_block_norm2_gamma_off_16_bytes(B):
    """Norm2's gains at an address off the 16-byte boundary: the separate
    norm pass runs instead of the norm folded into the products that read
    Norm2(h1); both agree with the oracle."""
    w = make_config("tiny", L=2, C=128, H=8, dtype="bf16")
    rp, col, d, h = setup(w)
    bwh = make_block_weights(w)
    bw = bw_device(bwh)
    g = bw["norm2"].reshape(-1)
    buf = torch.zeros(g.numel() + 8, dtype=g.dtype, device=g.device)
    buf[1:1 + g.numel()] = g
    off = dict(bw)
    off["norm2"] = buf[1:1 + g.numel()].view(bw["norm2"].shape)
    assert off["norm2"].data_ptr() % 16 != 0
    want = O.block(w.pos, rp, col, h, block_weights_f32(bwh), w.L, w.C, w.H, w.cutoff)
    for weights in (bw, off):
        got = gpu_block(B, w, d, d["h"], weights).cpu().numpy()
        err = rel_l2(got, want)
        log(f"[block] norm2 at {weights['norm2'].data_ptr() % 16} bytes past 16: rel-L2 {err:.3e}")
        assert err <= TOL_BF16


def test_block_graph_capture_replays(B):
    """The block enqueues only kernels (no memset or copy nodes, no host
    sync), so it records into a HIP graph.  Three replays, with eager work
    and synchronisation between them, each equal the eager result bitwise."""
    log("[block] graph capture, drug")
    w = make_config("drug")
    rp, col, d, h = setup(w)
    bw = bw_device(make_block_weights(w))
    eager = gpu_block(B, w, d, d["h"], bw).cpu().numpy()
    out = torch.empty_like(d["h"])
    ws = torch.empty(B.e2a_block_workspace_bytes(w.n_atoms, w.L, w.C, w.H, B.E2A_DTYPE_BF16), dtype=torch.uint8,
                     device="cuda")
    kw = dict(L=w.L, C=w.C, H=w.H, cutoff=w.cutoff, box=None if w.box is None else w.box.tolist(), out=out,
              workspace=ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on the capture stream
        B.e2a_block_fwd(d["pos"], d["row_ptr"], d["col"], d["h"], bw, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.e2a_block_fwd(d["pos"], d["row_ptr"], d["col"], d["h"], bw, **kw)
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager), f"replay {rep}"
