"""e2a_attention_fwd_noalloc (the forward on the library's fixed per-GPU
scratch, for callers that cannot allocate) against e2a_attention_fwd (the
same kernels on a caller workspace): two calls in a row, the second on a
smaller system, each bit-identical to the workspace entry point; the scalar
kernel too.  Calls go through the C ABI (the ctypes binding)."""
import numpy as np
import pytest
import torch

import oracle as O
from workloads import make_config

from gpu_util import log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import so_graph_attention_amd.e2a as mod
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return mod


def _both(B, w, variant):
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    d = to_device(w)
    d["row_ptr"] = torch.from_numpy(rp).cuda()
    d["col"] = torch.from_numpy(col).cuda()
    args = (d["pos"], d["row_ptr"], d["col"], d["feat"], d["w_q"], d["w_k"], d["w_rad"], d["w_so2"])
    kw = dict(L=w.L, C=w.C, H=w.H, cutoff=w.cutoff, box=None if w.box is None else w.box.tolist(), variant=variant,
              with_lse=True)
    ref, ref_lse = B.e2a_attention_fwd(*args, **kw)
    n, K = w.n_atoms, (w.L + 1) ** 2
    out = torch.full((n, K, w.C), float("nan"), device="cuda")
    lse = torch.full((n, w.H), float("nan"), device="cuda")
    B.e2a_attention_fwd_noalloc(*args, out=out, out_lse=lse, **kw)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), ref_lse.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()


def test_noalloc_equals_workspace_entry_point_two_calls(B):
    """The drug-like batch (15,057 atoms, L = 3, C = 128, bf16; 16 MiB of
    scratch), then the 64-atom system at L = 4 (a smaller input in the same
    array, after the larger one)."""
    for name, kw in (("drug", {}), ("tiny", dict(L=4, C=128, H=8, dtype="bf16"))):
        log(f"[noalloc] {name} {kw}")
        w = make_config(name, **kw)
        ref, ref_lse, out, lse = _both(B, w, "auto")
        assert np.all(np.isfinite(out))
        assert np.array_equal(out, ref), f"{name}: max diff {np.max(np.abs(out - ref))}"
        assert np.array_equal(lse, ref_lse)


def test_noalloc_scalar_kernel(B):
    log("[noalloc] tiny fp32, scalar kernel")
    w = make_config("tiny")
    ref, ref_lse, out, lse = _both(B, w, "reference")
    assert np.array_equal(out, ref) and np.array_equal(lse, ref_lse)


def test_noalloc_rejects_oversize_and_leaves_outputs(B):
    """200,000 atoms at L = 4 need more than the fixed scratch: refused before
    anything runs, so the output buffer keeps its contents."""
    w = make_config("tiny", L=4, C=128, H=8, dtype="bf16")
    n = 200000
    pos = torch.zeros((n, 3), device="cuda")
    rp = torch.zeros(n + 1, dtype=torch.int64, device="cuda")
    col = torch.zeros(0, dtype=torch.int32, device="cuda")
    d = to_device(w)
    feat = torch.zeros((n, 25, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full((n, 25, 128), 7.0, device="cuda")
    with pytest.raises(B.E2AError, match="scratch"):
        B.e2a_attention_fwd_noalloc(pos, rp, col, feat, d["w_q"], d["w_k"], d["w_rad"], d["w_so2"], L=4, C=128,
                                    H=8, cutoff=5.0, out=out)
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))
