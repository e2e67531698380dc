"""CPU-side checks of the C ABI: the library loads, exports what include/e2a.h
declares, and rejects invalid calls on the host before touching a device.
Also checks the host build of the per-edge geometry routines (edge rotation,
Ivanic-Ruedenberg Wigner-D recursion, radial basis) against the oracle."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle as O
import so_graph_attention_amd.e2a as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "e2a.h")


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(e2a_[a-z0-9_]+)\s*\(", txt)))


def test_header_declarations_are_exported():
    names = declared_functions()
    assert set(names) == set(B.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", B.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT\s+(e2a_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(B.lib(), n)


def test_version_and_status_strings():
    assert B.e2a_version() == 2
    assert B.status_string(0) == "E2A_OK"
    assert B.status_string(2) == "E2A_ERR_CAPACITY"
    assert B.status_string(99) == "E2A_ERR_UNKNOWN"


def test_param_count_and_workspace_queries():
    assert B.e2a_so2_param_count(4, 128) == 1392640
    assert B.e2a_so2_param_count(3, 128) == 720896
    assert B.e2a_so2_param_count(1, 16) == 1536
    assert B.e2a_neighbors_workspace_bytes(100000) > 100000 * 12
    assert B.e2a_attention_workspace_bytes(1000, 4, 128, 8, B.E2A_DTYPE_BF16) >= 2 * 1000 * 128 * 4
    assert B.e2a_attention_workspace_bytes(10, 5, 128, 8, 1) == 0


FAKE = 0x1000  # never dereferenced: every call below fails host validation first


def nb_call(**kw):
    args = dict(pos=FAKE, n=10, batch=None, box=None, cutoff=5.0, row_ptr=FAKE, col=FAKE, cap=100,
                ws=FAKE, ws_bytes=1 << 30)
    args.update(kw)
    ne = ctypes.c_int64(-1)
    box = args["box"]
    box_p = None if box is None else ctypes.cast((ctypes.c_float * 3)(*box), ctypes.c_void_p)
    st = B.lib().e2a_build_neighbors(args["pos"], args["n"], args["batch"], box_p, ctypes.c_float(args["cutoff"]),
                                     args["row_ptr"], args["col"], args["cap"], ctypes.byref(ne), args["ws"],
                                     args["ws_bytes"], None)
    return st, B.last_error_message()


@pytest.mark.parametrize("kw,status", [
    (dict(pos=None), B.E2A_ERR_INVALID_ARG),
    (dict(row_ptr=None), B.E2A_ERR_INVALID_ARG),
    (dict(col=None), B.E2A_ERR_INVALID_ARG),
    (dict(cutoff=0.0), B.E2A_ERR_INVALID_ARG),
    (dict(cutoff=float("nan")), B.E2A_ERR_INVALID_ARG),
    (dict(n=-1), B.E2A_ERR_INVALID_ARG),
    (dict(cap=-5), B.E2A_ERR_INVALID_ARG),
    (dict(ws=None), B.E2A_ERR_INVALID_ARG),
    (dict(ws_bytes=16), B.E2A_ERR_INVALID_ARG),
    (dict(box=(9.0, 20.0, 20.0)), B.E2A_ERR_BOX_TOO_SMALL),
    (dict(box=(20.0, -1.0, 20.0)), B.E2A_ERR_INVALID_ARG),
])
def test_build_neighbors_rejects_on_host(kw, status):
    st, msg = nb_call(**kw)
    assert st == status, (st, msg)
    assert msg


def attn_args(**kw):
    a = B.AttnArgs()
    a.pos = a.row_ptr = a.col = a.feat = a.w_q = a.w_k = a.w_rad = a.w_so2 = a.out = a.workspace = FAKE
    a.n_atoms, a.n_edges, a.cutoff = 10, 20, 5.0
    a.L, a.C, a.H, a.n_rbf, a.dtype, a.variant = 1, 16, 1, 8, 0, 0
    a.workspace_bytes = 1 << 30
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(C=16, H=3), B.E2A_ERR_INVALID_ARG),
    (dict(L=5), B.E2A_ERR_INVALID_ARG),
    (dict(L=-1), B.E2A_ERR_INVALID_ARG),
    (dict(n_rbf=6), B.E2A_ERR_INVALID_ARG),
    (dict(dtype=7), B.E2A_ERR_INVALID_ARG),
    (dict(variant=9), B.E2A_ERR_INVALID_ARG),
    (dict(cutoff=-1.0), B.E2A_ERR_INVALID_ARG),
    (dict(feat=None), B.E2A_ERR_INVALID_ARG),
    (dict(w_so2=None), B.E2A_ERR_INVALID_ARG),
    (dict(out=None), B.E2A_ERR_INVALID_ARG),
    (dict(col=None), B.E2A_ERR_INVALID_ARG),
    (dict(n_edges=-1), B.E2A_ERR_INVALID_ARG),
    (dict(variant=2), B.E2A_ERR_UNSUPPORTED),          # no MFMA build for L=1, C=16, fp32
    (dict(workspace_bytes=8), B.E2A_ERR_INVALID_ARG),
    (dict(workspace=None), B.E2A_ERR_INVALID_ARG),
    (dict(feat=FAKE + 8), B.E2A_ERR_INVALID_ARG),       # arrays start on 16-byte boundaries
    (dict(w_so2=FAKE + 2), B.E2A_ERR_INVALID_ARG),
    (dict(out=FAKE + 4), B.E2A_ERR_INVALID_ARG),
    (dict(pos=FAKE + 12), B.E2A_ERR_INVALID_ARG),
])
def test_attention_rejects_on_host(kw, status):
    a = attn_args(**kw)
    st = B.lib().e2a_attention_fwd(ctypes.byref(a), None)
    assert st == status, (st, B.last_error_message())
    assert B.last_error_message()


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """e2a_attention_fwd_noalloc refuses, on the host and before any device
    call, a system whose workspace exceeds its fixed scratch; shape errors
    come first, as in e2a_attention_fwd."""
    a = attn_args(n_atoms=200000, L=4, C=128, H=8, dtype=1, workspace=None, workspace_bytes=0)
    assert B.lib().e2a_attention_fwd_noalloc(ctypes.byref(a), None) == B.E2A_ERR_INVALID_ARG
    assert "scratch" in B.last_error_message()
    assert B.e2a_attention_workspace_bytes(200000, 4, 128, 8, 1) > B.NOALLOC_SCRATCH_BYTES
    a = attn_args(L=7, workspace=None)
    assert B.lib().e2a_attention_fwd_noalloc(ctypes.byref(a), None) == B.E2A_ERR_INVALID_ARG
    assert "L=7" in B.last_error_message()
    assert B.lib().e2a_attention_fwd_noalloc(None, None) == B.E2A_ERR_INVALID_ARG


def test_attention_null_args():
    assert B.lib().e2a_attention_fwd(None, None) == B.E2A_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,status", [
    (dict(C=16, H=3), B.E2A_ERR_INVALID_ARG),
    (dict(L=5), B.E2A_ERR_INVALID_ARG),
    (dict(n_rbf=6), B.E2A_ERR_INVALID_ARG),
    (dict(cutoff=-1.0), B.E2A_ERR_INVALID_ARG),
    (dict(feat=None), B.E2A_ERR_INVALID_ARG),
    (dict(w_rad=None), B.E2A_ERR_INVALID_ARG),
    (dict(w_so2=None), B.E2A_ERR_INVALID_ARG),
    (dict(out=None), B.E2A_ERR_INVALID_ARG),
    (dict(col=None), B.E2A_ERR_INVALID_ARG),
    (dict(variant=2), B.E2A_ERR_UNSUPPORTED),
    (dict(workspace=None), B.E2A_ERR_INVALID_ARG),
])
def test_conv_rejects_on_host(kw, status):
    a = attn_args(**kw)
    st = B.lib().e2a_conv_fwd(ctypes.byref(a), None)
    assert st == status, (st, B.last_error_message())
    assert B.last_error_message()


def test_conv_does_not_need_qk_weights():
    """W_q and W_k may be NULL for the convolution: with them NULL and the
    workspace missing, the call fails on the workspace, not on W_q."""
    a = attn_args(w_q=None, w_k=None, workspace=None)
    assert B.lib().e2a_attention_fwd(ctypes.byref(a), None) == B.E2A_ERR_INVALID_ARG
    assert "w_q" in B.last_error_message()
    assert B.lib().e2a_conv_fwd(ctypes.byref(a), None) == B.E2A_ERR_INVALID_ARG
    assert "workspace" in B.last_error_message()
    assert B.lib().e2a_conv_fwd(None, None) == B.E2A_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,grads,status", [
    (dict(), (None, FAKE), B.E2A_ERR_INVALID_ARG),                  # grad_out
    (dict(), (FAKE, None), B.E2A_ERR_INVALID_ARG),                  # grad_feat
    (dict(out=None), (FAKE, FAKE), B.E2A_ERR_INVALID_ARG),          # the forward's output is an input here
    (dict(out_lse=None), (FAKE, FAKE), B.E2A_ERR_INVALID_ARG),
    (dict(variant=2), (FAKE, FAKE), B.E2A_ERR_UNSUPPORTED),         # no MFMA backward
    (dict(C=16, H=3), (FAKE, FAKE), B.E2A_ERR_INVALID_ARG),
    (dict(workspace_bytes=8), (FAKE, FAKE), B.E2A_ERR_INVALID_ARG),
    (dict(), (FAKE + 4, FAKE), B.E2A_ERR_INVALID_ARG),              # a misaligned cotangent
])
def test_backward_rejects_on_host(kw, grads, status):
    kw = dict(out_lse=FAKE, **kw) if "out_lse" not in kw else kw
    a = attn_args(**kw)
    st = B.lib().e2a_attention_bwd(ctypes.byref(a), grads[0], grads[1], None)
    assert st == status, (st, B.last_error_message())
    assert B.last_error_message()
    assert B.lib().e2a_attention_bwd(None, FAKE, FAKE, None) == B.E2A_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,grads,status", [
    (dict(), (None, FAKE, FAKE), B.E2A_ERR_INVALID_ARG),             # grad_out
    (dict(), (FAKE, None, None), B.E2A_ERR_INVALID_ARG),             # no output requested
    (dict(out_lse=None), (FAKE, None, FAKE), B.E2A_ERR_INVALID_ARG),  # alpha needs the log-normaliser
    (dict(w_rad=None), (FAKE, None, FAKE), B.E2A_ERR_INVALID_ARG),
    (dict(variant=2), (FAKE, None, FAKE), B.E2A_ERR_UNSUPPORTED),
    (dict(C=16, H=3), (FAKE, None, FAKE), B.E2A_ERR_INVALID_ARG),
    (dict(workspace_bytes=8), (FAKE, None, FAKE), B.E2A_ERR_INVALID_ARG),
    (dict(), (FAKE + 8, None, FAKE), B.E2A_ERR_INVALID_ARG),         # a misaligned cotangent
    (dict(feat=FAKE + 2), (FAKE, None, FAKE), B.E2A_ERR_INVALID_ARG),
])
def test_weight_backward_rejects_on_host(kw, grads, status):
    """e2a_attention_bwd_weights (grad_out, grad_feat, grad_w_so2 here; the
    other outputs NULL) checks its arguments before any launch."""
    kw = dict(out_lse=FAKE, **kw) if "out_lse" not in kw else kw
    a = attn_args(**kw)
    st = B.lib().e2a_attention_bwd_weights(ctypes.byref(a), grads[0], grads[1], None, None, None, grads[2], None,
                                           None)
    assert st == status, (st, B.last_error_message())
    assert B.last_error_message()
    assert B.lib().e2a_attention_bwd_weights(None, FAKE, FAKE, None, None, None, None, None, None) == \
        B.E2A_ERR_INVALID_ARG


def test_weight_backward_workspace_query():
    """The weight-gradient workspace holds the feature-gradient one, dq, dk,
    and one batch of per-edge tensors (x, dyhat, SO2(x): 3 x (L+1)^2 C floats
    per edge, at most 65536 edges)."""
    n, e, L, C = 1000, 30000, 3, 128
    got = B.e2a_attention_bwd_weights_workspace_bytes(n, e, L, C, 8)
    assert got >= B.e2a_attention_bwd_workspace_bytes(n, e, L, C, 8) + 4 * (2 * n * C + 3 * e * (L + 1) ** 2 * C)
    assert B.e2a_attention_bwd_weights_workspace_bytes(n, 100, L, C, 8) < got   # the batch shrinks with E
    assert B.e2a_attention_bwd_weights_workspace_bytes(n, -1, L, C, 8) == 0


def test_backward_workspace_query():
    n, e = 1000, 30000
    got = B.e2a_attention_bwd_workspace_bytes(n, e, 3, 128, 8)
    assert got >= 4 * (3 * n * 128 + e * 8)
    assert B.e2a_attention_bwd_workspace_bytes(-1, e, 3, 128, 8) == 0


def test_binding_refuses_missing_library(tmp_path, monkeypatch):
    import importlib.util
    spec = importlib.util.spec_from_file_location("e2a_copy", B.__file__)
    mod = importlib.util.module_from_spec(spec)
    monkeypatch.setattr(os.path, "exists", lambda p: False)
    with pytest.raises(ImportError):
        spec.loader.exec_module(mod)


# ------------------------------------------------------ host geometry -------
HOSTGEOM = os.path.join(os.path.dirname(B.library_path()), "libe2a_hostgeom.so")


@pytest.fixture(scope="module")
def hg():
    return ctypes.CDLL(HOSTGEOM)


def _cp(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def test_host_edge_rotation_matches_oracle(hg):
    rng = np.random.default_rng(0)
    u = rng.standard_normal((300, 3))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    u[:4] = [[0, 0, 1], [0, 0, -1], [1, 0, 0], [0, -1, 0]]
    u32 = np.ascontiguousarray(u, dtype=np.float32)
    R = np.zeros((300, 9), dtype=np.float32)
    hg.e2a_host_edge_rotation(_cp(u32), 300, _cp(R))
    assert np.max(np.abs(R.reshape(-1, 3, 3) - O.edge_rotation(u32.astype(np.float64)))) < 2e-6


@pytest.mark.parametrize("L", [1, 2, 3, 4])
def test_host_wigner_recursion_matches_oracle(hg, L):
    rng = np.random.default_rng(L)
    u = rng.standard_normal((200, 3))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    u[:2] = [[0, 0, 1], [0, 0, -1]]
    R = np.ascontiguousarray(O.edge_rotation(u), dtype=np.float32)
    nw = sum((2 * l + 1) ** 2 for l in range(L + 1))
    D = np.zeros((200, nw), dtype=np.float32)
    hg.e2a_host_wigner(L, _cp(R), 200, _cp(D))
    off = 0
    for l in range(L + 1):
        k = 2 * l + 1
        want = O.wigner_d(l, R.astype(np.float64))
        assert np.max(np.abs(D[:, off:off + k * k].reshape(-1, k, k) - want)) < 1e-6, l
        off += k * k


@pytest.mark.parametrize("L", [1, 2, 3, 4])
def test_host_wigner_rows_match_oracle(hg, L):
    """The row-wise form of the recursion (ir_row, one row per thread: the form
    the matrix-core kernels and the weight-gradient gather evaluate) against
    the oracle's least-squares Wigner blocks, on generic directions and on
    edges exactly along +-z (where the frame's angle phi is undefined and the
    pole branch of the rotation runs), +-x and +-y."""
    rng = np.random.default_rng(100 + L)
    u = rng.standard_normal((150, 3))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    u[:6] = [[0, 0, 1], [0, 0, -1], [1, 0, 0], [-1, 0, 0], [0, 1, 0], [0, -1, 0]]
    u32 = np.ascontiguousarray(u, dtype=np.float32)
    R = np.zeros((150, 9), dtype=np.float32)
    hg.e2a_host_edge_rotation(_cp(u32), 150, _cp(R))
    nw = sum((2 * l + 1) ** 2 for l in range(L + 1))
    D = np.zeros((150, nw), dtype=np.float32)
    hg.e2a_host_wigner_rows(L, _cp(R), 150, _cp(D))
    Rw = O.edge_rotation(u32.astype(np.float64))
    off = 0
    for l in range(L + 1):
        k = 2 * l + 1
        want = O.wigner_d(l, Rw)
        got = D[:, off:off + k * k].reshape(-1, k, k)
        assert np.max(np.abs(got - want)) < 2e-6, l
        # the aligned harmonics keep only m = 0 (Lemma 4.1) through the device blocks
        Y = O.real_sph_harm(l, u32.astype(np.float64))[:, l * l:(l + 1) ** 2]
        yz = np.einsum("emn,en->em", got.astype(np.float64), Y)
        ref = np.zeros(k)
        ref[l] = np.sqrt((2 * l + 1) / (4 * np.pi))
        assert np.max(np.abs(yz - ref)) < 5e-6, l
        off += k * k


def test_host_edge_unit_zero_length(hg):
    """A zero-length edge takes r_hat = z (length 0); other edges their own
    direction, as the oracle's edge_unit gives them."""
    r = np.array([[0, 0, 0], [3, 4, 0], [0, 0, -2], [1e-20, 0, 0]], dtype=np.float32)
    u = np.zeros((4, 3), dtype=np.float32)
    ln = np.zeros(4, dtype=np.float32)
    hg.e2a_host_edge_unit(_cp(r), 4, _cp(u), _cp(ln))
    r64, u64 = O.edge_unit(r.astype(np.float64))
    assert np.array_equal(u[0], [0, 0, 1]) and ln[0] == 0.0
    assert np.max(np.abs(u[1:3] - u64[1:3])) < 1e-7
    assert np.allclose(ln[1:3], r64[1:3])
    assert np.all(np.isfinite(u))


def test_host_radial_basis_matches_oracle(hg):
    r = np.ascontiguousarray(np.linspace(0.5, 5.0, 97), dtype=np.float32)
    e = np.zeros((97, 8), dtype=np.float32)
    hg.e2a_host_radial_basis8(_cp(r), 97, ctypes.c_float(5.0), _cp(e))
    assert np.max(np.abs(e - O.radial_basis(r.astype(np.float64), 5.0))) < 2e-6


def test_host_radial_basis_derivative_matches_oracle(hg):
    """radial_basis8_deriv (the position gradient's edge-length factor) against
    fourth-order central differences of the oracle's basis in fp64."""
    r = np.ascontiguousarray(np.linspace(0.5, 4.99, 97), dtype=np.float32)
    de = np.zeros((97, 8), dtype=np.float32)
    hg.e2a_host_radial_basis8_deriv(_cp(r), 97, ctypes.c_float(5.0), _cp(de))
    r64, h = r.astype(np.float64), 1e-4
    f = lambda x: O.radial_basis(x, 5.0)
    want = (-f(r64 + 2 * h) + 8 * f(r64 + h) - 8 * f(r64 - h) + f(r64 - 2 * h)) / (12 * h)
    assert np.max(np.abs(de - want)) <= 2e-5 * np.max(np.abs(want))


def test_host_wigner_tangents_match_oracle(hg):
    """The three tangents of D^0..D^4 for the frame turned about x, y, z
    (R -> R exp(-t [e_a]x)), as the position gradient forms them, against
    central differences of the oracle's fp64 Wigner blocks; the edges include
    both poles, where the frame's angles are singular."""
    L = 4
    rng = np.random.default_rng(44)
    u = rng.standard_normal((60, 3))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    u[:2] = [[0, 0, 1], [0, 0, -1]]
    R = O.edge_rotation(u)
    R32 = np.ascontiguousarray(R, dtype=np.float32)
    nw = sum((2 * l + 1) ** 2 for l in range(L + 1))
    dD = np.zeros((60, 3, nw), dtype=np.float32)
    hg.e2a_host_wigner_tangents(L, _cp(R32), 60, _cp(dD))

    def turn(a, t):
        K = np.zeros((3, 3))
        K[(a + 2) % 3, (a + 1) % 3], K[(a + 1) % 3, (a + 2) % 3] = 1.0, -1.0   # [e_a]x
        return np.eye(3) + np.sin(t) * K + (1 - np.cos(t)) * (K @ K)          # exp(t [e_a]x)

    h = 1e-4
    R64 = R32.astype(np.float64)
    for a in range(3):
        off = 0
        for l in range(L + 1):
            k = 2 * l + 1
            f = lambda t: O.wigner_d(l, R64 @ turn(a, -t))
            want = (-f(2 * h) + 8 * f(h) - 8 * f(-h) + f(-2 * h)) / (12 * h)
            got = dD[:, a, off:off + k * k].reshape(-1, k, k)
            assert np.max(np.abs(got - want)) <= 2e-5 * max(1.0, np.max(np.abs(want))), (a, l)
            off += k * k


# ------------------------------------------------------ binding checks ------
def _fake_layer_tensors(n=4, L=1, C=16, H=1, dev="cpu"):
    import torch
    K = (L + 1) ** 2
    t = dict(pos=torch.zeros(n, 3), row_ptr=torch.zeros(n + 1, dtype=torch.int64),
             col=torch.zeros(0, dtype=torch.int32), feat=torch.zeros(n, K, C), w_q=torch.zeros(C, C),
             w_k=torch.zeros(C, C), w_rad=torch.zeros(8, L + 1, C),
             w_so2=torch.zeros(B.e2a_so2_param_count(L, C)))
    return t


def test_binding_refuses_cpu_tensors():
    """Host tensors never reach the library as device pointers: every entry
    point raises before its ctypes call."""
    import torch
    t = _fake_layer_tensors()
    with pytest.raises(ValueError, match="GPU"):
        B.e2a_attention_fwd(t["pos"], t["row_ptr"], t["col"], t["feat"], t["w_q"], t["w_k"], t["w_rad"],
                            t["w_so2"], L=1, C=16, H=1, cutoff=5.0)
    with pytest.raises(ValueError, match="GPU"):
        B.e2a_conv_fwd(t["pos"], t["row_ptr"], t["col"], t["feat"], t["w_rad"], t["w_so2"], L=1, C=16, cutoff=5.0)
    with pytest.raises(ValueError, match="GPU"):
        B.e2a_build_neighbors(t["pos"], 5.0)
    o = torch.zeros(4, 4, 16)
    with pytest.raises(ValueError, match="GPU"):
        B.e2a_attention_bwd(t["pos"], t["row_ptr"], t["col"], t["feat"], t["w_q"], t["w_k"], t["w_rad"],
                            t["w_so2"], o, torch.zeros(4, 1), o, L=1, C=16, H=1, cutoff=5.0)
    with pytest.raises(ValueError, match="GPU"):
        B.e2a_attention_bwd_weights(t["pos"], t["row_ptr"], t["col"], t["feat"], t["w_q"], t["w_k"], t["w_rad"],
                                    t["w_so2"], o, torch.zeros(4, 1), o, L=1, C=16, H=1, cutoff=5.0)


@pytest.mark.parametrize("name,bad", [
    ("pos", (4, 2)), ("row_ptr", (4,)), ("feat", (4, 3, 16)), ("w_q", (16, 8)), ("w_k", (8, 16)),
    ("w_rad", (6, 2, 16)), ("w_so2", (100,)),
])
def test_binding_checks_shapes_before_the_call(monkeypatch, name, bad):
    """With the device check passed (the tensors stand in for device ones), a
    wrong shape raises before the library is called."""
    import torch
    monkeypatch.setattr(B, "_gpu_device", lambda pos: torch.device("cpu"))

    class NoCall:
        def __getattr__(self, attr):
            raise AssertionError(f"library called: {attr}")

    monkeypatch.setattr(B, "_lib", NoCall())
    monkeypatch.setattr(B, "e2a_attention_workspace_bytes", lambda *a: 16)
    monkeypatch.setattr(B, "e2a_so2_param_count", lambda L, C: 1536)
    t = _fake_layer_tensors()
    dt = t["row_ptr"].dtype if name == "row_ptr" else torch.float32
    t[name] = torch.zeros(bad, dtype=dt)
    with pytest.raises(ValueError, match=name):
        B._layer(B.lib, t["pos"], t["row_ptr"], t["col"], t["feat"], t["w_q"], t["w_k"], t["w_rad"], t["w_so2"],
                 1, 16, 1, 5.0, None, "auto", None, None, None, None, True)


def block_args(**kw):
    a = B.BlockArgs()
    for f in ("pos", "row_ptr", "col", "h_in", "h_out", "norm1", "w_q", "w_k", "w_rad", "w_so2", "w_o", "norm2",
              "w_1", "w_gate", "w_2", "workspace"):
        setattr(a, f, FAKE)
    a.n_atoms, a.n_edges, a.cutoff = 10, 20, 5.0
    a.L, a.C, a.H, a.n_rbf, a.dtype, a.variant = 1, 16, 1, 8, 0, 0
    a.workspace_bytes = 1 << 30
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(h_in=None), B.E2A_ERR_INVALID_ARG),
    (dict(h_out=None), B.E2A_ERR_INVALID_ARG),
    (dict(norm1=None), B.E2A_ERR_INVALID_ARG),
    (dict(w_gate=None), B.E2A_ERR_INVALID_ARG),          # L = 1 needs the gate
    (dict(w_so2=None), B.E2A_ERR_INVALID_ARG),           # the layer's own check
    (dict(w_q=None), B.E2A_ERR_INVALID_ARG),
    (dict(C=16, H=3), B.E2A_ERR_INVALID_ARG),
    (dict(L=5), B.E2A_ERR_INVALID_ARG),
    (dict(dtype=4), B.E2A_ERR_INVALID_ARG),
    (dict(variant=2), B.E2A_ERR_UNSUPPORTED),            # no MFMA layer for L=1, C=16, fp32
    (dict(workspace_bytes=16), B.E2A_ERR_INVALID_ARG),
    (dict(h_in=FAKE + 8), B.E2A_ERR_INVALID_ARG),        # read and written 16 bytes a lane
    (dict(h_out=FAKE + 4), B.E2A_ERR_INVALID_ARG),
])
def test_block_rejects_on_host(kw, status):
    a = block_args(**kw)
    st = B.lib().e2a_block_fwd(ctypes.byref(a), None)
    assert st == status, (st, B.last_error_message())
    assert B.last_error_message()
    assert B.lib().e2a_block_fwd(None, None) == B.E2A_ERR_INVALID_ARG


def test_block_gate_optional_at_l0_and_workspace_query():
    a = block_args(L=0, w_gate=None, workspace=None)
    assert B.lib().e2a_block_fwd(ctypes.byref(a), None) == B.E2A_ERR_INVALID_ARG
    assert "workspace" in B.last_error_message()          # not the gate
    n, L, C = 1000, 3, 128
    got = B.e2a_block_workspace_bytes(n, L, C, 8, B.E2A_DTYPE_BF16)
    assert got >= B.e2a_attention_workspace_bytes(n, L, C, 8, 1) + n * 16 * C * (2 + 4 + 4 + 2)
    assert B.e2a_block_workspace_bytes(n, 5, C, 8, 1) == 0


def test_packer_and_order_queries():
    """The packed image holds the SO(2) weights once (no padding), only where a
    matrix-core build exists; the packer refuses other shapes on the host."""
    assert B.e2a_so2_packed_bytes(4, 128, B.E2A_DTYPE_BF16) == 2 * B.e2a_so2_param_count(4, 128)
    assert B.e2a_so2_packed_bytes(3, 128, B.E2A_DTYPE_BF16) == 2 * B.e2a_so2_param_count(3, 128)
    assert B.e2a_so2_packed_bytes(4, 128, B.E2A_DTYPE_F32) == 0
    assert B.e2a_so2_packed_bytes(1, 16, B.E2A_DTYPE_BF16) == 0
    assert B.e2a_so2_packed_bytes(0, 128, B.E2A_DTYPE_BF16) == 0
    assert B.lib().e2a_pack_so2_weights(FAKE, FAKE, 1, 16, 1, None) == B.E2A_ERR_UNSUPPORTED
    assert B.lib().e2a_pack_so2_weights(None, FAKE, 4, 128, 1, None) == B.E2A_ERR_INVALID_ARG
    assert B.lib().e2a_pack_so2_weights(FAKE, FAKE, 7, 128, 1, None) == B.E2A_ERR_INVALID_ARG
    assert B.e2a_destination_order_workspace_bytes(100000) > 100000 * 12
    assert B.lib().e2a_destination_order(FAKE, 10, FAKE, None, 0, None) == B.E2A_ERR_INVALID_ARG
    assert B.lib().e2a_destination_order(None, 10, FAKE, FAKE, 1 << 30, None) == B.E2A_ERR_INVALID_ARG
    assert B.lib().e2a_destination_order(None, 0, None, None, 0, None) == B.E2A_OK


def test_misaligned_arrays_are_named_in_the_message():
    a = attn_args(feat=FAKE + 8)
    assert B.lib().e2a_attention_fwd(ctypes.byref(a), None) == B.E2A_ERR_INVALID_ARG
    assert "feat" in B.last_error_message() and "16-byte" in B.last_error_message()
