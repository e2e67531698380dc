"""Pins of the fp64 oracle to facts outside itself (CPU only).

The pages print no worked example, so each pin is a fact of mathematics or an
invariant the pages assert: Lemma 4.1's m = 0 sparsity in the edge-aligned
frame, closed forms and SciPy for the spherical harmonics, group laws of the
Wigner-D blocks, gauge freedom about the edge axis, rotation/translation
equivariance and permutation invariance of the layer, an L = 1 closed form in
vector notation, softmax algebra, online == two-pass, brute-force neighbours,
the empty-row case, equality with a dense Clebsch-Gordan tensor product, the
convolution against uniform-weight attention, and the feature gradient (the
message adjoint identity and central finite differences of the layer).
"""
import math

import numpy as np
import pytest
from scipy.special import sph_harm_y

import oracle as O
from workloads import make_config
from workloads.generators import _rsa_periodic, _to_f32_periodic, isolated_atom_variant


def rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300)


def random_rotation(rng):
    q = rng.standard_normal(4)
    q /= np.linalg.norm(q)
    w, x, y, z = q
    return np.array([[1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)],
                     [2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)],
                     [2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)]])


def unit(rng, n):
    v = rng.standard_normal((n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


@pytest.fixture(scope="module")
def tiny():
    w = make_config("tiny")
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    return w, rp, col


def run(w, rp, col, pos=None, feat=None, **kw):
    pos = w.pos if pos is None else pos
    feat = w.as_f32("feat") if feat is None else feat
    return O.attention(pos, rp, col, feat, w.as_f32("w_q"), w.as_f32("w_k"), w.as_f32("w_rad"),
                       w.as_f32("w_so2"), w.L, w.C, w.H, w.cutoff, box=w.box, **kw)


# ---------------------------------------------------------------- P1 --------
def test_p1_lemma41_aligned_harmonics_are_m0_only():
    """Technical summary section 2.1 (Lemma 4.1): in the frame aligned with the
    edge vector only the m = 0 harmonic survives, with value sqrt((2l+1)/4pi)."""
    rng = np.random.default_rng(0)
    rhat = np.concatenate([unit(rng, 500), [[0, 0, 1.0], [0, 0, -1.0], [1.0, 0, 0]]])
    R = O.edge_rotation(rhat)
    aligned = np.einsum("eij,ej->ei", R, rhat)
    L = 6
    Y = O.real_sph_harm(L, aligned)
    for l in range(L + 1):
        want = np.zeros(2 * l + 1)
        want[l] = math.sqrt((2 * l + 1) / (4 * math.pi))
        assert np.max(np.abs(Y[:, l * l:(l + 1) ** 2] - want)) <= 1e-13


# ---------------------------------------------------------------- P2 --------
def test_p2_real_sh_vs_scipy_complex():
    rng = np.random.default_rng(1)
    v = unit(rng, 300)
    theta = np.arccos(v[:, 2])
    phi = np.arctan2(v[:, 1], v[:, 0])
    L = 6
    Y = O.real_sph_harm(L, v)
    for l in range(L + 1):
        for m in range(-l, l + 1):
            c = sph_harm_y(l, abs(m), theta, phi)   # includes the Condon-Shortley phase
            if m == 0:
                want = c.real
            elif m > 0:
                want = math.sqrt(2) * (-1) ** m * c.real
            else:
                want = math.sqrt(2) * (-1) ** m * c.imag
            assert np.max(np.abs(Y[:, l * l + l + m] - want)) <= 1e-13, (l, m)


def test_p2_real_sh_closed_forms():
    rng = np.random.default_rng(2)
    v = unit(rng, 200)
    x, y, z = v.T
    Y = O.real_sph_harm(2, v * 3.7)      # un-normalised input
    pi = math.pi
    want = np.stack([
        np.full_like(x, 0.5 / math.sqrt(pi)),
        math.sqrt(3 / (4 * pi)) * y, math.sqrt(3 / (4 * pi)) * z, math.sqrt(3 / (4 * pi)) * x,
        0.5 * math.sqrt(15 / pi) * x * y, 0.5 * math.sqrt(15 / pi) * y * z,
        0.25 * math.sqrt(5 / pi) * (3 * z * z - 1), 0.5 * math.sqrt(15 / pi) * x * z,
        0.25 * math.sqrt(15 / pi) * (x * x - y * y)], axis=1)
    assert np.max(np.abs(Y - want)) <= 1e-13


def test_p2_real_sh_orthonormal_by_quadrature():
    L = 5
    nt, nphi = L + 2, 2 * L + 3
    xg, wg = np.polynomial.legendre.leggauss(nt)          # exact in cos(theta)
    phi = 2 * np.pi * np.arange(nphi) / nphi               # exact for |m| < nphi/2 products
    ct, ph = np.meshgrid(xg, phi, indexing="ij")
    st = np.sqrt(1 - ct ** 2)
    pts = np.stack([st * np.cos(ph), st * np.sin(ph), ct], axis=-1).reshape(-1, 3)
    w = (wg[:, None] * np.full(nphi, 2 * np.pi / nphi)[None, :]).ravel()
    Y = O.real_sph_harm(L, pts)
    G = (Y * w[:, None]).T @ Y
    assert np.max(np.abs(G - np.eye(G.shape[0]))) <= 1e-13


# ---------------------------------------------------------------- P3 --------
def test_p3_wigner_d_group_laws():
    rng = np.random.default_rng(3)
    Ra, Rb = random_rotation(rng), random_rotation(rng)
    for l in range(6):
        Da, Db, Dab = O.wigner_d(l, Ra), O.wigner_d(l, Rb), O.wigner_d(l, Ra @ Rb)
        assert np.max(np.abs(Da @ Da.T - np.eye(2 * l + 1))) <= 1e-12
        assert np.max(np.abs(Da @ Db - Dab)) <= 1e-12
        # defining property on fresh points
        v = unit(rng, 20)
        Yv = O.real_sph_harm(l, v)[:, l * l:]
        YRv = O.real_sph_harm(l, v @ Ra.T)[:, l * l:]
        assert np.max(np.abs(YRv - Yv @ Da.T)) <= 1e-12
    # D^1 is the Cartesian matrix in (y, z, x) order
    P = np.array([[0, 1, 0], [0, 0, 1], [1, 0, 0]], dtype=float)
    assert np.max(np.abs(O.wigner_d(1, Ra) - P @ Ra @ P.T)) <= 1e-12
    assert np.max(np.abs(O.wigner_d(0, Ra) - 1.0)) <= 1e-12


# ---------------------------------------------------------------- P4 --------
def test_p4_gauge_about_edge_axis(tiny):
    """Any rotation with R r_hat = z is a valid frame; the per-m SO(2) map must
    commute with the residual rotation about z."""
    w, rp, col = tiny
    rng = np.random.default_rng(4)
    o0, _ = run(w, rp, col)
    o1, _ = run(w, rp, col, gauge=rng.uniform(0, 2 * np.pi, col.size))
    assert rel(o1, o0) <= 1e-12


# ---------------------------------------------------------------- P5 --------
def _block_rotate(feat, R, L):
    out = np.empty_like(feat, dtype=np.float64)
    for l in range(L + 1):
        D = O.wigner_d(l, R)
        out[:, l * l:(l + 1) ** 2, :] = np.einsum("mn,anc->amc", D, feat[:, l * l:(l + 1) ** 2, :])
    return out


def test_p5_equivariance_open_tiny(tiny):
    """Equivariance of the layer (technical summary section 1: the EGNN keeps
    rotational and translational symmetry): positions R x + t and features
    D(R) h give outputs D(R) o."""
    w, rp, col = tiny
    rng = np.random.default_rng(5)
    R = random_rotation(rng)
    t = rng.standard_normal(3) * 10
    f = w.as_f32("feat").astype(np.float64)
    o0, l0 = run(w, rp, col, pos=w.pos.astype(np.float64), feat=f)
    o1, l1 = run(w, rp, col, pos=w.pos.astype(np.float64) @ R.T + t, feat=_block_rotate(f, R, w.L))
    assert rel(o1, _block_rotate(o0, R, w.L)) <= 1e-12
    assert np.max(np.abs(l1 - l0)) <= 1e-12


def test_p5_equivariance_open_drug_L3():
    w = make_config("drug", C=16, H=4)
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    dest = np.arange(0, w.n_atoms, 401)
    rng = np.random.default_rng(55)
    R = random_rotation(rng)
    f = w.as_f32("feat").astype(np.float64)
    o0, _ = run(w, rp, col, pos=w.pos.astype(np.float64), feat=f, dest=dest)
    o1, _ = run(w, rp, col, pos=w.pos.astype(np.float64) @ R.T - 3.0, feat=_block_rotate(f, R, w.L),
                dest=dest)
    assert rel(o1, _block_rotate(o0, R, w.L)) <= 1e-12


def test_p5_equivariance_periodic_cube_symmetry():
    """Periodic boxes admit only the cube's 24 rotations (about the box centre)
    plus wrapped translations."""
    w = make_config("water", C=8, H=2, L=2)
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    dest = np.arange(0, w.n_atoms, 97)
    b = float(w.box[0])
    R = np.array([[0, -1, 0], [0, 0, -1], [1, 0, 0]], dtype=float)  # a proper cube symmetry
    assert abs(np.linalg.det(R) - 1) < 1e-12
    f = w.as_f32("feat").astype(np.float64)
    pos = w.pos.astype(np.float64)
    pos2 = np.mod((pos - b / 2) @ R.T + b / 2 + np.array([3.3, -7.1, 11.0]), b)
    o0, _ = run(w, rp, col, pos=pos, feat=f, dest=dest)
    o1, _ = run(w, rp, col, pos=pos2, feat=_block_rotate(f, R, w.L), dest=dest)
    assert rel(o1, _block_rotate(o0, R, w.L)) <= 1e-12


# ---------------------------------------------------------------- P6 --------
def test_p6_permutation(tiny):
    w, rp, col = tiny
    rng = np.random.default_rng(6)
    perm = rng.permutation(w.n_atoms)
    o0, _ = run(w, rp, col)
    pos_p = w.pos[perm]
    feat_p = w.as_f32("feat")[perm]
    rp2, col2 = O.neighbor_list(pos_p, w.cutoff, None, None)
    o1, _ = run(w, rp2, col2, pos=pos_p, feat=feat_p)
    assert rel(o1, o0[perm]) <= 1e-12


# ---------------------------------------------------------------- P7 --------
def test_p7_l1_closed_form_vector_identities():
    """With rho = 1, W0[1,1] = a I, W1 = b I, W2 = c I (m = 1), the value is
    a (r.x) r + b (x - (r.x) r) + c (r x x) in Cartesian terms; W0[0,1] = w I
    gives w x0 r and W0[1,0] = w I gives w (r.x)."""
    rng = np.random.default_rng(7)
    C, L, E = 3, 1, 50
    a, b, c, w01, w10 = 0.7, -1.3, 0.45, 0.9, -0.6
    W0 = np.zeros((2 * C, 2 * C))
    W0[C:, C:] = a * np.eye(C)
    W0[:C, C:] = w01 * np.eye(C)      # l_in = 0 -> l_out = 1
    W0[C:, :C] = w10 * np.eye(C)      # l_in = 1 -> l_out = 0
    W1 = b * np.eye(C)
    W2 = c * np.eye(C)
    w_so2 = np.concatenate([W0.ravel(), W1.ravel(), W2.ravel()])
    rvec = rng.standard_normal((E, 3)) * 2
    h = rng.standard_normal((E, 4, C))
    v = O.edge_messages(rvec, h, None, w_so2, L, C, 5.0, rho=1.0)
    rh = rvec / np.linalg.norm(rvec, axis=1, keepdims=True)
    xcart = np.stack([h[:, 3, :], h[:, 1, :], h[:, 2, :]], axis=1)     # (y,z,x) -> (x,y,z)
    dot = np.einsum("ei,eic->ec", rh, xcart)
    want_vec = (a * dot[:, None, :] * rh[:, :, None]
                + b * (xcart - dot[:, None, :] * rh[:, :, None])
                + c * np.cross(rh[:, :, None], xcart, axis=1)
                + w01 * h[:, 0, None, :] * rh[:, :, None])
    got_vec = np.stack([v[:, 3, :], v[:, 1, :], v[:, 2, :]], axis=1)
    assert np.max(np.abs(got_vec - want_vec)) <= 1e-13
    assert np.max(np.abs(v[:, 0, :] - w10 * dot)) <= 1e-13


# ---------------------------------------------------------------- P8 --------
def test_p8_attention_limits(tiny):
    w, rp, col = tiny
    # W_q = 0: uniform weights, output is the neighbour mean of v
    o, _ = run(w, rp, col, w_q_zero=True)
    i = 5
    e = np.arange(rp[i], rp[i + 1])
    src = col[e]
    rvec = O.min_image(w.pos[src].astype(np.float64) - w.pos[i], None)
    v = O.edge_messages(rvec, w.as_f32("feat")[src], w.as_f32("w_rad"), w.as_f32("w_so2"),
                        w.L, w.C, w.cutoff)
    assert rel(o[i], v.mean(axis=0)) <= 1e-12
    # softmax algebra: per-segment constant shift changes nothing; x100 stays finite and -> argmax
    rng = np.random.default_rng(8)
    s = rng.standard_normal((30, 3))
    st, ln = np.array([0, 7, 19]), np.array([7, 12, 11])
    a0, _ = O.segment_softmax(s, st, ln)
    shift = np.repeat(rng.standard_normal((3, 3)) * 50, ln, axis=0)
    a1, _ = O.segment_softmax(s + shift, st, ln)
    assert np.max(np.abs(a1 - a0)) <= 1e-12
    a2, _ = O.segment_softmax(s * 1e4, st, ln)
    assert np.all(np.isfinite(a2))
    for k in range(3):
        blk = s[st[k]:st[k] + ln[k]]
        assert np.allclose(a2[st[k]:st[k] + ln[k]], (blk == blk.max(axis=0)).astype(float), atol=1e-4)


def test_p8_single_neighbour_row():
    pos = np.array([[0, 0, 0], [1.5, 0.3, -0.2], [40, 40, 40]], dtype=np.float32)
    w = make_config("tiny", geometry=(pos, None, None, {}))
    rp, col = O.neighbor_list(w.pos, w.cutoff)
    assert list(np.diff(rp)) == [1, 1, 0]
    o, lse = run(w, rp, col)
    v = O.edge_messages(O.min_image(w.pos[[1]].astype(np.float64) - w.pos[0], None),
                        w.as_f32("feat")[[1]], w.as_f32("w_rad"), w.as_f32("w_so2"), w.L, w.C, w.cutoff)
    assert rel(o[0], v[0]) <= 1e-13
    assert np.all(o[2] == 0) and np.all(np.isneginf(lse[2]))


# ---------------------------------------------------------------- P9 --------
def test_p9_online_equals_two_pass(tiny):
    w, rp, col = tiny
    o2, l2 = run(w, rp, col)
    o1, l1 = O.attention_online(w.pos, rp, col, w.as_f32("feat"), w.as_f32("w_q"), w.as_f32("w_k"),
                                w.as_f32("w_rad"), w.as_f32("w_so2"), w.L, w.C, w.H, w.cutoff)
    assert rel(o1, o2) <= 1e-13
    assert np.max(np.abs(l1 - l2)) <= 1e-12


def test_p9_online_equals_two_pass_multihead():
    w = make_config("water", C=16, H=4, L=2)
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box)
    dest = np.arange(0, w.n_atoms, 613)
    args = (rp, col, w.as_f32("feat"), w.as_f32("w_q"), w.as_f32("w_k"), w.as_f32("w_rad"),
            w.as_f32("w_so2"), w.L, w.C, w.H, w.cutoff)
    o2, _ = O.attention(w.pos, *args, box=w.box, dest=dest)
    o1, _ = O.attention_online(w.pos, *args, box=w.box, dest=dest, block=7)
    assert rel(o1, o2) <= 1e-13


# ---------------------------------------------------------------- P10 -------
@pytest.mark.parametrize("name", ["tiny", "drug", "drug_origin"])
def test_p10_neighbours_bruteforce_open(name):
    w = make_config(name, C=4, H=1, L=0)
    a = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    b = O.neighbor_list_bruteforce(w.pos, w.cutoff, w.box, w.batch)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # symmetric relation: i in N(j) <=> j in N(i)
    rp, col = a
    src = np.repeat(np.arange(w.n_atoms), np.diff(rp))
    fwd = set(zip(src.tolist(), col.tolist()))
    assert all((j, i) in fwd for i, j in fwd)
    assert col.size % 2 == 0


def test_p10_neighbours_bruteforce_periodic():
    rng = np.random.default_rng(10)
    side = (2000 / 0.1) ** (1 / 3)
    box = np.full(3, side)
    pos = _to_f32_periodic(_rsa_periodic(rng, 2000, side, 0.9), box)
    a = O.neighbor_list(pos, 5.0, box.astype(np.float32))
    b = O.neighbor_list_bruteforce(pos, 5.0, box.astype(np.float32))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert a[1].size % 2 == 0 and a[1].size > 2000 * 40


def test_p10_fp32_predicate_boundary():
    """Strict '<' on the fp32 d^2, no self loop, one-image periodic wrap."""
    rc = np.float32(5.0)
    pos = np.array([[0, 0, 0], [5, 0, 0], [0, 4.9999995, 0], [9.5, 0, 0]], dtype=np.float32)
    rp, col = O.neighbor_list_bruteforce(pos, rc, np.full(3, 11.0, dtype=np.float32))
    nb = {i: set(col[rp[i]:rp[i + 1]].tolist()) for i in range(4)}
    assert 1 not in nb[0]                    # d = 5 exactly: excluded
    assert 2 in nb[0]                        # just inside
    assert 3 in nb[0]                        # wrapped: 9.5 - 11 = -1.5
    assert all(i not in nb[i] for i in range(4))


def test_p10_coincident_atoms_are_not_neighbours():
    """Two atoms at one point (d2 = 0 in fp32) have no edge direction and are
    not each other's neighbours (the reading of the predicate's lower bound);
    each still sees the third atom 1 A away, which sees both.  Expected lists
    written out by hand."""
    pos = np.array([[1, 1, 1], [1, 1, 1], [2, 1, 1], [1, 1, 1]], dtype=np.float32)
    for fn in (O.neighbor_list, O.neighbor_list_bruteforce):
        rp, col = fn(pos, 5.0)
        assert rp.tolist() == [0, 1, 2, 5, 6]
        assert col.tolist() == [2, 2, 0, 1, 3, 2]
    # periodic: a wrapped image at distance 0 is the same point
    box = np.full(3, 10.0, dtype=np.float32)
    pos = np.array([[0, 5, 5], [0, 5, 5], [9, 5, 5]], dtype=np.float32)
    rp, col = O.neighbor_list_bruteforce(pos, 4.0, box)
    assert rp.tolist() == [0, 1, 2, 4]
    assert col.tolist() == [2, 2, 0, 1]


def test_zero_length_edge_is_the_limit_along_z():
    """A zero-length edge takes r_hat = z: its message equals the limit of
    edges (0, 0, t) as t -> 0 (a continuous limit along that direction:
    the frame is fixed, the radial basis is smooth in r)."""
    rng = np.random.default_rng(12)
    L, C = 3, 4
    h = rng.standard_normal((1, (L + 1) ** 2, C))
    w_rad = rng.standard_normal((8, L + 1, C))
    w_so2 = rng.standard_normal(sum((1 if m == 0 else 2) * ((L + 1 - m) * C) ** 2 for m in range(L + 1)))
    v0 = O.edge_messages(np.zeros((1, 3)), h, w_rad, w_so2, L, C, 5.0)
    assert np.all(np.isfinite(v0))
    # the gap shrinks in proportion to t (the radial basis has a nonzero slope)
    gaps = [rel(v0, O.edge_messages(np.array([[0.0, 0.0, t]]), h, w_rad, w_so2, L, C, 5.0)) for t in (1e-6, 1e-9)]
    assert gaps[0] < 1e-5 and gaps[1] < 1e-8 and 300 < gaps[0] / gaps[1] < 3000
    # and differs from the limit along another direction (the reading matters)
    v2 = O.edge_messages(np.array([[1e-9, 0.0, 0.0]]), h, w_rad, w_so2, L, C, 5.0)
    assert rel(v0, v2) > 1e-3
    r, u = O.edge_unit(np.array([[0.0, 0.0, 0.0], [0.0, 3.0, 4.0]]))
    assert r.tolist() == [0.0, 5.0] and np.allclose(u, [[0, 0, 1], [0, 0.6, 0.8]])


# ---------------------------------------------------------------- P11 -------
def _cg_complex(j1, m1, j2, m2, J, M):
    """Clebsch-Gordan <j1 m1 j2 m2 | J M> by Racah's formula."""
    if M != m1 + m2 or J < abs(j1 - j2) or J > j1 + j2 or abs(m1) > j1 or abs(m2) > j2 or abs(M) > J:
        return 0.0
    f = math.factorial
    pre = math.sqrt((2 * J + 1) * f(J + j1 - j2) * f(J - j1 + j2) * f(j1 + j2 - J) / f(j1 + j2 + J + 1))
    pre *= math.sqrt(f(J + M) * f(J - M) * f(j1 - m1) * f(j1 + m1) * f(j2 - m2) * f(j2 + m2))
    s = 0.0
    for k in range(0, j1 + j2 - J + 1):
        args = [k, j1 + j2 - J - k, j1 - m1 - k, j2 + m2 - k, J - j2 + m1 + k, J - j1 - m2 + k]
        if min(args) < 0:
            continue
        s += (-1) ** k / np.prod([f(a) for a in args])
    return pre * s


def _U(l):
    """Real (no Condon-Shortley phase) <- complex (with the phase) change of basis."""
    U = np.zeros((2 * l + 1, 2 * l + 1), dtype=complex)
    U[l, l] = 1
    for m in range(1, l + 1):
        U[l + m, l + m] = (-1) ** m / math.sqrt(2)
        U[l + m, l - m] = 1 / math.sqrt(2)
        U[l - m, l + m] = (-1) ** m / (1j * math.sqrt(2))
        U[l - m, l - m] = -1 / (1j * math.sqrt(2))
    return U


def _cg_real(l1, l2, l3):
    Cc = np.zeros((2 * l3 + 1, 2 * l1 + 1, 2 * l2 + 1))
    for M in range(-l3, l3 + 1):
        for m1 in range(-l1, l1 + 1):
            m2 = M - m1
            if abs(m2) <= l2:
                Cc[M + l3, m1 + l1, m2 + l2] = _cg_complex(l1, m1, l2, m2, l3, M)
    Cr = np.einsum("Ma,abc,mb,nc->Mmn", _U(l3), Cc, _U(l1).conj(), _U(l2).conj())
    if np.max(np.abs(Cr.real)) > 1e-12:
        assert np.max(np.abs(Cr.imag)) < 1e-12
        return Cr.real
    assert np.max(np.abs(Cr.real)) < 1e-12
    return Cr.imag


def test_p11_cg_real_basis_is_equivariant():
    rng = np.random.default_rng(11)
    R = random_rotation(rng)
    for (l1, l2, l3) in [(1, 1, 1), (1, 1, 2), (2, 1, 2), (2, 3, 3), (3, 2, 4), (1, 2, 2)]:
        Cr = _cg_real(l1, l2, l3)
        D1, D2, D3 = O.wigner_d(l1, R), O.wigner_d(l2, R), O.wigner_d(l3, R)
        lhs = np.einsum("Mm,mab->Mab", D3, Cr)
        rhs = np.einsum("Mcd,ca,db->Mab", Cr, D1, D2)
        assert np.max(np.abs(lhs - rhs)) <= 1e-12


@pytest.mark.parametrize("L", [1, 2, 3])
def test_p11_eaas_equals_dense_tensor_product(L):
    """EAAS (technical summary section 2.1; abstract: "sparse parity
    re-indexing"): with W1/W2 built from Clebsch-Gordan coefficients of the
    aligned-frame filter Y^{l_f}(z) (only m_f = 0 survives), the per-m SO(2)
    path equals the global-frame dense product sum_{l_f} w (h_j (x) Y^{l_f}(r_hat))."""
    rng = np.random.default_rng(110 + L)
    C, E = 2, 200
    paths = {}
    for li in range(L + 1):
        for lo in range(L + 1):
            for lf in range(abs(li - lo), min(li + lo, 2 * L) + 1):
                paths[(li, lf, lo)] = rng.standard_normal()
    blocks = {m: [np.zeros(((L + 1 - m) * C,) * 2) for _ in range(1 if m == 0 else 2)] for m in range(L + 1)}
    for (li, lf, lo), wp in paths.items():
        Cr = _cg_real(li, lf, lo) * math.sqrt((2 * lf + 1) / (4 * math.pi)) * wp
        c0 = Cr[:, :, lf]                              # m_f = 0 column, [2lo+1, 2li+1]
        for m in range(0, min(li, lo) + 1):
            rs, cs = (li - m) * C, (lo - m) * C
            if m == 0:
                blocks[0][0][rs:rs + C, cs:cs + C] += c0[lo, li] * np.eye(C)
                continue
            a = c0[lo + m, li + m]     # x_{+m} -> y_{+m}
            d = c0[lo - m, li - m]     # x_{-m} -> y_{-m}
            bb = c0[lo + m, li - m]    # x_{-m} -> y_{+m}
            cc = c0[lo - m, li + m]    # x_{+m} -> y_{-m}
            assert abs(a - d) < 1e-12 and abs(bb + cc) < 1e-12   # SO(2) form
            blocks[m][0][rs:rs + C, cs:cs + C] += a * np.eye(C)
            blocks[m][1][rs:rs + C, cs:cs + C] += cc * np.eye(C)
    w_so2 = np.concatenate([blocks[m][k].ravel() for m in range(L + 1) for k in range(len(blocks[m]))])
    rvec = rng.standard_normal((E, 3))
    rvec[0] = [0, 0, 2.0]
    rvec[1] = [0, 0, -1.0]
    h = rng.standard_normal((E, (L + 1) ** 2, C))
    v = O.edge_messages(rvec, h, None, w_so2, L, C, 5.0, rho=1.0)
    Yf = O.real_sph_harm(2 * L, rvec)
    want = np.zeros_like(v)
    for (li, lf, lo), wp in paths.items():
        Cr = _cg_real(li, lf, lo) * wp
        want[:, lo * lo:(lo + 1) ** 2, :] += np.einsum(
            "Mab,eac,eb->eMc", Cr, h[:, li * li:(li + 1) ** 2, :], Yf[:, lf * lf:(lf + 1) ** 2])
    assert np.max(np.abs(v - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


# ---------------------------------------------------------------- P12 -------
def test_p12_empty_row_is_zero():
    w = isolated_atom_variant(make_config("tiny"))
    rp, col = O.neighbor_list(w.pos, w.cutoff)
    assert rp[-1] == rp[-2]
    o, lse = run(w, rp, col)
    assert np.all(o[-1] == 0) and np.all(np.isneginf(lse[-1]))
    assert np.all(np.abs(o[:-1]).sum(axis=(1, 2)) > 0)


# ---------------------------------------------------------------- P13 -------
def conv(w, rp, col, pos=None, feat=None, **kw):
    pos = w.pos if pos is None else pos
    feat = w.as_f32("feat") if feat is None else feat
    return O.convolution(pos, rp, col, feat, w.as_f32("w_rad"), w.as_f32("w_so2"), w.L, w.C, w.cutoff,
                         box=w.box, **kw)


@pytest.mark.parametrize("name", ["tiny", "drug"])
def test_p13_convolution_is_degree_times_uniform_attention(name):
    """With W_q = 0 every logit is 0, so softmax gives each of the deg_i
    neighbours weight exactly 1/deg_i and the attention output is the
    neighbour mean of v_ij; the convolution (the plain sum) must be deg_i
    times it.  Checks the convolution against the pinned attention oracle on
    rows of every degree, including the empty ones."""
    w = make_config(name) if name == "tiny" else make_config(name, C=8, H=2, L=2)
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    dest = np.arange(min(w.n_atoms, 400))
    oc = conv(w, rp, col, dest=dest)
    oa, _ = run(w, rp, col, dest=dest, w_q_zero=True)
    deg = (rp[dest + 1] - rp[dest]).astype(np.float64)
    assert rel(oc, deg[:, None, None] * oa) <= 1e-13
    assert np.all(oc[deg == 0] == 0)


def test_p13_convolution_equivariance_and_linearity(tiny):
    """Positions R x + t and features D(R) h give D(R) o; and the sum of
    messages is linear in the features (the logits, the only nonlinear part of
    attention, are absent)."""
    w, rp, col = tiny
    rng = np.random.default_rng(13)
    R = random_rotation(rng)
    t = rng.standard_normal(3) * 10
    f = w.as_f32("feat").astype(np.float64)
    o0 = conv(w, rp, col, pos=w.pos.astype(np.float64), feat=f)
    o1 = conv(w, rp, col, pos=w.pos.astype(np.float64) @ R.T + t, feat=_block_rotate(f, R, w.L))
    assert rel(o1, _block_rotate(o0, R, w.L)) <= 1e-12
    g = rng.standard_normal(f.shape)
    a, b = 0.7, -1.9
    assert rel(conv(w, rp, col, feat=a * f + b * g), a * o0 + b * conv(w, rp, col, feat=g)) <= 1e-12


# ---------------------------------------------------------------- P14 -------
def _so2_count(L, C):
    return sum((1 if m == 0 else 2) * ((L + 1 - m) * C) ** 2 for m in range(L + 1))


@pytest.mark.parametrize("L,C", [(1, 4), (3, 5), (4, 3)])
def test_p14_message_adjoint_identity(L, C):
    """The message is linear in the neighbour's features, so its adjoint must
    satisfy <edge_messages(h), g> = <h, edge_messages_vjp(g)> exactly (up to
    rounding) for any edges, features, cotangents and weights."""
    rng = np.random.default_rng(140 + L)
    E = 9
    rvec = rng.standard_normal((E, 3)) * 2.0
    h = rng.standard_normal((E, (L + 1) ** 2, C))
    g = rng.standard_normal((E, (L + 1) ** 2, C))
    w_rad = rng.standard_normal((8, L + 1, C))
    w_so2 = rng.standard_normal(_so2_count(L, C))
    a = np.sum(O.edge_messages(rvec, h, w_rad, w_so2, L, C, 5.0) * g)
    b = np.sum(h * O.edge_messages_vjp(rvec, g, w_rad, w_so2, L, C, 5.0))
    assert abs(a - b) <= 1e-12 * max(abs(a), 1.0)


def _small_periodic(L, C, H):
    rng = np.random.default_rng(1414)
    box = np.full(3, 11.0)
    pos = _to_f32_periodic(_rsa_periodic(rng, 120, 11.0, 0.9), box)
    return make_config("tiny", L=L, C=C, H=H, geometry=(pos, box.astype(np.float32), None, {}))


@pytest.mark.parametrize("case", ["tiny_L1_H2", "tiny_L3_H2", "periodic_L2_H2"])
def test_p14_feature_gradient_finite_differences(case):
    """dL/dh from attention_backward against central differences of
    L(h) = <G, attention(h)> along two random directions: one that moves only
    the l = 0 block (the path through the logits, q and k, and the values) and
    one that moves only l >= 1 (the values alone).  fp64, fourth-order
    central differences with eps = 2e-4 (the error falls as eps^4 and is
    about 1e-10 relative here)."""
    if case == "tiny_L1_H2":
        w = make_config("tiny", C=16, H=2)
    elif case == "tiny_L3_H2":
        w = make_config("tiny", L=3, C=8, H=2)
    else:
        w = _small_periodic(2, 8, 2)
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    rng = np.random.default_rng(1415)
    f = w.as_f32("feat").astype(np.float64)
    # scale the weights up so that the logits vary and the softmax is not flat
    wq, wk = 3.0 * w.as_f32("w_q").astype(np.float64), 3.0 * w.as_f32("w_k").astype(np.float64)
    G = rng.standard_normal(f.shape)

    def loss(ff):
        o, _ = O.attention(w.pos, rp, col, ff, wq, wk, w.as_f32("w_rad"), w.as_f32("w_so2"), w.L, w.C, w.H,
                           w.cutoff, box=w.box)
        return float(np.sum(G * o))

    grad = O.attention_backward(w.pos, rp, col, f, wq, wk, w.as_f32("w_rad"), w.as_f32("w_so2"), w.L, w.C, w.H,
                                w.cutoff, G, box=w.box)
    eps = 2e-4
    for part in ("l0", "rest"):
        u = rng.standard_normal(f.shape)
        if part == "l0":
            u[:, 1:, :] = 0
        else:
            u[:, 0, :] = 0
        # fourth-order central difference (error O(eps^4))
        fd = (-loss(f + 2 * eps * u) + 8 * loss(f + eps * u) - 8 * loss(f - eps * u) + loss(f - 2 * eps * u)) \
            / (12 * eps)
        an = float(np.sum(grad * u))
        assert abs(fd - an) <= 1e-8 * max(abs(an), 1e-3), (part, fd, an)


def test_p14_feature_gradient_subset_equals_full(tiny):
    """Asking for the gradient of some atoms only gives the same rows as the
    full gradient."""
    w, rp, col = tiny
    G = np.random.default_rng(1416).standard_normal((w.n_atoms, (w.L + 1) ** 2, w.C))
    args = (w.pos, rp, col, w.as_f32("feat"), w.as_f32("w_q"), w.as_f32("w_k"), w.as_f32("w_rad"),
            w.as_f32("w_so2"), w.L, w.C, w.H, w.cutoff, G)
    full = O.attention_backward(*args)
    dest = np.array([0, 5, 17, 63])
    assert rel(O.attention_backward(*args, dest=dest), full[dest]) <= 1e-13


# ---------------------------------------------------------------- P15 -------
@pytest.mark.parametrize("L,C", [(1, 4), (3, 5), (4, 3)])
def test_p15_weight_vjp_adjoint_identities(L, C):
    """The message is linear in W_so2 for fixed W_rad and linear in W_rad for
    fixed W_so2, so for any direction U the weight adjoints must satisfy
    <edge_messages(W_rad, U), g> = <dW_so2, U> and
    <edge_messages(U, W_so2), g> = <dW_rad, U> exactly (up to rounding)."""
    rng = np.random.default_rng(150 + L)
    E = 9
    rvec = rng.standard_normal((E, 3)) * 2.0
    h = rng.standard_normal((E, (L + 1) ** 2, C))
    g = rng.standard_normal((E, (L + 1) ** 2, C))
    w_rad = rng.standard_normal((8, L + 1, C))
    w_so2 = rng.standard_normal(_so2_count(L, C))
    dw_rad, dw_so2 = O.edge_messages_weight_vjp(rvec, h, g, w_rad, w_so2, L, C, 5.0)
    assert dw_rad.shape == w_rad.shape and dw_so2.shape == w_so2.shape
    u_so2 = rng.standard_normal(w_so2.shape)
    a = np.sum(O.edge_messages(rvec, h, w_rad, u_so2, L, C, 5.0) * g)
    assert abs(a - np.sum(dw_so2 * u_so2)) <= 1e-12 * max(abs(a), 1.0)
    u_rad = rng.standard_normal(w_rad.shape)
    b = np.sum(O.edge_messages(rvec, h, u_rad, w_so2, L, C, 5.0) * g)
    assert abs(b - np.sum(dw_rad * u_rad)) <= 1e-12 * max(abs(b), 1.0)


@pytest.mark.parametrize("case", ["tiny_L1_H2", "periodic_L2_H2"])
def test_p15_weight_gradient_finite_differences(case):
    """dL/dW for W_q, W_k, W_rad and W_so2 from attention_weight_backward
    against fourth-order central differences of L(W) = <G, attention(W)>
    along a random direction per weight (fp64, eps = 2e-4; W_q and W_k reach
    the loss through the softmax, W_rad and W_so2 linearly)."""
    if case == "tiny_L1_H2":
        w = make_config("tiny", C=16, H=2)
    else:
        w = _small_periodic(2, 8, 2)
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    rng = np.random.default_rng(1515)
    f = w.as_f32("feat").astype(np.float64)
    W = {"w_q": 3.0 * w.as_f32("w_q").astype(np.float64), "w_k": 3.0 * w.as_f32("w_k").astype(np.float64),
         "w_rad": w.as_f32("w_rad").astype(np.float64), "w_so2": w.as_f32("w_so2").astype(np.float64)}
    G = rng.standard_normal(f.shape)

    def loss(WW):
        o, _ = O.attention(w.pos, rp, col, f, WW["w_q"], WW["w_k"], WW["w_rad"], WW["w_so2"], w.L, w.C, w.H,
                           w.cutoff, box=w.box)
        return float(np.sum(G * o))

    grads = O.attention_weight_backward(w.pos, rp, col, f, W["w_q"], W["w_k"], W["w_rad"], W["w_so2"], w.L, w.C,
                                        w.H, w.cutoff, G, box=w.box)
    eps = 2e-4
    for name in ("w_q", "w_k", "w_rad", "w_so2"):
        assert grads[name].shape == W[name].shape
        u = rng.standard_normal(W[name].shape)

        def at(t):
            WW = dict(W)
            WW[name] = W[name] + t * u
            return loss(WW)

        fd = (-at(2 * eps) + 8 * at(eps) - 8 * at(-eps) + at(-2 * eps)) / (12 * eps)
        an = float(np.sum(grads[name] * u))
        assert abs(fd - an) <= 1e-8 * max(abs(an), 1e-3), (name, fd, an)


def test_p15_weight_gradient_centres_with_sparse_cotangent(tiny):
    """With G zero outside a set of destinations, summing over those
    destinations' edges only gives the full weight gradients."""
    w, rp, col = tiny
    G = np.random.default_rng(1517).standard_normal((w.n_atoms, (w.L + 1) ** 2, w.C))
    keep = np.array([3, 10, 11, 40])
    G[np.setdiff1d(np.arange(w.n_atoms), keep)] = 0.0
    args = (w.pos, rp, col, w.as_f32("feat"), w.as_f32("w_q"), w.as_f32("w_k"), w.as_f32("w_rad"),
            w.as_f32("w_so2"), w.L, w.C, w.H, w.cutoff, G)
    a = O.attention_weight_backward(*args)
    b = O.attention_weight_backward(*args, centres=keep)
    for name in a:
        assert rel(a[name], b[name]) <= 1e-13, name


def test_p15_weight_gradient_chunking_invariant(tiny):
    """The weight gradients do not depend on how the edges are grouped."""
    w, rp, col = tiny
    G = np.random.default_rng(1516).standard_normal((w.n_atoms, (w.L + 1) ** 2, w.C))
    args = (w.pos, rp, col, w.as_f32("feat"), w.as_f32("w_q"), w.as_f32("w_k"), w.as_f32("w_rad"),
            w.as_f32("w_so2"), w.L, w.C, w.H, w.cutoff, G)
    a = O.attention_weight_backward(*args)
    b = O.attention_weight_backward(*args, chunk_edges=7)
    for name in a:
        assert rel(a[name], b[name]) <= 1e-13, name


# ---------------------------------------------------------------- P16 -------
def _pos_case(L, C, H, seed=1600):
    w = make_config("tiny", L=L, C=C, H=H)
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    G = np.random.default_rng(seed).standard_normal((w.n_atoms, (L + 1) ** 2, C))
    f = w.as_f32("feat").astype(np.float64)
    W = [w.as_f32(n).astype(np.float64) for n in ("w_q", "w_k", "w_rad", "w_so2")]
    return w, rp, col, G, f, W


def _pos_grad(w, pos, rp, col, f, W, G, **kw):
    return O.attention_position_backward(pos, rp, col, f, *W, w.L, w.C, w.H, w.cutoff, G, box=w.box, **kw)


def test_p16_position_gradient_translation_invariance():
    """The layer depends on positions only through edge vectors, so the
    gradients of all atoms sum to zero."""
    w, rp, col, G, f, W = _pos_case(2, 8, 2)
    g = _pos_grad(w, w.pos.astype(np.float64), rp, col, f, W, G)
    assert np.abs(g.sum(axis=0)).max() <= 1e-8 * np.abs(g).max()


def test_p16_position_gradient_rotation_equivariance():
    """Rotating the positions by Q and every degree-l block of the features
    and of the cotangent by D^l(Q) leaves L = <G, o> unchanged (o rotates with
    them), so the position gradients rotate: g(Q x) = Q g(x)."""
    w, rp, col, G, f, W = _pos_case(2, 8, 2, seed=1601)
    rng = np.random.default_rng(1602)
    Q, _ = np.linalg.qr(rng.standard_normal((3, 3)))
    if np.linalg.det(Q) < 0:
        Q[:, 0] = -Q[:, 0]
    pos = w.pos.astype(np.float64)
    c = pos.mean(axis=0)
    pos_r = (pos - c) @ Q.T + c
    f_r, G_r = f.copy(), G.copy()
    for l in range(w.L + 1):
        D = O.wigner_d(l, Q)
        sl = slice(l * l, (l + 1) ** 2)
        f_r[:, sl, :] = np.einsum("mn,anc->amc", D, f[:, sl, :])
        G_r[:, sl, :] = np.einsum("mn,anc->amc", D, G[:, sl, :])
    atoms = np.array([0, 7, 21, 40, 63])
    g = _pos_grad(w, pos, rp, col, f, W, G, atoms=atoms)
    g_r = _pos_grad(w, pos_r, rp, col, f_r, W, G_r, atoms=atoms)
    assert rel(g_r, g @ Q.T) <= 1e-8


def test_p16_position_gradient_zero_torque_for_scalars():
    """With only l = 0 features (L = 0) the loss is rotation invariant, so the
    total torque sum_a x_a x g_a vanishes."""
    w, rp, col, G, f, W = _pos_case(0, 8, 2, seed=1603)
    pos = w.pos.astype(np.float64)
    g = _pos_grad(w, pos, rp, col, f, W, G)
    torque = np.cross(pos - pos.mean(axis=0), g).sum(axis=0)
    assert np.abs(torque).max() <= 1e-8 * np.abs(np.cross(pos, g)).max()


def test_p16_position_gradient_two_atoms_closed_form():
    """Two atoms within the cutoff, L = 0, one head: each has one neighbour
    (softmax weight 1), so o_i[c] = rho(r)[c] (h_j W0)[c] with
    rho[c] = sum_k e_k(r) W_rad[k][0][c], and L = sum_i <G_i, o_i> depends on
    the positions through r = |x_1 - x_0| alone:
    dL/dx_1 = -dL/dx_0 = r_hat sum_i sum_c G_i[c] (h_j W0)[c] sum_k W_rad[k][0][c] e_k'(r),
    with e_k(r) = exp(-gamma (r - mu_k)^2) (cos(pi r / r_c) + 1) / 2 differentiated by hand."""
    rc = 5.0
    pos = np.array([[1.0, 2.0, 3.0], [2.3, 1.1, 4.2]], dtype=np.float32)
    w = make_config("tiny", L=0, C=4, H=1, geometry=(pos, None, None, {}))
    rp, col = O.neighbor_list(w.pos, w.cutoff, w.box, w.batch)
    assert col.size == 2 and abs(w.cutoff - rc) < 1e-6
    rng = np.random.default_rng(1605)
    G = rng.standard_normal((2, 1, 4))
    f = w.as_f32("feat").astype(np.float64)
    W = [w.as_f32(n).astype(np.float64) for n in ("w_q", "w_k", "w_rad", "w_so2")]
    g = _pos_grad(w, pos.astype(np.float64), rp, col, f, W, G)
    d = pos[1].astype(np.float64) - pos[0].astype(np.float64)
    r = np.linalg.norm(d)
    delta = rc / 7
    gamma = 1.0 / (2 * delta * delta)
    mu = np.arange(8) * delta
    gauss = np.exp(-gamma * (r - mu) ** 2)
    env = 0.5 * (np.cos(np.pi * r / rc) + 1)
    denv = -0.5 * np.pi / rc * np.sin(np.pi * r / rc)
    de = gauss * (-2 * gamma * (r - mu)) * env + gauss * denv          # e_k'(r)
    drho = np.einsum("k,kc->c", de, W[2][:, 0, :])                      # d rho[c] / dr
    W0 = W[3].reshape(4, 4)
    dldr = sum(float(np.sum(G[i, 0] * (f[1 - i, 0] @ W0) * drho)) for i in range(2))
    want = dldr * d / r
    assert rel(g[1], want) <= 1e-8 and rel(g[0], -want) <= 1e-8


def test_p16_position_gradient_step_size():
    """Halving the difference step changes the result by far less than the
    bounds it is held to (the truncation error falls as eps^4)."""
    w, rp, col, G, f, W = _pos_case(1, 8, 2, seed=1604)
    pos = w.pos.astype(np.float64)
    atoms = np.array([3, 30])
    a = _pos_grad(w, pos, rp, col, f, W, G, atoms=atoms, eps=1e-4)
    b = _pos_grad(w, pos, rp, col, f, W, G, atoms=atoms, eps=5e-5)
    assert rel(a, b) <= 1e-9


# ------------------------------------------------------------ radial basis --
def test_radial_basis_definition_points():
    rc = 5.0
    e = O.radial_basis(np.array([0.0, rc, rc / 7 * 3]), rc)
    assert abs(e[0, 0] - 1.0) < 1e-15                 # centre 0 at r = 0, envelope 1
    assert np.all(np.abs(e[1]) < 1e-15)               # envelope vanishes at the cutoff
    env = 0.5 * (math.cos(math.pi * 3 / 7) + 1)
    assert abs(e[2, 3] - env) < 1e-15                 # a Gaussian's own centre
    assert abs(e[2, 4] - env * math.exp(-0.5)) < 1e-15  # one width away
