"""Plain fp64 oracle of E2Former-V2's on-the-fly equivariant attention layer.

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It is slow on purpose: every edge is
materialised (in chunks of destination atoms), the softmax is two-pass, and the
Wigner-D blocks come from a least-squares fit of rotated spherical harmonics.

Source: arXiv 2601.16622, "E2Former-V2: On-the-Fly Equivariant Attention with
Linear Activation Memory".  The pages that describe it print no equations, so
every step below is the plainest reading of the English technical summary
(section 2.1 "Equivariant Axis-Aligned Sparsification" and section 2.2
"On-the-Fly Equivariant Attention") and of the author abstract.  Each function
names the passage it follows and the reading it takes.

Parity status: every function here is pinned by the CPU test suite (Lemma 4.1
sparsity, spherical-harmonic closed forms and SciPy, Wigner-D group laws, gauge
invariance, rotation equivariance, permutation invariance, an L=1 closed form,
softmax limits, online == two-pass, brute-force neighbours, and equality with a
dense Clebsch-Gordan tensor product; the convolution against the attention
layer with uniform weights; the message adjoint by the exact adjoint identity
and the feature gradient by central finite differences of the layer; the
block's norm against a library RMS norm, its gate against a library SiLU,
and the block's equivariance, permutation equivariance and residual
identity).  The conventions those invariants leave
free (edge direction, W2 sign, radial basis widths, 1/sqrt(d_h), head split, no
self loop) are readings, not facts the pages fix.
"""
from __future__ import annotations

import math
from functools import lru_cache

import numpy as np
from scipy.spatial import cKDTree

# ---------------------------------------------------------------------------
# Neighbourhoods N(i)
# ---------------------------------------------------------------------------


def _pair_test_f32(pos32, box32, i, j, rc2):
    """The exact fp32 neighbour predicate for pairs (i, j), evaluated with
    NumPy float32 arithmetic (each operation correctly rounded, no fusion):
    dx = x_j - x_i per axis; periodic wrap by one box length when |dx| > box/2;
    d2 = (dx*dx + dy*dy) + dz*dz; neighbour iff 0 < d2 < rc2.  The lower bound
    is a reading: two atoms at one point (d2 = 0 in fp32) have no edge
    direction, so they are not each other's neighbours."""
    d = pos32[j] - pos32[i]                       # float32
    if box32 is not None:
        half = np.float32(0.5) * box32
        d = np.where(d > half, d - box32, np.where(d < -half, d + box32, d)).astype(np.float32)
    sq = d * d
    d2 = (sq[..., 0] + sq[..., 1]) + sq[..., 2]
    return (d2 > 0) & (d2 < rc2)


def _csr_from_pairs(n, src_i, dst_j):
    order = np.lexsort((dst_j, src_i))
    i_s = src_i[order]
    j_s = dst_j[order].astype(np.int32)
    counts = np.bincount(i_s, minlength=n)
    row_ptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    return row_ptr, j_s


def neighbor_list(pos, cutoff, box=None, batch=None):
    """Radius graph j in N(i), |E| ~ kN (technical summary section 1, "Problem
    Statement"; section 2.2, "Streaming Reduction" iterates j in N(i)).

    Readings (the pages fix none of them): strict d < r_c, no self loop, no
    pair of atoms at one point (d = 0),
    same-batch only, minimum image in a periodic box, the fp32 predicate of
    ``_pair_test_f32``.  Rows are sorted by destination i, then ascending j.
    Candidate pairs come from a KD-tree query at a slightly larger radius
    (a library primitive); the decision itself is the fp32 predicate.
    Returns (row_ptr int64[N+1], col int32[E])."""
    pos32 = np.ascontiguousarray(pos, dtype=np.float32)
    n = pos32.shape[0]
    rc = np.float32(cutoff)
    rc2 = rc * rc
    box32 = None if box is None else np.asarray(box, dtype=np.float32)
    if n == 0:
        return np.zeros(1, dtype=np.int64), np.zeros(0, dtype=np.int32)
    slack = float(cutoff) * 1e-3 + 1e-3
    if box32 is None:
        tree = cKDTree(pos32.astype(np.float64))
    else:
        tree = cKDTree(pos32.astype(np.float64), boxsize=box32.astype(np.float64))
    pairs = tree.query_pairs(float(cutoff) + slack, output_type="ndarray")
    if pairs.size == 0:
        return np.zeros(n + 1, dtype=np.int64), np.zeros(0, dtype=np.int32)
    i = np.concatenate([pairs[:, 0], pairs[:, 1]])
    j = np.concatenate([pairs[:, 1], pairs[:, 0]])
    keep = _pair_test_f32(pos32, box32, i, j, rc2)
    if batch is not None:
        b = np.asarray(batch)
        keep &= b[i] == b[j]
    return _csr_from_pairs(n, i[keep], j[keep])


def neighbor_list_bruteforce(pos, cutoff, box=None, batch=None, block=256):
    """O(N^2) version of ``neighbor_list``: every ordered pair i != j is tested
    with the same fp32 predicate."""
    pos32 = np.ascontiguousarray(pos, dtype=np.float32)
    n = pos32.shape[0]
    rc = np.float32(cutoff)
    rc2 = rc * rc
    box32 = None if box is None else np.asarray(box, dtype=np.float32)
    src, dst = [], []
    allj = np.arange(n)
    for s in range(0, n, block):
        ii = np.arange(s, min(n, s + block))
        I = np.repeat(ii, n)
        J = np.tile(allj, ii.size)
        ok = _pair_test_f32(pos32, box32, I, J, rc2) & (I != J)
        if batch is not None:
            b = np.asarray(batch)
            ok &= b[I] == b[J]
        src.append(I[ok])
        dst.append(J[ok])
    return _csr_from_pairs(n, np.concatenate(src), np.concatenate(dst))


# ---------------------------------------------------------------------------
# Real spherical harmonics and the edge-aligned frame
# ---------------------------------------------------------------------------


def real_sph_harm(L, vecs):
    """Orthonormal real spherical harmonics Y_lm(r_hat), l = 0..L, m = -l..l,
    stored at index l*l + l + m, without the Condon-Shortley phase:

        Y_l0 = N_l0 P_l(cos t),  Y_lm = sqrt2 N_lm P_l^m(cos t) cos(m p)  (m > 0),
        Y_l,-m = sqrt2 N_lm P_l^m(cos t) sin(m p),
        N_lm = sqrt((2l+1)/(4 pi) (l-m)!/(l+m)!).

    The pages (technical summary section 2.1; the Chinese and Japanese pages
    say "real" spherical harmonics where the English page says "solid") fix
    only that the harmonics are real; any r^l factor of the solid form is taken
    to live in the radial weights.  So l = 1 is proportional to (y, z, x).

    P_l^m (1 - z^2)^(-m/2) is built by the standard three-term recursion and
    (1 - z^2)^(m/2) (cos mp, sin mp) = (Re, Im) (x + i y)^m, which is exact at
    the poles.  Input need not be normalised.  Returns [..., (L+1)^2] fp64."""
    v = np.asarray(vecs, dtype=np.float64)
    r = np.linalg.norm(v, axis=-1, keepdims=True)
    u = v / r
    x, y, z = u[..., 0], u[..., 1], u[..., 2]
    out = np.zeros(v.shape[:-1] + ((L + 1) ** 2,))
    xy = x + 1j * y
    for m in range(L + 1):
        # Q_l^m(z) = P_l^m(z) / (1 - z^2)^(m/2), no Condon-Shortley phase
        q_prev = None
        q = np.full(z.shape, float(np.prod(np.arange(2 * m - 1, 0, -2))) if m > 0 else 1.0)
        pw = xy ** m
        for l in range(m, L + 1):
            if l == m:
                q_l = q
            elif l == m + 1:
                q_prev, q = q, z * (2 * m + 1) * q
                q_l = q
            else:
                q_new = ((2 * l - 1) * z * q - (l + m - 1) * q_prev) / (l - m)
                q_prev, q = q, q_new
                q_l = q
            norm = math.sqrt((2 * l + 1) / (4 * math.pi) * math.factorial(l - m) / math.factorial(l + m))
            base = l * l + l
            if m == 0:
                out[..., base] = norm * q_l
            else:
                out[..., base + m] = math.sqrt(2.0) * norm * q_l * pw.real
                out[..., base - m] = math.sqrt(2.0) * norm * q_l * pw.imag
    return out


def edge_rotation(rhat):
    """R_ij = R_y(-theta) R_z(-phi), theta = arccos(r_z), phi = atan2(r_y, r_x),
    so that R_ij r_hat = z_hat: the SO(3) -> SO(2) change of basis that aligns
    the frame with the edge vector (technical summary section 2.1).  The angle
    about z is a free gauge; phi = atan2(0, 0) = 0 at r_hat = +-z.  [...,3,3]."""
    u = np.asarray(rhat, dtype=np.float64)
    theta = np.arccos(np.clip(u[..., 2], -1.0, 1.0))
    phi = np.arctan2(u[..., 1], u[..., 0])
    ct, st, cp, sp = np.cos(theta), np.sin(theta), np.cos(phi), np.sin(phi)
    Rz = np.zeros(u.shape[:-1] + (3, 3))
    Rz[..., 0, 0], Rz[..., 0, 1] = cp, sp
    Rz[..., 1, 0], Rz[..., 1, 1] = -sp, cp
    Rz[..., 2, 2] = 1.0
    Ry = np.zeros(u.shape[:-1] + (3, 3))
    Ry[..., 0, 0], Ry[..., 0, 2] = ct, -st
    Ry[..., 1, 1] = 1.0
    Ry[..., 2, 0], Ry[..., 2, 2] = st, ct
    return Ry @ Rz


def rotation_z(gamma):
    """Rotation by angle gamma about z. [...,3,3]."""
    g = np.asarray(gamma, dtype=np.float64)
    c, s = np.cos(g), np.sin(g)
    R = np.zeros(g.shape + (3, 3))
    R[..., 0, 0], R[..., 0, 1] = c, -s
    R[..., 1, 0], R[..., 1, 1] = s, c
    R[..., 2, 2] = 1.0
    return R


@lru_cache(maxsize=None)
def _wigner_fit_points(l):
    rng = np.random.default_rng(97 + l)
    p = rng.standard_normal((2 * (2 * l + 1) + 4, 3))
    p /= np.linalg.norm(p, axis=1, keepdims=True)
    Y = real_sph_harm(l, p)[:, l * l:(l + 1) ** 2]          # [npts, 2l+1]
    return p, np.linalg.pinv(Y.T)                             # pinv of [2l+1, npts]


def wigner_d(l, R):
    """Real Wigner-D block D^l(R), defined by Y^l(R v) = D^l(R) Y^l(v) for all
    unit v (so features transform as h^l -> D^l h^l).  Computed by a
    least-squares fit over a fixed set of generic points P:
    D^l = Y^l(R P) pinv(Y^l(P)).  [..., 2l+1, 2l+1]."""
    P, pinv = _wigner_fit_points(l)
    RP = np.einsum("...ij,pj->...pi", np.asarray(R, dtype=np.float64), P)
    Y_RP = real_sph_harm(l, RP)[..., l * l:(l + 1) ** 2]     # [..., npts, 2l+1]
    return np.einsum("...pm,pn->...mn", Y_RP, pinv)


# ---------------------------------------------------------------------------
# Radial basis, SO(2) blocks, per-edge messages
# ---------------------------------------------------------------------------


def radial_basis(r, cutoff, n_rbf=8):
    """Gaussian smearing with a cosine envelope (a reading: the pages name no
    radial basis).  mu_k = k r_c/(n_rbf-1), width = spacing, gamma = 1/(2 w^2),
    e_k(r) = exp(-gamma (r - mu_k)^2) * (cos(pi r / r_c) + 1)/2.  [..., n_rbf]."""
    r = np.asarray(r, dtype=np.float64)
    rc = float(cutoff)
    delta = rc / (n_rbf - 1)
    mu = np.arange(n_rbf) * delta
    gamma = 1.0 / (2.0 * delta * delta)
    env = 0.5 * (np.cos(np.pi * r / rc) + 1.0)
    return np.exp(-gamma * (r[..., None] - mu) ** 2) * env[..., None]


def so2_blocks(w_so2, L, C):
    """Split the flat SO(2) weights into per-m blocks.  For m = 0 one matrix
    W0 with row (l_in - m)*C + c_in and column (l_out - m)*C + c_out; for m >= 1
    two such matrices W1, W2; concatenated in m order.  Returns a list:
    [W0, (W1_1, W2_1), ..., (W1_L, W2_L)] in fp64."""
    w = np.asarray(w_so2, dtype=np.float64).ravel()
    out = []
    off = 0
    for m in range(L + 1):
        k = (L + 1 - m) * C
        if m == 0:
            out.append(w[off:off + k * k].reshape(k, k))
            off += k * k
        else:
            w1 = w[off:off + k * k].reshape(k, k)
            off += k * k
            w2 = w[off:off + k * k].reshape(k, k)
            off += k * k
            out.append((w1, w2))
    if off != w.size:
        raise ValueError(f"w_so2 has {w.size} values, expected {off}")
    return out


def edge_unit(rvec):
    """Length r and unit vector r_hat of edge vectors [..., 3].  A zero-length
    edge has no direction; the reading taken here gives it r_hat = z (the
    identity frame), so its message stays finite.  ``neighbor_list`` never
    pairs two atoms at one point; only a hand-made graph has such an edge."""
    rvec = np.asarray(rvec, dtype=np.float64)
    r = np.linalg.norm(rvec, axis=-1)
    safe = np.where(r > 0, r, 1.0)
    u = np.where((r > 0)[..., None], rvec / safe[..., None], np.array([0.0, 0.0, 1.0]))
    return r, u


def min_image(rvec, box):
    """Minimum-image difference vector in fp64 (positions in [0, box))."""
    r = np.asarray(rvec, dtype=np.float64)
    if box is None:
        return r
    b = np.asarray(box, dtype=np.float64)
    half = 0.5 * b
    return np.where(r > half, r - b, np.where(r < -half, r + b, r))


def edge_messages(rvec, h_src, w_rad, w_so2, L, C, cutoff, gauge=None, rho=None, blocks=None):
    """Value v_ij for a batch of edges, following the EAAS path (technical
    summary section 2.1 and the abstract: an SO(3) -> SO(2) change of basis
    turns the dense tensor contraction into sparse blockwise per-m maps):

      1. R_ij aligns r_hat with z; D^l = D^l(R_ij) (optionally R_z(gauge) R_ij);
      2. rotate in: x^l = D^l h_j^l, per channel;
      3. per-m SO(2) mix (the reading of the unprinted Eq. 13):
           m = 0: y_{l_out,0} = sum_{l_in} x_{l_in,0} W0[l_in, l_out]
           m > 0: y_{l_out,+m} = sum_{l_in} x_{l_in,+m} W1 - x_{l_in,-m} W2
                  y_{l_out,-m} = sum_{l_in} x_{l_in,+m} W2 + x_{l_in,-m} W1
      4. radial scale: yhat_{l,m}[c] = rho[l, c] y_{l,m}[c],
         rho[l, c] = sum_k e_k(r) W_rad[k, l, c];
      5. rotate out: v^l = D^l^T yhat^l.

    rvec [E,3] points from the destination (centre) i to the neighbour j.
    h_src [E,(L+1)^2,C].  ``rho`` overrides step 4's factor ([E, L+1, C] or a
    scalar).  Returns v [E,(L+1)^2,C] fp64."""
    rvec = np.asarray(rvec, dtype=np.float64)
    h = np.asarray(h_src, dtype=np.float64)
    E = rvec.shape[0]
    r, rhat = edge_unit(rvec)
    R = edge_rotation(rhat)
    if gauge is not None:
        R = rotation_z(gauge) @ R
    if blocks is None:
        blocks = so2_blocks(w_so2, L, C)
    D = [wigner_d(l, R) for l in range(L + 1)]
    x = [np.einsum("emn,enc->emc", D[l], h[:, l * l:(l + 1) ** 2, :]) for l in range(L + 1)]
    y = [np.zeros_like(x[l]) for l in range(L + 1)]
    # m = 0
    X0 = np.concatenate([x[l][:, l, :] for l in range(L + 1)], axis=1)
    Y0 = X0 @ blocks[0]
    for l in range(L + 1):
        y[l][:, l, :] = Y0[:, l * C:(l + 1) * C]
    # m >= 1
    for m in range(1, L + 1):
        W1, W2 = blocks[m]
        Xp = np.concatenate([x[l][:, l + m, :] for l in range(m, L + 1)], axis=1)
        Xm = np.concatenate([x[l][:, l - m, :] for l in range(m, L + 1)], axis=1)
        Yp = Xp @ W1 - Xm @ W2
        Ym = Xp @ W2 + Xm @ W1
        for l in range(m, L + 1):
            s = (l - m) * C
            y[l][:, l + m, :] = Yp[:, s:s + C]
            y[l][:, l - m, :] = Ym[:, s:s + C]
    if rho is None:
        e = radial_basis(r, cutoff, np.asarray(w_rad).shape[0])
        rho = np.einsum("ek,klc->elc", e, np.asarray(w_rad, dtype=np.float64))
    rho = np.broadcast_to(np.asarray(rho, dtype=np.float64), (E, L + 1, C))
    v = np.empty((E, (L + 1) ** 2, C))
    for l in range(L + 1):
        yh = rho[:, l, None, :] * y[l]
        v[:, l * l:(l + 1) ** 2, :] = np.einsum("enm,enc->emc", D[l], yh)
    return v


def edge_messages_vjp(rvec, g, w_rad, w_so2, L, C, cutoff, blocks=None):
    """Adjoint of ``edge_messages`` with respect to h_src: for cotangents g
    [E,(L+1)^2,C] of the messages returns dh [E,(L+1)^2,C].  Every step of the
    message is linear in h_src, so this is the transpose of each step taken in
    reverse order: dyhat^l = D^l g^l (transpose of the rotate-out), dy = rho *
    dyhat (the radial scale is diagonal), the transposed per-m blocks
      m = 0: dx_0 = dy_0 W0^T
      m > 0: dx_+ = dy_+ W1^T + dy_- W2^T,  dx_- = -dy_+ W2^T + dy_- W1^T
    and dh^l = D^l^T dx^l (transpose of the rotate-in)."""
    rvec = np.asarray(rvec, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    E = rvec.shape[0]
    r, rhat = edge_unit(rvec)
    R = edge_rotation(rhat)
    if blocks is None:
        blocks = so2_blocks(w_so2, L, C)
    D = [wigner_d(l, R) for l in range(L + 1)]
    e = radial_basis(r, cutoff, np.asarray(w_rad).shape[0])
    rho = np.einsum("ek,klc->elc", e, np.asarray(w_rad, dtype=np.float64))
    dy = [rho[:, l, None, :] * np.einsum("enm,emc->enc", D[l], g[:, l * l:(l + 1) ** 2, :]) for l in range(L + 1)]
    dx = [np.zeros_like(dy[l]) for l in range(L + 1)]
    dY0 = np.concatenate([dy[l][:, l, :] for l in range(L + 1)], axis=1)
    dX0 = dY0 @ blocks[0].T
    for l in range(L + 1):
        dx[l][:, l, :] = dX0[:, l * C:(l + 1) * C]
    for m in range(1, L + 1):
        W1, W2 = blocks[m]
        dYp = np.concatenate([dy[l][:, l + m, :] for l in range(m, L + 1)], axis=1)
        dYm = np.concatenate([dy[l][:, l - m, :] for l in range(m, L + 1)], axis=1)
        dXp = dYp @ W1.T + dYm @ W2.T
        dXm = -dYp @ W2.T + dYm @ W1.T
        for l in range(m, L + 1):
            s = (l - m) * C
            dx[l][:, l + m, :] = dXp[:, s:s + C]
            dx[l][:, l - m, :] = dXm[:, s:s + C]
    dh = np.empty((E, (L + 1) ** 2, C))
    for l in range(L + 1):
        dh[:, l * l:(l + 1) ** 2, :] = np.einsum("emn,emc->enc", D[l], dx[l])
    return dh


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------


def qk_projection(feat, w_q, w_k):
    """Query and key from SO(3)-invariant scalars (technical summary section
    2.2, "Node-Centric Factorization", Eq. 6): the plainest invariant is the
    l = 0 block, q_i = h_{i,0} W_q and k_j = h_{j,0} W_k.  fp64 [N, C] each."""
    h0 = np.asarray(feat[:, 0, :], dtype=np.float64)
    return h0 @ np.asarray(w_q, dtype=np.float64), h0 @ np.asarray(w_k, dtype=np.float64)


def segment_softmax(s, seg_start, seg_len):
    """Two-pass, numerically stable softmax of s [E, H] within each segment
    (segments are contiguous and non-empty).  Returns (alpha [E,H], lse [S,H])."""
    mx = np.maximum.reduceat(s, seg_start, axis=0)
    rep = np.repeat(np.arange(seg_start.size), seg_len)
    ex = np.exp(s - mx[rep])
    den = np.add.reduceat(ex, seg_start, axis=0)
    return ex / den[rep], mx + np.log(den)


def attention(pos, row_ptr, col, feat, w_q, w_k, w_rad, w_so2, L, C, H, cutoff, box=None,
              dest=None, chunk_edges=4096, gauge=None, rho=None, w_q_zero=False):
    """The layer's output o_i for destinations ``dest`` (default: all).

    Node-centric attention with invariant logits (technical summary section
    2.2): s_ij^h = <q_i^h, k_j^h>/sqrt(C/H), head h owning channels
    [h C/H, (h+1) C/H); alpha = softmax over j in N(i) (two-pass here; the
    pages stream it with an online softmax, which is equal up to rounding);
    o_i = sum_j alpha_ij^{h(c)} v_ij[., c] with v_ij from ``edge_messages``.
    No residual, output projection or normalisation (readings).  An empty
    N(i) gives o_i = 0 and lse = -inf.

    ``feat`` [N,(L+1)^2,C] in any float dtype (cast to fp64 on use).
    ``gauge`` (per edge, indexed like ``col``) multiplies R_ij by R_z(gauge).
    Returns (out [len(dest),(L+1)^2,C] fp64, lse [len(dest),H] fp64)."""
    pos = np.asarray(pos, dtype=np.float64)
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col = np.asarray(col, dtype=np.int64)
    n = pos.shape[0]
    dest = np.arange(n) if dest is None else np.asarray(dest, dtype=np.int64)
    K = (L + 1) ** 2
    blocks = so2_blocks(w_so2, L, C)
    h0 = np.asarray(feat[:, 0, :], dtype=np.float64)
    Wq = np.zeros((C, C)) if w_q_zero else np.asarray(w_q, dtype=np.float64)
    q = h0[dest] @ Wq
    Wk = np.asarray(w_k, dtype=np.float64)
    out = np.zeros((dest.size, K, C))
    lse = np.full((dest.size, H), -np.inf)
    head_of_c = np.arange(C) // (C // H)
    deg = row_ptr[dest + 1] - row_ptr[dest]
    t = 0
    while t < dest.size:
        # gather a chunk of destinations holding about chunk_edges edges
        u = t
        tot = 0
        while u < dest.size and (u == t or tot + deg[u] <= chunk_edges):
            tot += deg[u]
            u += 1
        sel = np.arange(t, u)
        nz = sel[deg[sel] > 0]
        if nz.size:
            e_idx = np.concatenate([np.arange(row_ptr[dest[a]], row_ptr[dest[a] + 1]) for a in nz])
            lens = deg[nz]
            starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
            dst_local = np.repeat(nz, lens)
            src = col[e_idx]
            rvec = min_image(pos[src] - pos[dest[dst_local]], box)
            h_src = np.asarray(feat[src], dtype=np.float64)
            g = None if gauge is None else np.asarray(gauge)[e_idx]
            v = edge_messages(rvec, h_src, w_rad, w_so2, L, C, cutoff, gauge=g, rho=rho, blocks=blocks)
            k_src = h0[src] @ Wk
            s = (q[dst_local] * k_src).reshape(-1, H, C // H).sum(axis=2) / math.sqrt(C // H)
            alpha, seg_lse = segment_softmax(s, starts, lens)
            contrib = alpha[:, head_of_c][:, None, :] * v
            out[nz] = np.add.reduceat(contrib, starts, axis=0)
            lse[nz] = seg_lse
        t = u
    return out, lse


def convolution(pos, row_ptr, col, feat, w_rad, w_so2, L, C, cutoff, box=None, dest=None, chunk_edges=4096):
    """The EAAS convolution stage (technical summary section 2.1, "Equivariant
    Axis-Aligned Sparsification", whose result is stated for the convolution
    stage): the same per-edge messages v_ij as the attention layer (from
    ``edge_messages``), summed over the neighbourhood with no attention
    weights, o_i = sum_{j in N(i)} v_ij.  Readings: a plain sum (no division
    by the degree), no residual or output projection; an empty N(i) gives
    o_i = 0.  Returns out [len(dest),(L+1)^2,C] fp64."""
    pos = np.asarray(pos, dtype=np.float64)
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col = np.asarray(col, dtype=np.int64)
    n = pos.shape[0]
    dest = np.arange(n) if dest is None else np.asarray(dest, dtype=np.int64)
    K = (L + 1) ** 2
    blocks = so2_blocks(w_so2, L, C)
    out = np.zeros((dest.size, K, C))
    deg = row_ptr[dest + 1] - row_ptr[dest]
    t = 0
    while t < dest.size:
        u = t
        tot = 0
        while u < dest.size and (u == t or tot + deg[u] <= chunk_edges):
            tot += deg[u]
            u += 1
        sel = np.arange(t, u)
        nz = sel[deg[sel] > 0]
        if nz.size:
            e_idx = np.concatenate([np.arange(row_ptr[dest[a]], row_ptr[dest[a] + 1]) for a in nz])
            lens = deg[nz]
            starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
            src = col[e_idx]
            rvec = min_image(pos[src] - pos[dest[np.repeat(nz, lens)]], box)
            v = edge_messages(rvec, np.asarray(feat[src], dtype=np.float64), w_rad, w_so2, L, C, cutoff,
                              blocks=blocks)
            out[nz] = np.add.reduceat(v, starts, axis=0)
        t = u
    return out


def attention_backward(pos, row_ptr, col, feat, w_q, w_k, w_rad, w_so2, L, C, H, cutoff, grad_out, box=None,
                       dest=None, chunk_edges=4096):
    """Gradient of the layer with respect to the node features, dL/dh, for a
    cotangent grad_out = dL/do [N,(L+1)^2,C] (the backward the technical
    summary section 2.2 implies for training: per-edge quantities are
    recomputed from the saved per-destination softmax statistics instead of
    being stored).  Chain rule through ``attention``:

      dv_ij     = alpha_ij^{h(c)} G_i                       (value path)
      dalpha_ij = sum_{k, c in h} G_i v_ij,  delta_i = sum_{k, c in h} G_i o_i
      ds_ij     = alpha_ij (dalpha_ij - delta_i)            (softmax)
      dq_i = sum_j ds_ij k_j / sqrt(C/H),  dk_j = sum_i ds_ij q_i / sqrt(C/H)
      dh_j = sum_{i: j in N(i)} edge_messages_vjp(r_ij, dv_ij)
             + [l = 0 block] dq_j W_q^T + dk_j W_k^T.

    Returns dh for the atoms ``dest`` (default all) [len(dest),(L+1)^2,C]
    fp64; only the destinations whose edges reach ``dest`` are evaluated."""
    pos = np.asarray(pos, dtype=np.float64)
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col = np.asarray(col, dtype=np.int64)
    n = pos.shape[0]
    dest = np.arange(n) if dest is None else np.asarray(dest, dtype=np.int64)
    K = (L + 1) ** 2
    dh_ = C // H
    blocks = so2_blocks(w_so2, L, C)
    G = np.asarray(grad_out, dtype=np.float64)
    q, k = qk_projection(np.asarray(feat, dtype=np.float64), w_q, w_k)
    head_of_c = np.arange(C) // dh_
    want = np.zeros(n, dtype=bool)
    want[dest] = True
    # centres i whose edges reach a wanted atom (as neighbour) or that are wanted themselves
    src_rows = np.repeat(np.arange(n), np.diff(row_ptr))
    centres = np.zeros(n, dtype=bool)
    centres[src_rows[want[col]]] = True
    centres |= want
    cen = np.nonzero(centres & (np.diff(row_ptr) > 0))[0]
    dfeat = np.zeros((n, K, C))
    dq = np.zeros((n, C))
    dk = np.zeros((n, C))
    deg = row_ptr[cen + 1] - row_ptr[cen]
    t = 0
    while t < cen.size:
        u = t
        tot = 0
        while u < cen.size and (u == t or tot + deg[u] <= chunk_edges):
            tot += deg[u]
            u += 1
        ci = cen[t:u]
        lens = deg[t:u]
        starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
        e_idx = np.concatenate([np.arange(row_ptr[i], row_ptr[i + 1]) for i in ci])
        i_of_e = np.repeat(ci, lens)
        j_of_e = col[e_idx]
        rvec = min_image(pos[j_of_e] - pos[i_of_e], box)
        v = edge_messages(rvec, np.asarray(feat[j_of_e], dtype=np.float64), w_rad, w_so2, L, C, cutoff,
                          blocks=blocks)
        s = (q[i_of_e] * k[j_of_e]).reshape(-1, H, dh_).sum(axis=2) / math.sqrt(dh_)
        alpha, _ = segment_softmax(s, starts, lens)
        o = np.add.reduceat(alpha[:, head_of_c][:, None, :] * v, starts, axis=0)
        Gi = G[i_of_e]
        dalpha = (Gi * v).reshape(-1, K, H, dh_).sum(axis=(1, 3))
        delta = (G[ci] * o).reshape(-1, K, H, dh_).sum(axis=(1, 3))
        ds = alpha * (dalpha - np.repeat(delta, lens, axis=0))
        dq[ci] += np.add.reduceat(np.repeat(ds, dh_, axis=1) * k[j_of_e], starts, axis=0) / math.sqrt(dh_)
        np.add.at(dk, j_of_e, np.repeat(ds, dh_, axis=1) * q[i_of_e] / math.sqrt(dh_))
        sel = want[j_of_e]
        if sel.any():
            dv = alpha[sel][:, head_of_c][:, None, :] * Gi[sel]
            dh = edge_messages_vjp(rvec[sel], dv, w_rad, w_so2, L, C, cutoff, blocks=blocks)
            np.add.at(dfeat, j_of_e[sel], dh)
        t = u
    dfeat[:, 0, :] += dq @ np.asarray(w_q, dtype=np.float64).T + dk @ np.asarray(w_k, dtype=np.float64).T
    return dfeat[dest]


def edge_messages_weight_vjp(rvec, h_src, g, w_rad, w_so2, L, C, cutoff, blocks=None):
    """Gradients of sum_e <edge_messages(r_e, h_e), g_e> with respect to the
    radial weights and the per-m SO(2) blocks, summed over the edges.  With
    the message v = D^T (rho * y), y = SO2(x), x = D h, rho = e(r) W_rad
    (the steps of ``edge_messages``), the chain rule taken step by step:

      dyhat^l = D^l g^l                          (edge-frame cotangent of rho*y)
      drho[l, c] = sum_m y^l[m][c] dyhat^l[m][c],   dW_rad[k, l, c] = sum_e e_k drho
      dy = rho * dyhat
      m = 0: dW0 = X0^T dY0
      m > 0: dW1 = Xp^T dYp + Xm^T dYm,   dW2 = -Xm^T dYp + Xp^T dYm

    (from y_+ = x_+ W1 - x_- W2 and y_- = x_+ W2 + x_- W1).  Returns
    (dw_rad [n_rbf, L+1, C], dw_so2 flat in the layout of w_so2), fp64."""
    rvec = np.asarray(rvec, dtype=np.float64)
    h = np.asarray(h_src, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    r, rhat = edge_unit(rvec)
    R = edge_rotation(rhat)
    if blocks is None:
        blocks = so2_blocks(w_so2, L, C)
    D = [wigner_d(l, R) for l in range(L + 1)]
    x = [np.einsum("emn,enc->emc", D[l], h[:, l * l:(l + 1) ** 2, :]) for l in range(L + 1)]
    e = radial_basis(r, cutoff, np.asarray(w_rad).shape[0])
    rho = np.einsum("ek,klc->elc", e, np.asarray(w_rad, dtype=np.float64))
    dyhat = [np.einsum("enm,emc->enc", D[l], g[:, l * l:(l + 1) ** 2, :]) for l in range(L + 1)]
    # y = SO2(x), as in edge_messages
    y = [np.zeros_like(x[l]) for l in range(L + 1)]
    X0 = np.concatenate([x[l][:, l, :] for l in range(L + 1)], axis=1)
    Y0 = X0 @ blocks[0]
    for l in range(L + 1):
        y[l][:, l, :] = Y0[:, l * C:(l + 1) * C]
    Xp_, Xm_ = {}, {}
    for m in range(1, L + 1):
        W1, W2 = blocks[m]
        Xp = np.concatenate([x[l][:, l + m, :] for l in range(m, L + 1)], axis=1)
        Xm = np.concatenate([x[l][:, l - m, :] for l in range(m, L + 1)], axis=1)
        Xp_[m], Xm_[m] = Xp, Xm
        Yp = Xp @ W1 - Xm @ W2
        Ym = Xp @ W2 + Xm @ W1
        for l in range(m, L + 1):
            s = (l - m) * C
            y[l][:, l + m, :] = Yp[:, s:s + C]
            y[l][:, l - m, :] = Ym[:, s:s + C]
    # radial weights
    drho = np.stack([np.sum(y[l] * dyhat[l], axis=1) for l in range(L + 1)], axis=1)   # [E, L+1, C]
    dw_rad = np.einsum("ek,elc->klc", e, drho)
    # SO(2) blocks
    dy = [rho[:, l, None, :] * dyhat[l] for l in range(L + 1)]
    parts = []
    dY0 = np.concatenate([dy[l][:, l, :] for l in range(L + 1)], axis=1)
    parts.append((X0.T @ dY0).ravel())
    for m in range(1, L + 1):
        dYp = np.concatenate([dy[l][:, l + m, :] for l in range(m, L + 1)], axis=1)
        dYm = np.concatenate([dy[l][:, l - m, :] for l in range(m, L + 1)], axis=1)
        Xp, Xm = Xp_[m], Xm_[m]
        parts.append((Xp.T @ dYp + Xm.T @ dYm).ravel())
        parts.append((-Xm.T @ dYp + Xp.T @ dYm).ravel())
    return dw_rad, np.concatenate(parts)


def attention_weight_backward(pos, row_ptr, col, feat, w_q, w_k, w_rad, w_so2, L, C, H, cutoff, grad_out,
                              box=None, chunk_edges=4096, centres=None):
    """Gradients of the layer with respect to its weights for a cotangent
    grad_out = dL/do (what training the layer needs besides dL/dh; technical
    summary section 2.2 recomputes per-edge quantities from the per-destination
    softmax statistics in the backward).  Chain rule through ``attention``,
    with ds, dq and dk as in ``attention_backward``:

      dW_q = sum_i h_{i,0}^T dq_i,   dW_k = sum_j h_{j,0}^T dk_j   (q = h_0 W_q, k = h_0 W_k)
      dW_rad, dW_so2 = sum over edges (i, j) of edge_messages_weight_vjp(r_ij, h_j, alpha_ij G_i).

    ``centres`` (default all) limits the sums to the edges of those
    destinations: every term of an edge (i, j) carries G_i (through
    alpha_ij G_i or ds_ij), so when G vanishes outside ``centres`` the result
    is the full gradient.

    Returns a dict with w_q [C, C], w_k [C, C], w_rad [n_rbf, L+1, C] and
    w_so2 (flat, the layout of w_so2), fp64."""
    pos = np.asarray(pos, dtype=np.float64)
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col = np.asarray(col, dtype=np.int64)
    n = pos.shape[0]
    K = (L + 1) ** 2
    dh_ = C // H
    blocks = so2_blocks(w_so2, L, C)
    feat = np.asarray(feat, dtype=np.float64)
    G = np.asarray(grad_out, dtype=np.float64)
    q, k = qk_projection(feat, w_q, w_k)
    head_of_c = np.arange(C) // dh_
    cen = np.nonzero(np.diff(row_ptr) > 0)[0]
    if centres is not None:
        cen = np.intersect1d(cen, np.asarray(centres, dtype=np.int64))
    dq = np.zeros((n, C))
    dk = np.zeros((n, C))
    dw_rad = np.zeros(np.asarray(w_rad).shape)
    dw_so2 = np.zeros(np.asarray(w_so2).size)
    deg = row_ptr[cen + 1] - row_ptr[cen]
    t = 0
    while t < cen.size:
        u = t
        tot = 0
        while u < cen.size and (u == t or tot + deg[u] <= chunk_edges):
            tot += deg[u]
            u += 1
        ci = cen[t:u]
        lens = deg[t:u]
        starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
        e_idx = np.concatenate([np.arange(row_ptr[i], row_ptr[i + 1]) for i in ci])
        i_of_e = np.repeat(ci, lens)
        j_of_e = col[e_idx]
        rvec = min_image(pos[j_of_e] - pos[i_of_e], box)
        v = edge_messages(rvec, feat[j_of_e], w_rad, w_so2, L, C, cutoff, blocks=blocks)
        s = (q[i_of_e] * k[j_of_e]).reshape(-1, H, dh_).sum(axis=2) / math.sqrt(dh_)
        alpha, _ = segment_softmax(s, starts, lens)
        o = np.add.reduceat(alpha[:, head_of_c][:, None, :] * v, starts, axis=0)
        Gi = G[i_of_e]
        dalpha = (Gi * v).reshape(-1, K, H, dh_).sum(axis=(1, 3))
        delta = (G[ci] * o).reshape(-1, K, H, dh_).sum(axis=(1, 3))
        ds = alpha * (dalpha - np.repeat(delta, lens, axis=0))
        dq[ci] += np.add.reduceat(np.repeat(ds, dh_, axis=1) * k[j_of_e], starts, axis=0) / math.sqrt(dh_)
        np.add.at(dk, j_of_e, np.repeat(ds, dh_, axis=1) * q[i_of_e] / math.sqrt(dh_))
        dv = alpha[:, head_of_c][:, None, :] * Gi
        gr, gs = edge_messages_weight_vjp(rvec, feat[j_of_e], dv, w_rad, w_so2, L, C, cutoff, blocks=blocks)
        dw_rad += gr
        dw_so2 += gs
        t = u
    h0 = feat[:, 0, :]
    return {"w_q": h0.T @ dq, "w_k": h0.T @ dk, "w_rad": dw_rad, "w_so2": dw_so2}


def attention_position_backward(pos, row_ptr, col, feat, w_q, w_k, w_rad, w_so2, L, C, H, cutoff, grad_out,
                                box=None, atoms=None, eps=1e-4):
    """Gradient of L = <grad_out, o> with respect to the atom positions
    (the forces of an energy are its negative), for the neighbour graph
    (row_ptr, col) held fixed: the plain definition, a derivative, taken by
    fourth-order central differences of ``attention`` in fp64 (truncation
    error O(eps^4), about 1e-14 relative at eps = 1e-4 A; rounding about
    1e-12).  The layer is smooth in the positions for a fixed graph: an edge
    enters through its unit vector (the Wigner blocks) and its length (the
    radial basis, whose envelope and its slope vanish at the cutoff).

    Moving atom a changes only the edges that touch it, so only o_a and o_i
    for i with a in N(i) change; each difference evaluates those outputs
    alone.  ``atoms`` (default all) selects the rows returned.  Returns
    [len(atoms), 3] fp64."""
    pos = np.asarray(pos, dtype=np.float64)
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col = np.asarray(col, dtype=np.int64)
    n = pos.shape[0]
    atoms = np.arange(n) if atoms is None else np.asarray(atoms, dtype=np.int64)
    G = np.asarray(grad_out, dtype=np.float64)
    src = np.repeat(np.arange(n), np.diff(row_ptr))
    out = np.zeros((atoms.size, 3))
    for t, a in enumerate(atoms):
        touched = np.unique(np.concatenate([[a], src[col == a]]))
        touched = touched[np.diff(row_ptr)[touched] > 0]
        if touched.size == 0:
            continue

        def loss(p):
            o, _ = attention(p, row_ptr, col, feat, w_q, w_k, w_rad, w_so2, L, C, H, cutoff, box=box, dest=touched)
            return float(np.sum(G[touched] * o))

        for d in range(3):
            def at(h):
                p = pos.copy()
                p[a, d] += h
                return loss(p)
            out[t, d] = (-at(2 * eps) + 8 * at(eps) - 8 * at(-eps) + at(-2 * eps)) / (12 * eps)
    return out


def attention_online(pos, row_ptr, col, feat, w_q, w_k, w_rad, w_so2, L, C, H, cutoff, box=None,
                     dest=None, block=5):
    """Same layer with the streaming reduction of technical summary section 2.2
    ("Streaming Reduction", "Online Softmax"): neighbours are visited in blocks
    of ``block``; a running max m_h, normaliser l_h and value accumulator are
    rescaled by exp(m_old - m_new) as each block arrives.  Used only to check
    that the streamed form equals the two-pass form."""
    pos = np.asarray(pos, dtype=np.float64)
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col = np.asarray(col, dtype=np.int64)
    n = pos.shape[0]
    dest = np.arange(n) if dest is None else np.asarray(dest, dtype=np.int64)
    K = (L + 1) ** 2
    blocks = so2_blocks(w_so2, L, C)
    q, k = qk_projection(np.asarray(feat, dtype=np.float64), w_q, w_k)
    head_of_c = np.arange(C) // (C // H)
    out = np.zeros((dest.size, K, C))
    lse = np.full((dest.size, H), -np.inf)
    for a, i in enumerate(dest):
        m_run = np.full(H, -np.inf)
        l_run = np.zeros(H)
        acc = np.zeros((K, C))
        for b0 in range(row_ptr[i], row_ptr[i + 1], block):
            e = np.arange(b0, min(b0 + block, row_ptr[i + 1]))
            src = col[e]
            rvec = min_image(pos[src] - pos[i], box)
            v = edge_messages(rvec, np.asarray(feat[src], dtype=np.float64), w_rad, w_so2, L, C,
                              cutoff, blocks=blocks)
            s = (q[i] * k[src]).reshape(-1, H, C // H).sum(axis=2) / math.sqrt(C // H)
            m_new = np.maximum(m_run, s.max(axis=0))
            scale = np.exp(m_run - m_new)
            p = np.exp(s - m_new)
            l_run = l_run * scale + p.sum(axis=0)
            acc = acc * scale[head_of_c][None, :] + np.einsum("ec,ekc->kc", p[:, head_of_c], v)
            m_run = m_new
        if row_ptr[i + 1] > row_ptr[i]:
            out[a] = acc / l_run[head_of_c][None, :]
            lse[a] = m_run + np.log(l_run)
    return out, lse


# ---------------------------------------------------------------------------
# One block around the layer
# ---------------------------------------------------------------------------
#
# The pages place the on-the-fly attention layer inside the E2Former-V2 model
# (abstract; technical summary section 2 "Methodology") but print none of the
# block around it.  The readings below are the plainest equivariant block:
# a pre-norm residual block, h1 = h + Proj(Attn(Norm1(h))), then
# h2 = h1 + FFN(Norm2(h1)); every node-wise map acts on channels only and is
# the same for every m of a degree (or gates by invariant scalars), so it
# commutes with rotations.

NORM_EPS = 1e-6


def degree_rms_norm(h, gamma, L, eps=NORM_EPS):
    """Per-degree RMS normalisation (a reading): for each atom and degree l,
    n[l,m,c] = gamma[l,c] h[l,m,c] / sqrt(mean over (m, c) of h[l,m,c]^2 + eps).
    Rotations mix m within a degree and keep that mean, so the map is
    equivariant.  h [N,(L+1)^2,C], gamma [L+1,C].  fp64."""
    h = np.asarray(h, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)
    out = np.empty_like(h)
    for l in range(L + 1):
        blk = h[:, l * l:(l + 1) ** 2, :]
        rms = np.sqrt(np.mean(blk * blk, axis=(1, 2)) + eps)
        out[:, l * l:(l + 1) ** 2, :] = blk / rms[:, None, None] * g[l][None, None, :]
    return out


def degree_linear(x, w, L):
    """Per-degree channel map y[l,m,:] = x[l,m,:] W[l] (a reading of the
    node-wise projection: one C_in x C_out matrix per degree, no bias).
    x [N,(L+1)^2,C_in], w [L+1,C_in,C_out].  fp64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    out = np.empty(x.shape[:2] + (w.shape[2],))
    for l in range(L + 1):
        out[:, l * l:(l + 1) ** 2, :] = x[:, l * l:(l + 1) ** 2, :] @ w[l]
    return out


def gated_ffn(n, w1, w_gate, w2, L, C):
    """Gated feed-forward (a reading): u = degree_linear(n, W1);
    z = n[l=0] W_gate (C -> L C); act[l=0] = SiLU(u[0]);
    act[l>=1][m][c] = u[l][m][c] sigmoid(z[(l-1) C + c]) (an invariant gate
    per channel, shared by every m of the degree); f = degree_linear(act, W2).
    n [N,(L+1)^2,C]; w1, w2 [L+1,C,C]; w_gate [C, L C].  fp64."""
    n = np.asarray(n, dtype=np.float64)
    u = degree_linear(n, w1, L)
    z = n[:, 0, :] @ np.asarray(w_gate, dtype=np.float64)
    act = np.empty_like(u)
    s = u[:, 0, :]
    # exp(-x) overflows to inf for x < -709: 1 / (1 + inf) = 0 and s / inf = -0
    # are then the exact limits, so the overflow is expected, not an error
    with np.errstate(over="ignore"):
        act[:, 0, :] = s / (1.0 + np.exp(-s))
        for l in range(1, L + 1):
            gate = 1.0 / (1.0 + np.exp(-z[:, (l - 1) * C:l * C]))
            act[:, l * l:(l + 1) ** 2, :] = u[:, l * l:(l + 1) ** 2, :] * gate[:, None, :]
    return degree_linear(act, w2, L)


def block(pos, row_ptr, col, h, bw, L, C, H, cutoff, box=None, dest=None):
    """One block: h1 = h + degree_linear(attention(Norm1(h)), W_o);
    out = h1 + gated_ffn(Norm2(h1)).  ``bw`` holds the block's weights:
    norm1, norm2 [L+1,C]; w_q, w_k [C,C]; w_rad [8,L+1,C]; w_so2 (flat);
    w_o, w_1, w_2 [L+1,C,C]; w_gate [C,L C].  The residual stream h is read
    as given (fp64).  ``dest`` selects the output rows (the attention reads
    Norm1 of every neighbour).  Returns [len(dest),(L+1)^2,C] fp64."""
    h = np.asarray(h, dtype=np.float64)
    n = h.shape[0]
    dest = np.arange(n) if dest is None else np.asarray(dest, dtype=np.int64)
    n1 = degree_rms_norm(h, bw["norm1"], L)
    a, _ = attention(pos, row_ptr, col, n1, bw["w_q"], bw["w_k"], bw["w_rad"], bw["w_so2"], L, C, H, cutoff,
                     box=box, dest=dest)
    h1 = h[dest] + degree_linear(a, bw["w_o"], L)
    n2 = degree_rms_norm(h1, bw["norm2"], L)
    return h1 + gated_ffn(n2, bw["w_1"], bw["w_gate"], bw["w_2"], L, C)
