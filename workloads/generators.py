"""Seeded synthetic workloads for the on-the-fly equivariant attention layer.

The pages (arXiv 2601.16622, "E2Former-V2: On-the-Fly Equivariant Attention with
Linear Activation Memory") evaluate on drug-like molecules (SPICE), bulk water,
a solvated protein of about 30k atoms and 100k-atom OMol25-scale systems
(English technical summary, section 4 "Experimental Results").  None of those
datasets is used: every input here is drawn from a seeded NumPy PCG64 stream
with the shapes, densities and neighbour counts of those workloads.

Draw order for every config: geometry, then node features ~N(0,1) of shape
[N, (L+1)^2, C], then weights ~N(0, 1/C) in the order W_q [C,C], W_k [C,C],
W_rad [n_rbf, L+1, C], and the SO(2) blocks (m ascending, W1 before W2).
Values are drawn in fp64, rounded to fp32 and, for bf16 configs, rounded again
to bf16 with round-to-nearest-even.  bf16 arrays are kept as uint16 bit
patterns; ``as_f32`` widens them exactly.

Nothing in this module computes any part of the layer.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
from scipy.spatial import cKDTree

N_RBF = 8
FEAT_CHUNK_NODES = 4096

# ---------------------------------------------------------------------------
# bf16 helpers (storage only)
# ---------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 -> bf16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 value, returned as fp32."""
    return bf16_to_f32(f32_to_bf16_bits(x))


def so2_param_count(L: int, C: int) -> int:
    """Number of SO(2) mixing weights: one [(L+1)C]^2 block for m=0, two
    [(L+1-m)C]^2 blocks (W1, W2) for each m >= 1."""
    n = ((L + 1) * C) ** 2
    for m in range(1, L + 1):
        n += 2 * ((L + 1 - m) * C) ** 2
    return n


# ---------------------------------------------------------------------------
# Workload container
# ---------------------------------------------------------------------------


@dataclass
class Workload:
    name: str
    pos: np.ndarray                 # float32 [N, 3]
    box: Optional[np.ndarray]       # float32 [3] (periodic) or None (open)
    batch: Optional[np.ndarray]     # int32 [N] or None
    cutoff: float                   # an fp32-representable value
    L: int
    C: int
    H: int
    dtype: str                      # "f32" or "bf16"
    feat: np.ndarray                # f32 [N,(L+1)^2,C] or uint16 bf16 bits
    w_q: np.ndarray                 # [C, C]
    w_k: np.ndarray                 # [C, C]
    w_rad: np.ndarray               # [n_rbf, L+1, C]
    w_so2: np.ndarray               # flat, logical layout
    n_rbf: int = N_RBF
    meta: dict = field(default_factory=dict)

    @property
    def n_atoms(self) -> int:
        return int(self.pos.shape[0])

    @property
    def ncomp(self) -> int:
        return (self.L + 1) ** 2

    def as_f32(self, name: str, rows=None) -> np.ndarray:
        """fp32 values of a stored array (bf16 bits are widened exactly)."""
        a = getattr(self, name)
        if rows is not None:
            a = a[rows]
        if a.dtype == np.uint16:
            return bf16_to_f32(a)
        return np.asarray(a, dtype=np.float32)


# ---------------------------------------------------------------------------
# Random helpers
# ---------------------------------------------------------------------------


def _unit_vectors(rng: np.random.Generator, n: int) -> np.ndarray:
    v = rng.standard_normal((n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def _quat_to_matrix(q: np.ndarray) -> np.ndarray:
    q = q / np.linalg.norm(q, axis=-1, keepdims=True)
    w, x, y, z = q[..., 0], q[..., 1], q[..., 2], q[..., 3]
    R = np.empty(q.shape[:-1] + (3, 3))
    R[..., 0, 0] = 1 - 2 * (y * y + z * z)
    R[..., 0, 1] = 2 * (x * y - w * z)
    R[..., 0, 2] = 2 * (x * z + w * y)
    R[..., 1, 0] = 2 * (x * y + w * z)
    R[..., 1, 1] = 1 - 2 * (x * x + z * z)
    R[..., 1, 2] = 2 * (y * z - w * x)
    R[..., 2, 0] = 2 * (x * z - w * y)
    R[..., 2, 1] = 2 * (y * z + w * x)
    R[..., 2, 2] = 1 - 2 * (x * x + y * y)
    return R


def _to_f32_periodic(pos64: np.ndarray, box: np.ndarray) -> np.ndarray:
    """Wrap into [0, box), round to fp32, and map any value equal to box to 0."""
    p = np.mod(pos64, box)
    p32 = p.astype(np.float32)
    b32 = box.astype(np.float32)
    for d in range(3):
        col = p32[:, d]
        col[col >= b32[d]] = np.float32(0.0)
        col[col < 0] = np.float32(0.0)
    return p32


def _water_template() -> np.ndarray:
    """Rigid H2O: O at the origin, O-H 0.96 A, H-O-H 104.5 degrees."""
    half = np.deg2rad(104.5) / 2
    d = 0.96
    return np.array([[0.0, 0.0, 0.0],
                     [d * np.sin(half), 0.0, d * np.cos(half)],
                     [-d * np.sin(half), 0.0, d * np.cos(half)]])


def _waters_at(rng: np.random.Generator, sites: np.ndarray, jitter: float) -> np.ndarray:
    """One randomly oriented water per site (O on the jittered site). [n,3,3]."""
    n = sites.shape[0]
    o = sites + rng.uniform(-jitter, jitter, size=(n, 3))
    R = _quat_to_matrix(rng.standard_normal((n, 4)))
    tpl = _water_template()
    return o[:, None, :] + np.einsum("nij,aj->nai", R, tpl)


# ---------------------------------------------------------------------------
# Geometry recipes
# ---------------------------------------------------------------------------


def _geom_tiny(rng):
    pos = rng.uniform(0.0, 9.0, size=(64, 3)).astype(np.float32)
    return pos, None, None, {}


def _random_walk_molecule(rng, n, bond_lo, bond_hi, dmin, max_tries=2000):
    pts = [np.zeros(3)]
    while len(pts) < n:
        placed = False
        arr = np.asarray(pts)
        for _ in range(max_tries):
            step = _unit_vectors(rng, 1)[0] * rng.uniform(bond_lo, bond_hi)
            cand = arr[-1] + step
            if np.min(np.linalg.norm(arr - cand, axis=1)) >= dmin:
                pts.append(cand)
                placed = True
                break
        if not placed:  # trapped: branch from a random earlier atom instead
            k = int(rng.integers(0, len(pts)))
            step = _unit_vectors(rng, 1)[0] * rng.uniform(bond_lo, bond_hi)
            cand = arr[k] + step
            if np.min(np.linalg.norm(arr - cand, axis=1)) >= dmin:
                pts.append(cand)
    return np.asarray(pts)


def _geom_drug(rng, at_origin=False, cutoff=5.0):
    n_mol = 256
    sizes = rng.integers(16, 101, size=n_mol)
    mols = []
    elems = []
    for b in range(n_mol):
        m = _random_walk_molecule(rng, int(sizes[b]), 1.0, 1.5, 1.0)
        mols.append(m - m.mean(axis=0))
        elems.append(rng.choice(6, size=int(sizes[b]), p=[0.5, 0.3, 0.08, 0.08, 0.02, 0.02]))
    extent = max(float(np.max(m.max(axis=0) - m.min(axis=0))) for m in mols)
    spacing = float(np.ceil(extent + cutoff + 1.0))
    pos = []
    batch = []
    for b, m in enumerate(mols):
        if at_origin:
            site = np.zeros(3)
        else:
            site = np.array([b % 8, (b // 8) % 8, b // 64], dtype=np.float64) * spacing
        pos.append(m + site)
        batch.append(np.full(m.shape[0], b, dtype=np.int32))
    pos = np.concatenate(pos).astype(np.float32)
    batch = np.concatenate(batch)
    meta = {"elements": np.concatenate(elems).astype(np.int8), "grid_spacing": spacing,
            "element_symbols": ["H", "C", "N", "O", "F", "S"]}
    return pos, None, batch, meta


WATER_DENSITY = 0.03343  # molecules per cubic angstrom at 1.0 g/cm^3


def _water_box_side(n_water: int) -> float:
    grams = n_water * 18.01528 / 6.02214076e23
    return float((grams / 1.0 * 1e24) ** (1.0 / 3.0))


def _geom_water(rng):
    n_water = 3000
    box_side = _water_box_side(n_water)           # 44.771 A
    n_lat = 15
    spacing = box_side / n_lat                    # 2.985 A
    site_ids = rng.choice(n_lat ** 3, size=n_water, replace=False)
    ijk = np.stack(np.unravel_index(site_ids, (n_lat,) * 3), axis=1).astype(np.float64)
    mols = _waters_at(rng, ijk * spacing, 0.15)
    box = np.full(3, box_side)
    pos = _to_f32_periodic(mols.reshape(-1, 3), box)
    return pos, box.astype(np.float32), None, {"n_water": n_water}


def _polymer_in_sphere(rng, n, radius, centre, bond=1.5, dmin=1.2, max_tries=200):
    """Self-avoiding random walk confined to a sphere, with backtracking."""
    cell = dmin
    grid: dict = {}
    pts = np.zeros((n, 3))

    def key(p):
        return tuple(np.floor(p / cell).astype(np.int64))

    def ok(p, upto):
        if np.linalg.norm(p - centre) > radius:
            return False
        k = key(p)
        for dx in (-1, 0, 1):
            for dy in (-1, 0, 1):
                for dz in (-1, 0, 1):
                    for idx in grid.get((k[0] + dx, k[1] + dy, k[2] + dz), ()):
                        if idx < upto and np.linalg.norm(pts[idx] - p) < dmin:
                            return False
        return True

    def add(idx, p):
        pts[idx] = p
        grid.setdefault(key(p), []).append(idx)

    def remove(idx):
        grid[key(pts[idx])].remove(idx)

    add(0, centre.copy())
    i = 1
    fails = 0
    while i < n:
        placed = False
        for _ in range(max_tries):
            cand = pts[i - 1] + _unit_vectors(rng, 1)[0] * bond
            if ok(cand, i):
                add(i, cand)
                i += 1
                placed = True
                break
        if not placed:
            fails += 1
            back = min(i - 1, 5 + fails % 20)
            for _ in range(back):
                i -= 1
                remove(i)
    return pts


# Frozen box side for the protein-in-water config: chosen once by scanning
# 64.0-72.0 A in 0.1 A steps with the seed below and keeping the side whose
# total atom count is closest to 30,000 (see _protein_total).
PROTEIN_BOX_SIDE = 67.1


def _protein_waters(box_side, poly, seed=(4, 1)):
    wrng = np.random.default_rng(list(seed))
    n_lat = max(1, int(round(box_side / 2.985)))
    spacing = box_side / n_lat
    g = np.arange(n_lat, dtype=np.float64) * spacing
    sites = np.stack(np.meshgrid(g, g, g, indexing="ij"), axis=-1).reshape(-1, 3)
    mols = _waters_at(wrng, sites, 0.15)
    box = np.full(3, box_side)
    tree = cKDTree(np.mod(poly, box), boxsize=box_side)
    d, _ = tree.query(np.mod(mols.reshape(-1, 3), box), k=1)
    clash = (d < 2.4).reshape(-1, 3).any(axis=1)
    avail = np.nonzero(~clash)[0]
    n_water = int(round(WATER_DENSITY * avail.size * spacing ** 3))
    n_water = min(n_water, avail.size)
    chosen = np.sort(wrng.choice(avail, size=n_water, replace=False))
    return mols[chosen], spacing


def _protein_total(box_side, poly):
    w, _ = _protein_waters(box_side, poly)
    return poly.shape[0] + 3 * w.shape[0]


def _geom_protein(rng, box_side=PROTEIN_BOX_SIDE):
    centre = np.full(3, box_side / 2)
    poly = _polymer_in_sphere(rng, 4000, 21.0, centre)
    poly_el = rng.choice(4, size=4000, p=[0.62, 0.17, 0.19, 0.02])
    waters, spacing = _protein_waters(box_side, poly)
    pos64 = np.concatenate([poly, waters.reshape(-1, 3)])
    box = np.full(3, box_side)
    pos = _to_f32_periodic(pos64, box)
    meta = {"n_polymer": 4000, "n_water": waters.shape[0], "lattice_spacing": spacing,
            "polymer_elements": poly_el.astype(np.int8), "element_symbols": ["C", "N", "O", "S"]}
    return pos, box.astype(np.float32), None, meta


def _rsa_periodic(rng, n, box_side, dmin, batch=20000):
    """Random sequential addition with a minimum-image separation."""
    acc = np.zeros((0, 3))
    while acc.shape[0] < n:
        cand = rng.uniform(0.0, box_side, size=(batch, 3))
        if acc.shape[0]:
            d, _ = cKDTree(acc, boxsize=box_side).query(cand, k=1)
            cand = cand[d >= dmin]
        # resolve conflicts inside the batch in draw order
        pairs = cKDTree(cand, boxsize=box_side).query_pairs(dmin, output_type="ndarray")
        keep = np.ones(cand.shape[0], dtype=bool)
        if pairs.size:
            pairs = np.sort(pairs, axis=1)
            later_of = {}
            for a, b in pairs:
                later_of.setdefault(int(b), []).append(int(a))
            for b in sorted(later_of):
                if any(keep[a] for a in later_of[b]):
                    keep[b] = False
        cand = cand[keep]
        acc = np.concatenate([acc, cand[: n - acc.shape[0]]])
    return acc


def _geom_large(rng):
    box_side = 100.0
    pos64 = _rsa_periodic(rng, 100_000, box_side, 0.9)
    box = np.full(3, box_side)
    return _to_f32_periodic(pos64, box), box.astype(np.float32), None, {}


# ---------------------------------------------------------------------------
# Config table
# ---------------------------------------------------------------------------

CONFIGS = {
    # name: (seed, geometry, cutoff, L, C, H, dtype)
    "tiny": (1, _geom_tiny, 5.0, 1, 16, 1, "f32"),
    "drug": (2, _geom_drug, 5.0, 3, 128, 8, "bf16"),
    "drug_origin": (2, lambda r: _geom_drug(r, at_origin=True), 5.0, 3, 128, 8, "bf16"),
    "water": (3, _geom_water, 6.0, 3, 128, 8, "bf16"),
    "protein": (4, _geom_protein, 5.0, 3, 128, 8, "bf16"),
    "large": (5, _geom_large, 5.0, 4, 128, 8, "bf16"),
}


def _draw_features(rng, n, ncomp, C, dtype):
    if dtype == "bf16":
        out = np.empty((n, ncomp, C), dtype=np.uint16)
    else:
        out = np.empty((n, ncomp, C), dtype=np.float32)
    for s in range(0, n, FEAT_CHUNK_NODES):
        e = min(n, s + FEAT_CHUNK_NODES)
        blk = rng.standard_normal((e - s, ncomp, C)).astype(np.float32)
        out[s:e] = f32_to_bf16_bits(blk) if dtype == "bf16" else blk
    return out


def _draw_weight(rng, shape, C, dtype):
    w = (rng.standard_normal(shape) / np.sqrt(C)).astype(np.float32)
    return f32_to_bf16_bits(w) if dtype == "bf16" else w


def make_config(name: str, seed: Optional[int] = None, *, L=None, C=None, H=None,
                dtype=None, geometry=None) -> Workload:
    """Build one named workload.  Keyword overrides give smaller variants of the
    same geometry (e.g. the drug-like batch at L=1, C=32)."""
    base_seed, geom_fn, cutoff, L0, C0, H0, dt0 = CONFIGS[name]
    seed = base_seed if seed is None else seed
    L = L0 if L is None else L
    C = C0 if C is None else C
    H = H0 if H is None else H
    dtype = dt0 if dtype is None else dtype
    rng = np.random.default_rng(seed)
    if geometry is None:
        pos, box, batch, meta = geom_fn(rng)
    else:
        pos, box, batch, meta = geometry
    n = pos.shape[0]
    ncomp = (L + 1) ** 2
    feat = _draw_features(rng, n, ncomp, C, dtype)
    w_q = _draw_weight(rng, (C, C), C, dtype)
    w_k = _draw_weight(rng, (C, C), C, dtype)
    w_rad = _draw_weight(rng, (N_RBF, L + 1, C), C, dtype)
    blocks = []
    for m in range(L + 1):
        k = (L + 1 - m) * C
        for _ in range(1 if m == 0 else 2):
            blocks.append(_draw_weight(rng, (k * k,), C, dtype))
    w_so2 = np.concatenate(blocks)
    return Workload(name=name, pos=np.ascontiguousarray(pos, dtype=np.float32), box=box,
                    batch=batch, cutoff=float(np.float32(cutoff)), L=L, C=C, H=H, dtype=dtype,
                    feat=feat, w_q=w_q, w_k=w_k, w_rad=w_rad, w_so2=w_so2, meta=meta)


def isolated_atom_variant(w: Workload, far: float = 1000.0) -> Workload:
    """A copy of an open-boundary workload with one extra atom far from all others
    (its neighbour list is empty)."""
    assert w.box is None
    pos = np.concatenate([w.pos, np.array([[far, far, far]], dtype=np.float32)])
    feat = np.concatenate([w.feat, w.feat[:1]])
    batch = None if w.batch is None else np.concatenate([w.batch, w.batch[:1]])
    return Workload(name=w.name + "+isolated", pos=pos, box=None, batch=batch, cutoff=w.cutoff,
                    L=w.L, C=w.C, H=w.H, dtype=w.dtype, feat=feat, w_q=w.w_q, w_k=w.w_k,
                    w_rad=w.w_rad, w_so2=w.w_so2, meta=dict(w.meta))


def axis_lattice_geometry(n_side: int = 4, spacing: float = 1.5):
    """Open-boundary cubic lattice of n_side^3 atoms with the given spacing
    (exact in fp32): every lattice row gives edges exactly along +-x, +-y and
    +-z, so the edge frame meets its poles (r_hat = +-z) and the axes.
    Returns a ``make_config`` geometry tuple."""
    g = np.arange(n_side, dtype=np.float64) * spacing
    pos = np.stack(np.meshgrid(g, g, g, indexing="ij"), axis=-1).reshape(-1, 3) + 1.0
    return pos.astype(np.float32), None, None, {"kind": "axis lattice", "spacing": spacing}


def coincident_geometry(rng: np.random.Generator, n: int = 64, n_dup: int = 6, side: float = 9.0):
    """``n`` atoms uniform in an open cube, then ``n_dup`` of them duplicated
    at exactly the same fp32 coordinates (two atoms at one point)."""
    pos = rng.uniform(0.0, side, size=(n, 3)).astype(np.float32)
    dup = rng.choice(n, size=n_dup, replace=False)
    pos = np.concatenate([pos, pos[dup]])
    return pos, None, None, {"kind": "coincident", "duplicated": dup.tolist()}


BLOCK_NODE_WEIGHTS = ("norm1", "w_o", "norm2", "w_1", "w_gate", "w_2")
ATTN_WEIGHTS = ("w_q", "w_k", "w_rad", "w_so2")


def make_block_weights(w: Workload, index: int = 0) -> dict:
    """Weights of block ``index`` around the attention layer of workload w,
    in w's storage (fp32, or bf16 bits).  Drawn from their own seeded stream
    (seed (base seed, 1000 + index)), so the workload's own draws do not
    change: norm gains 1 + 0.1 N(0,1) [L+1, C]; W_o, W_1, W_2 [L+1, C, C] and
    W_gate [C, L C] ~ N(0, 1/C).  Block 0 takes the workload's attention
    weights; later blocks draw their own (W_q, W_k, W_rad, W_so2, same
    shapes and scales)."""
    base = CONFIGS[w.name][0] if w.name in CONFIGS else 0
    rng = np.random.default_rng((base, 1000 + index))
    L, C = w.L, w.C

    def store(x):
        x = np.asarray(x, dtype=np.float32)
        return f32_to_bf16_bits(x) if w.dtype == "bf16" else x

    out = {
        "norm1": store(1.0 + 0.1 * rng.standard_normal((L + 1, C))),
        "w_o": _draw_weight(rng, (L + 1, C, C), C, w.dtype),
        "norm2": store(1.0 + 0.1 * rng.standard_normal((L + 1, C))),
        "w_1": _draw_weight(rng, (L + 1, C, C), C, w.dtype),
        "w_gate": _draw_weight(rng, (C, L * C), C, w.dtype),
        "w_2": _draw_weight(rng, (L + 1, C, C), C, w.dtype),
    }
    if index == 0:
        for k in ATTN_WEIGHTS:
            out[k] = getattr(w, k)
    else:
        out["w_q"] = _draw_weight(rng, (C, C), C, w.dtype)
        out["w_k"] = _draw_weight(rng, (C, C), C, w.dtype)
        out["w_rad"] = _draw_weight(rng, (N_RBF, L + 1, C), C, w.dtype)
        blocks = []
        for m in range(L + 1):
            k = (L + 1 - m) * C
            for _ in range(1 if m == 0 else 2):
                blocks.append(_draw_weight(rng, (k * k,), C, w.dtype))
        out["w_so2"] = np.concatenate(blocks)
    return out


def block_weights_f32(bw: dict) -> dict:
    """fp32 values of stored block weights (bf16 bits widened exactly)."""
    return {k: (bf16_to_f32(v) if v.dtype == np.uint16 else np.asarray(v, dtype=np.float32)) for k, v in bw.items()}
