"""Seeded synthetic inputs for the Tessera hot path (positions, species, weights, velocities).

This module holds input generation only: it contains none of the method's arithmetic (no
wrapping, keys, neighbour tests, model or integrator). Both the GPU path and the fp64
oracle receive exactly the arrays produced here.

Workloads follow the systems the Tessera abstract (Ab Initio Accuracy Beyond the Cutoff,
abstract) runs on: a salt solution (water-density box with Na/Cl) and a virus capsid
(protein shell in water). Neither structure nor trained weights exist here, so each is a
seeded stand-in of the same shape, density and species mix:

  water648  648 atoms: 216 O on a jittered 6x6x6 lattice + 2 H each at 0.96 A (box 18.6 A)
  salt4k    4,096 atoms at 0.1 atoms/A^3 (box 34.5 A), H/O/Na/Cl, 0.9 A exclusion
  salt60k   60,000 atoms at 0.1 atoms/A^3 (box 84.34 A): one GPU's share of 30.7M/512
  capsid39k 39,300 atoms: a protein-density (0.12) curved shell section in water (0.1)
  salt500k  500,000 atoms at 0.1 atoms/A^3 (box 171 A)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
from scipy.spatial import cKDTree

# Standard atomic weights (amu).
MASS = {"H": 1.008, "C": 12.011, "N": 14.007, "O": 15.999, "Ow": 15.999,
        "Na": 22.990, "S": 32.06, "Cl": 35.45}
# Boltzmann constant (eV/K) and 1 eV/amu expressed in A^2/fs^2, used only to draw
# Maxwell velocities in A/fs.
KB_EV = 8.617333262e-5
EV_PER_AMU_A2FS2 = 9.648533e-3

MIN_SEP = 0.9  # A, exclusion distance for random sequential addition


@dataclass
class ModelSpec:
    n_species: int
    n_layers: int
    channels: int
    l_max: int
    n_heads: int
    n_rbf: int = 8
    radial_hidden: int = 64
    r_cut: float = 5.75

    @property
    def n_paths(self) -> int:
        return sum(1 for l1 in range(self.l_max + 1) for l2 in range(self.l_max + 1)
                   for l3 in range(self.l_max + 1)
                   if abs(l1 - l2) <= l3 <= l1 + l2 and (l1 + l2 + l3) % 2 == 0)

    def as_tuple(self):
        return (self.n_species, self.n_layers, self.channels, self.l_max, self.n_heads,
                self.n_rbf, self.radial_hidden, float(self.r_cut))


@dataclass
class Workload:
    name: str
    box: np.ndarray          # float32[3]
    pos: np.ndarray          # float32[N,3]
    species: np.ndarray      # int32[N]
    species_names: list
    model: ModelSpec
    skin: float = 1.0
    dt_fs: float = 0.5
    rebuild_every: int = 20
    extra: dict = field(default_factory=dict)

    @property
    def n(self) -> int:
        return int(self.pos.shape[0])

    def masses(self) -> np.ndarray:
        return np.array([MASS[s] for s in self.species_names], dtype=np.float64)


def _rsa_fill(rng, n_target, box, accept_region=None, existing=None, batch=None):
    """Random sequential addition in a periodic box: uniform proposals, each accepted
    only if no accepted atom lies within MIN_SEP (minimum image). Proposals are handled
    in seeded batches; inside a batch they are accepted greedily in proposal order."""
    L = float(box[0])
    acc = [] if existing is None else [existing]
    n_have = 0 if existing is None else existing.shape[0]
    n_new = 0
    batch = batch or max(256, n_target // 4)
    out = []
    while n_new < n_target:
        props = rng.uniform(0.0, L, size=(batch, 3))
        if accept_region is not None:
            props = props[accept_region(props)]
            if props.shape[0] == 0:
                continue
        ok = np.ones(props.shape[0], dtype=bool)
        if n_have + n_new > 0:
            allpts = np.concatenate(acc + out, axis=0) if out else np.concatenate(acc, axis=0)
            tree = cKDTree(np.mod(allpts, L), boxsize=L)
            d, _ = tree.query(np.mod(props, L), k=1)
            ok &= d >= MIN_SEP
        cand = props[ok]
        if cand.shape[0] == 0:
            continue
        t2 = cKDTree(np.mod(cand, L), boxsize=L)
        pairs = t2.query_pairs(MIN_SEP, output_type="ndarray")
        keep = np.ones(cand.shape[0], dtype=bool)
        if pairs.size:
            nbrs = [[] for _ in range(cand.shape[0])]
            for a, b in pairs:
                lo, hi = (a, b) if a < b else (b, a)
                nbrs[hi].append(lo)
            for idx in range(cand.shape[0]):
                if any(keep[p] for p in nbrs[idx]):
                    keep[idx] = False
        cand = cand[keep][: n_target - n_new]
        out.append(cand)
        n_new += cand.shape[0]
    return np.concatenate(out, axis=0)


def _species_by_fraction(rng, n, fractions):
    """Largest-remainder rounding of n * fractions, then a seeded shuffle."""
    f = np.asarray(fractions, dtype=np.float64)
    raw = n * f / f.sum()
    cnt = np.floor(raw).astype(np.int64)
    rem = n - cnt.sum()
    order = np.argsort(-(raw - cnt), kind="stable")
    cnt[order[:rem]] += 1
    sp = np.repeat(np.arange(len(f), dtype=np.int32), cnt)
    rng.shuffle(sp)
    return sp


def water648(seed: int = 1001) -> Workload:
    rng = np.random.default_rng(seed)
    L = 18.6
    a = L / 6
    o = []
    for ix in range(6):
        for iy in range(6):
            for iz in range(6):
                o.append([(ix + 0.5) * a, (iy + 0.5) * a, (iz + 0.5) * a])
    o = np.array(o) + rng.normal(0.0, 0.3, size=(216, 3))
    placed = [p for p in o]
    pos, sp = [], []
    for k in range(216):
        pos.append(o[k]); sp.append(1)
        for _ in range(2):
            while True:
                v = rng.normal(size=3)
                v /= np.linalg.norm(v)
                hpos = o[k] + 0.96 * v
                d = np.array(placed) - hpos
                d -= L * np.round(d / L)
                dist = np.sqrt((d * d).sum(1))
                # the H's own O sits at exactly 0.96 A; any other atom must be >= 0.9 A away
                dist[k] = 10.0
                if dist.min() >= MIN_SEP:
                    break
            placed.append(hpos)
            pos.append(hpos); sp.append(0)
    pos = np.mod(np.array(pos), L)
    model = ModelSpec(n_species=2, n_layers=1, channels=16, l_max=1, n_heads=1,
                      n_rbf=8, radial_hidden=32)
    return Workload("water648", np.full(3, L, np.float32), pos.astype(np.float32),
                    np.array(sp, np.int32), ["H", "O"], model)


def salt_box(n: int, seed: int, model: ModelSpec, name: str, box_edge: float | None = None) -> Workload:
    rng = np.random.default_rng(seed)
    L = box_edge if box_edge is not None else (n / 0.1) ** (1.0 / 3.0)
    box = np.full(3, L)
    pos = _rsa_fill(rng, n, box)
    sp = _species_by_fraction(rng, n, [0.64, 0.32, 0.02, 0.02])
    return Workload(name, box.astype(np.float32), pos.astype(np.float32), sp,
                    ["H", "O", "Na", "Cl"], model)


def salt4k(seed: int = 1002) -> Workload:
    m = ModelSpec(n_species=4, n_layers=2, channels=32, l_max=2, n_heads=4, n_rbf=8,
                  radial_hidden=32)
    return salt_box(4096, seed, m, "salt4k", box_edge=34.5)


def big_model(n_species: int = 4) -> ModelSpec:
    return ModelSpec(n_species=n_species, n_layers=4, channels=64, l_max=2, n_heads=4,
                     n_rbf=8, radial_hidden=64)


def salt60k(seed: int = 1003) -> Workload:
    return salt_box(60000, seed, big_model(), "salt60k")


def salt500k(seed: int = 1005) -> Workload:
    return salt_box(500000, seed, big_model(), "salt500k", box_edge=171.0)


def capsid39k(seed: int = 1004) -> Workload:
    """Protein-density shell section (60-70 A from a centre 65 A to the -x side of the box
    centre, 0.12 atoms/A^3) in water (0.1 atoms/A^3), 39,300 atoms in a periodic cube."""
    rng = np.random.default_rng(seed)
    n_total = 39300
    probe = np.random.default_rng(seed + 7).uniform(0.0, 1.0, size=(400000, 3))

    def shell_mask(p, L):
        c = np.array([L / 2 - 65.0, L / 2, L / 2])
        r = np.sqrt(((p - c) ** 2).sum(1))
        return (r >= 60.0) & (r <= 70.0)

    def count(L):
        frac = shell_mask(probe * L, L).mean()
        return L ** 3 * (0.12 * frac + 0.1 * (1 - frac))

    lo, hi = 60.0, 80.0
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        if count(mid) < n_total:
            lo = mid
        else:
            hi = mid
    L = 0.5 * (lo + hi)
    frac = shell_mask(probe * L, L).mean()
    n_shell = int(round(0.12 * frac * L ** 3))
    n_water = n_total - n_shell
    box = np.full(3, L)
    shell = _rsa_fill(rng, n_shell, box, accept_region=lambda p: shell_mask(p, L))
    water = _rsa_fill(rng, n_water, box, accept_region=lambda p: ~shell_mask(p, L),
                      existing=shell)
    names = ["C", "N", "O", "S", "H", "Na", "Cl", "Ow"]
    sp_shell = _species_by_fraction(rng, n_shell, [0.31, 0.085, 0.10, 0.005, 0.50, 0, 0, 0])
    sp_water = _species_by_fraction(rng, n_water, [0, 0, 0, 0, 0.96 * 2 / 3, 0.02, 0.02, 0.96 / 3])
    pos = np.concatenate([shell, water], axis=0)
    sp = np.concatenate([sp_shell, sp_water]).astype(np.int32)
    perm = rng.permutation(n_total)
    return Workload("capsid39k", box.astype(np.float32), pos[perm].astype(np.float32), sp[perm],
                    names, big_model(8), extra={"n_shell": n_shell})


WORKLOADS = {"water648": water648, "salt4k": salt4k, "salt60k": salt60k,
             "capsid39k": capsid39k, "salt500k": salt500k}


def weight_count(m: ModelSpec) -> int:
    C, R, P, S, T, Lm, K = (m.channels, m.radial_hidden, m.n_paths, m.n_species,
                            m.n_layers, m.l_max, m.n_rbf)
    per_layer = 2 * C * C + R * K + P * R + C * (1 + Lm) * C + Lm * C * C
    return S * C + T * per_layer + C


def make_weights(m: ModelSpec, seed: int) -> np.ndarray:
    """One fp32 blob, row-major [out][in], in this order: Emb[S][C]; per layer W_q[C][C],
    W_k[C][C], W1[R][K], W2[P][R], W_lin0[C(1+l_max)][C], W_lin^l[C][C] (l=1..l_max);
    w_E[C]. Entries are N(0, 1/fan_in); the embedding table is N(0, 1)."""
    rng = np.random.default_rng(seed)
    C, R, P, S, K = m.channels, m.radial_hidden, m.n_paths, m.n_species, m.n_rbf
    parts = [rng.normal(0.0, 1.0, size=S * C)]
    for _ in range(m.n_layers):
        for (o, i) in [(C, C), (C, C), (R, K), (P, R), (C * (1 + m.l_max), C)] + [(C, C)] * m.l_max:
            parts.append(rng.normal(0.0, 1.0 / math.sqrt(i), size=o * i))
    parts.append(rng.normal(0.0, 1.0 / math.sqrt(C), size=C))
    w = np.concatenate(parts).astype(np.float32)
    assert w.size == weight_count(m)
    return w


def maxwell_velocities(species: np.ndarray, masses: np.ndarray, temperature: float, seed: int) -> np.ndarray:
    """N(0, kT/m) per axis in A/fs, centre-of-mass momentum removed, no rescale."""
    rng = np.random.default_rng(seed)
    m = masses[species]
    sigma = np.sqrt(KB_EV * temperature / m * EV_PER_AMU_A2FS2)
    v = rng.normal(size=(species.shape[0], 3)) * sigma[:, None]
    p = (v * m[:, None]).sum(0)
    v -= p / m.sum()
    return v.astype(np.float32)


def load(name: str, seed_offset: int = 0) -> Workload:
    return WORKLOADS[name]() if seed_offset == 0 else WORKLOADS[name](1000 + seed_offset)


def random_small_box(n: int, L: float, seed: int, n_species: int = 2):
    """Tiny uniform random boxes (no exclusion) for brute-force neighbour checks."""
    rng = np.random.default_rng(seed)
    pos = rng.uniform(-0.5 * L, 1.5 * L, size=(n, 3)).astype(np.float32)
    sp = rng.integers(0, n_species, size=n).astype(np.int32)
    return np.full(3, L, np.float32), pos, sp
