"""Pins of the oracle's model (harmonics, coupling, energy, forces, MD) against facts that do
not come from the oracle itself: closed forms (dimer), an independent quadrature (scipy's
Lebedev rule), symmetry (rotation, translation, permutation invariance), finite
differences, and the time reversibility of velocity Verlet."""
import math

import numpy as np
import pytest
from scipy.integrate import lebedev_rule
from scipy.spatial.transform import Rotation

from molecular_dynamics_hilbert_amd import workloads as W

RC, SKIN = 5.75, 1.0


def _rand_unit(rng, n):
    v = rng.normal(size=(n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


# ---- spherical harmonics and coupling ------------------------------------------------

def test_sph_component_normalisation(oracle_mod):
    rng = np.random.default_rng(0)
    for nv in _rand_unit(rng, 200):
        Y = oracle_mod.sph(2, nv)
        assert Y[0] == 1.0
        assert abs((Y[1:4] ** 2).sum() - 3) < 1e-12
        assert abs((Y[4:9] ** 2).sum() - 5) < 1e-12


def test_sph_orthonormal_lebedev(oracle_mod):
    x, w = lebedev_rule(17)
    Ys = np.array([oracle_mod.sph(2, x[:, k]) for k in range(x.shape[1])])
    G = (Ys * (w / w.sum())[:, None]).T @ Ys  # (1/4pi) int Y_a Y_b
    assert np.abs(G - np.eye(9)).max() < 1e-12


def test_sph_rotation_equivariance(oracle_mod):
    """Y^l(R n) = D^l(R) Y^l(n) with an orthogonal D^l: fit D on random points, check on
    fresh points; a wrong sign or term in any component breaks it."""
    rng = np.random.default_rng(1)
    R = Rotation.random(random_state=7).as_matrix()
    pts = _rand_unit(rng, 60)
    Y = np.array([oracle_mod.sph(2, p) for p in pts])
    YR = np.array([oracle_mod.sph(2, R @ p) for p in pts])
    for lo, hi in [(1, 4), (4, 9)]:
        Dl, *_ = np.linalg.lstsq(Y[:, lo:hi], YR[:, lo:hi], rcond=None)
        Dl = Dl.T
        assert np.abs(Dl @ Dl.T - np.eye(hi - lo)).max() < 1e-10
        test = _rand_unit(rng, 20)
        for p in test:
            assert np.abs(oracle_mod.sph(2, R @ p)[lo:hi] - Dl @ oracle_mod.sph(2, p)[lo:hi]).max() < 1e-10


def test_paths_list(oracle_mod):
    assert oracle_mod.paths(1) == [(0, 0, 0), (0, 1, 1), (1, 0, 1), (1, 1, 0)]
    assert oracle_mod.paths(2) == [(0, 0, 0), (0, 1, 1), (0, 2, 2), (1, 0, 1), (1, 1, 0),
                                   (1, 1, 2), (1, 2, 1), (2, 0, 2), (2, 1, 1), (2, 2, 0),
                                   (2, 2, 2)]


def test_coupling_vs_lebedev_and_closed_forms(oracle_mod):
    cg = oracle_mod.coupling(2)
    x, w = lebedev_rule(17)
    wn = w / w.sum()
    Ys = np.array([oracle_mod.sph(2, x[:, k]) for k in range(x.shape[1])])
    for p, (l1, l2, l3) in enumerate(oracle_mod.paths(2)):
        G = np.einsum("q,qa,qb,qc->abc", wn, Ys[:, l1 * l1:(l1 + 1) ** 2],
                      Ys[:, l2 * l2:(l2 + 1) ** 2], Ys[:, l3 * l3:(l3 + 1) ** 2])
        Cref = G * math.sqrt(2 * l3 + 1) / np.linalg.norm(G)
        Cp = cg[p, :2 * l1 + 1, :2 * l2 + 1, :2 * l3 + 1]
        assert np.abs(Cp - Cref).max() < 1e-12, (l1, l2, l3)
        # padding beyond 2l+1 stays zero
        assert np.abs(cg[p]).sum() - np.abs(Cp).sum() < 1e-15
        if l1 == 0:
            assert np.abs(Cp[0] - np.eye(2 * l2 + 1)).max() < 1e-12  # identity
        if l2 == 0:
            assert np.abs(Cp[:, 0, :] - np.eye(2 * l1 + 1)).max() < 1e-12
        if (l1, l2, l3) == (1, 1, 0):
            assert np.abs(Cp[:, :, 0] - np.eye(3) / math.sqrt(3)).max() < 1e-12


# ---- energy ---------------------------------------------------------------------------

def _silu(z):
    return z / (1 + np.exp(-z))


def _dimer_energy(m, w, r, z0, z1):
    """Closed form for two atoms with one edge each, H = 1 and W_q = 0 (so the softmax weight
    of the only edge is 1): only paths leaving from l1 = 0 (first layer) and the l=1 -> 0
    contraction (second layer) reach the energy. Written from the layer definition
    independently of the oracle's general code."""
    C, R, K, P = m.channels, m.radial_hidden, m.n_rbf, m.n_paths
    off = 0
    emb = w[off:off + m.n_species * C].reshape(m.n_species, C); off += m.n_species * C
    layers = []
    for _ in range(m.n_layers):
        d = {}
        for nm, (o, i) in [("Wq", (C, C)), ("Wk", (C, C)), ("W1", (R, K)), ("W2", (P, R)),
                           ("W0", (C * (1 + m.l_max), C))] + [("Wl%d" % l, (C, C)) for l in range(1, m.l_max + 1)]:
            d[nm] = w[off:off + o * i].reshape(o, i).astype(np.float64); off += o * i
        layers.append(d)
    wE = w[off:off + C].astype(np.float64)
    rc = m.r_cut
    u = 0.5 * (np.cos(np.pi * r / rc) + 1) if r < rc else 0.0
    b = np.array([u * math.sqrt(2 / rc) * math.sin(k * math.pi * r / rc) / r for k in range(1, K + 1)])
    nvec = {0: np.array([0, 0, 1.0]), 1: np.array([0, 0, -1.0])}  # n for dest 0 / dest 1
    z = [z0, z1]
    h0 = {a: emb[z[a]].astype(np.float64) for a in (0, 1)}
    h1 = {a: np.zeros((C, 3)) for a in (0, 1)}
    for t, d in enumerate(layers):
        wr = d["W2"] @ _silu(d["W1"] @ b)  # paths (0,0,0),(0,1,1),(1,0,1),(1,1,0)
        alpha = 1.0 if u > 0 else 0.0
        new0, new1 = {}, {}
        for a in (0, 1):
            j = 1 - a
            n = nvec[a]
            m0 = alpha * (wr[0] * h0[j] + wr[3] * (h1[j] @ n))
            m1 = alpha * (wr[1] * np.outer(h0[j], math.sqrt(3) * n) + wr[2] * h1[j])
            y0 = d["W0"][:C] @ m0
            g = d["W0"][C:2 * C] @ m0
            new0[a] = h0[a] + _silu(y0)
            new1[a] = h1[a] + (1 / (1 + np.exp(-g)))[:, None] * (d["Wl1"] @ m1)
        h0, h1 = new0, new1
    return float(wE @ h0[0] + wE @ h0[1])


def _dimer_case(oracle_mod, m, w, r):
    L = 50.0
    box = np.full(3, L, np.float32)
    pos = np.array([[20.0, 20.0, 20.0], [20.0, 20.0, 20.0 + r]], np.float32)
    sp = np.array([0, 1], np.int32)
    nb = oracle_mod.build_neighbors(box, pos, sp, RC, SKIN)
    out = oracle_mod.energy_forces(m, w, box, nb["pos"].astype(np.float64), nb["species"],
                                   nb["row_ptr"], nb["col_shift"])
    rr = float(np.float64(nb["pos"][1, 2]) - np.float64(nb["pos"][0, 2]))
    return out, abs(rr), nb


@pytest.mark.parametrize("T", [1, 2])
def test_dimer_closed_form(oracle_mod, T):
    m = W.ModelSpec(n_species=2, n_layers=T, channels=8, l_max=1, n_heads=1, n_rbf=8,
                    radial_hidden=16)
    w = W.make_weights(m, 99 + T)
    C = m.channels
    per = 2 * C * C + m.radial_hidden * m.n_rbf + m.n_paths * m.radial_hidden + 2 * C * C + C * C
    for t in range(T):
        base = m.n_species * C + t * per
        w[base:base + C * C] = 0.0  # W_q = 0
    for r in (1.3, 2.9, 4.4, 5.6):
        out, rr, nb = _dimer_case(oracle_mod, m, w, r)
        z0, z1 = (0, 1) if nb["species"][0] == 0 else (1, 0)
        ref = _dimer_energy(m, w, rr, z0, z1)
        assert abs(out["energy"] - ref) < 1e-11 * max(1, abs(ref)), (r, out["energy"], ref)


def test_dimer_continuity_across_cutoff(oracle_mod):
    """E is C1 as the pair crosses r_c: values and slopes meet (envelope in the weights)."""
    m = W.ModelSpec(n_species=2, n_layers=2, channels=8, l_max=1, n_heads=1, radial_hidden=16)
    w = W.make_weights(m, 5)
    rc = float(np.float32(RC))
    es = {}
    for d in (-2e-3, -1e-3, 1e-3, 2e-3):
        es[d] = _dimer_case(oracle_mod, m, w, rc + d)[0]["energy"]
    far = _dimer_case(oracle_mod, m, w, rc + 0.5)[0]["energy"]
    assert abs(es[1e-3] - far) < 1e-12 and abs(es[2e-3] - far) < 1e-12
    assert abs(es[-1e-3] - far) < 1e-6   # value continuous
    slope_in = (es[-1e-3] - es[-2e-3]) / 1e-3
    assert abs(slope_in) < 1e-3          # slope -> 0 at r_c (C1)


def _system(oracle_mod, wl, seed=2001, pos=None, box=None):
    box = wl.box if box is None else box
    pos = wl.pos if pos is None else pos
    nb = oracle_mod.build_neighbors(box, pos, wl.species, RC, SKIN)
    w = W.make_weights(wl.model, seed)
    out = oracle_mod.energy_forces(wl.model, w, box, nb["pos"].astype(np.float64), nb["species"],
                                   nb["row_ptr"], nb["col_shift"])
    return nb, w, out


@pytest.mark.parametrize("wname", ["water648", "salt4k"])
def test_forces_finite_difference(oracle_mod, wname):
    wl = W.load(wname)
    nb, w, out = _system(oracle_mod, wl)
    pos = nb["pos"].astype(np.float64)
    F = out["forces"]
    assert np.abs(F.sum(0)).max() < 1e-10  # translation invariance: net force 0
    h = 1e-4
    rng = np.random.default_rng(4)
    for k in rng.choice(wl.n, 4, replace=False):
        for a in range(3):
            ps = []
            for sgn in (1, -1):
                p = pos.copy(); p[k, a] += sgn * h
                ps.append(oracle_mod.energy_forces(wl.model, w, wl.box, p, nb["species"],
                                                   nb["row_ptr"], nb["col_shift"],
                                                   want_forces=False)["energy"])
            fd = -(ps[0] - ps[1]) / (2 * h)
            assert abs(fd - F[k, a]) <= 1e-6, (k, a, fd, F[k, a])


def test_energy_translation_and_permutation_invariance(oracle_mod):
    wl = W.load("water648")
    nb, w, out = _system(oracle_mod, wl)
    # the model: translating every fp64 position (same pair list) leaves E and F unchanged
    t = np.array([3.3, -7.1, 11.9])
    outt = oracle_mod.energy_forces(wl.model, w, wl.box, nb["pos"].astype(np.float64) + t,
                                    nb["species"], nb["row_ptr"], nb["col_shift"])
    assert abs(outt["energy"] - out["energy"]) < 1e-12 * abs(out["energy"])
    assert np.abs(outt["forces"] - out["forces"]).max() < 1e-12
    # the full rebuild: translated fp32 input (rounded to fp32, so only to that precision)
    shift = np.array([3.3, -7.1, 11.9], np.float32)
    nb2, _, out2 = _system(oracle_mod, wl, pos=wl.pos + shift)
    assert abs(out2["energy"] - out["energy"]) < 1e-8 * abs(out["energy"])
    # per-atom energies follow the atoms
    ea1 = np.empty(wl.n); ea1[nb["perm"]] = out["e_atom"]
    ea2 = np.empty(wl.n); ea2[nb2["perm"]] = out2["e_atom"]
    assert np.abs(ea1 - ea2).max() < 1e-6
    # relabelling the atoms (same positions, different input order) changes nothing
    rng = np.random.default_rng(8)
    p = rng.permutation(wl.n)
    wl_p = W.Workload(wl.name, wl.box, wl.pos[p], wl.species[p], wl.species_names, wl.model)
    nb3, _, out3 = _system(oracle_mod, wl_p)
    assert abs(out3["energy"] - out["energy"]) < 1e-10 * abs(out["energy"])


def _isolated_cluster(wl, L=50.0):
    pos = wl.pos.astype(np.float64)
    pos = pos - pos.mean(0) + L / 2
    return np.full(3, L, np.float32), pos


def test_rotation_invariance_isolated_cluster(oracle_mod):
    """Random SO(3) rotations of an isolated cluster (no periodic image within the cutoff, so
    every shift is zero and the pair list is rotation invariant): E is invariant and F
    rotates with the cluster, in fp64 with the same pair list."""
    wl = W.load("water648")
    box, pos = _isolated_cluster(wl)
    nb, w, out = _system(oracle_mod, wl, pos=pos.astype(np.float32), box=box)
    assert np.all((nb["col_shift"] >> 27) == 13)
    x = nb["pos"].astype(np.float64)
    c = x.mean(0)
    for s in range(3):
        R = Rotation.random(random_state=100 + s).as_matrix()
        xr = (x - c) @ R.T + c
        outr = oracle_mod.energy_forces(wl.model, w, box, xr, nb["species"], nb["row_ptr"],
                                        nb["col_shift"])
        assert abs(outr["energy"] - out["energy"]) < 1e-12 * abs(out["energy"])
        assert np.abs(outr["forces"] - out["forces"] @ R.T).max() < 1e-12
        # and through a full rebuild from the rotated fp32 coordinates
        pr = ((pos - 25.0) @ R.T + 25.0).astype(np.float32)
        nbr, _, outf = _system(oracle_mod, wl, pos=pr, box=box)
        assert abs(outf["energy"] - out["energy"]) < 1e-8 * abs(out["energy"])


def test_cube_rotations_periodic(oracle_mod):
    wl = W.load("water648")
    nb, w, out = _system(oracle_mod, wl)
    F = np.empty((wl.n, 3)); F[nb["perm"]] = out["forces"]
    L = float(wl.box[0])
    import itertools
    mats = []
    for perm in itertools.permutations(range(3)):
        for signs in itertools.product((1, -1), repeat=3):
            Rm = np.zeros((3, 3))
            for a in range(3):
                Rm[a, perm[a]] = signs[a]
            if np.linalg.det(Rm) > 0:
                mats.append(Rm)
    assert len(mats) == 24
    for Rm in mats[1:6]:
        pr = (wl.pos.astype(np.float64) @ Rm.T) % L
        nbr, _, outr = _system(oracle_mod, wl, pos=pr.astype(np.float32))
        assert abs(outr["energy"] - out["energy"]) < 1e-6 * abs(out["energy"])
        Fr = np.empty((wl.n, 3)); Fr[nbr["perm"]] = outr["forces"]
        assert np.abs(Fr - F @ Rm.T).max() < 1e-6


def _sub_cluster(wl, radius, L=50.0):
    """Atoms of `wl` within `radius` (minimum image) of its box centre, moved into an
    L-edge box (no periodic image inside the cutoff: every shift code is 13)."""
    x = wl.pos.astype(np.float64)
    Lw = wl.box.astype(np.float64)
    d = x - Lw / 2
    d -= Lw * np.round(d / Lw)
    sel = np.where((d * d).sum(1) < radius * radius)[0]
    pos = d[sel] + L / 2
    sub = W.Workload(wl.name + "_cluster", np.full(3, L, np.float32), pos.astype(np.float32),
                     wl.species[sel], wl.species_names, wl.model)
    return sub


@pytest.mark.parametrize("case", [("salt4k", 9.0, 2002), ("salt60k", 7.5, 2003)])
def test_rotation_invariance_lmax2_cluster(oracle_mod, case):
    """l_max = 2 models (salt4k's two layers; the four-layer 64-channel model of the large
    workloads): every l = 2 path, the gated l = 2 update and their adjoints enter E and F.
    Under random SO(3) rotations of an isolated cluster (same pair list) E is invariant and
    F rotates with it, in fp64. A mistake that mixes m-components of a degree in any way
    other than a rotation does (a cyclic m-shift, a sign, a transposed block) breaks this."""
    name, radius, seed = case
    wl = _sub_cluster(W.load(name), radius)
    assert wl.model.l_max == 2 and wl.model.n_layers >= 2
    nb, w, out = _system(oracle_mod, wl, seed=seed)
    assert np.all((nb["col_shift"] >> 27) == 13)
    x = nb["pos"].astype(np.float64)
    c = x.mean(0)
    E0, F0 = out["energy"], out["forces"]
    assert np.abs(F0).max() > 1e-3  # forces are not trivially zero
    for s in range(3):
        R = Rotation.random(random_state=200 + s).as_matrix()
        xr = (x - c) @ R.T + c
        outr = oracle_mod.energy_forces(wl.model, w, wl.box, xr, nb["species"], nb["row_ptr"],
                                        nb["col_shift"])
        assert abs(outr["energy"] - E0) < 1e-12 * abs(E0), (outr["energy"], E0)
        assert np.abs(outr["forces"] - F0 @ R.T).max() < 1e-12 * max(1.0, np.abs(F0).max())


def test_cube_rotations_periodic_lmax2(oracle_mod):
    """The 24 proper rotations of a cube map the periodic salt4k box (l_max = 2, two layers)
    onto itself; through a full rebuild from the rotated fp32 coordinates E is unchanged
    and every atom's force rotates (up to the fp32 rounding of the rotated input)."""
    import itertools
    wl = W.load("salt4k")
    nb, w, out = _system(oracle_mod, wl, seed=2002)
    F = np.empty((wl.n, 3)); F[nb["perm"]] = out["forces"]
    L = float(wl.box[0])
    mats = []
    for perm in itertools.permutations(range(3)):
        for signs in itertools.product((1, -1), repeat=3):
            Rm = np.zeros((3, 3))
            for a in range(3):
                Rm[a, perm[a]] = signs[a]
            if np.linalg.det(Rm) > 0:
                mats.append(Rm)
    for Rm in (mats[3], mats[8], mats[17]):
        pr = (wl.pos.astype(np.float64) @ Rm.T) % L
        nbr, _, outr = _system(oracle_mod, wl, seed=2002, pos=pr.astype(np.float32))
        assert abs(outr["energy"] - out["energy"]) < 1e-6 * abs(out["energy"])
        Fr = np.empty((wl.n, 3)); Fr[nbr["perm"]] = outr["forces"]
        assert np.abs(Fr - F @ Rm.T).max() < 1e-6 * max(1.0, np.abs(F).max())


def test_skin_invariance_exact(oracle_mod):
    """Edges with r_c <= r < r_c+skin contribute exactly zero: E and F from the skin-0 list
    equal those from the skin-1 list bit for bit."""
    wl = W.load("salt4k")
    nb, w, out = _system(oracle_mod, wl)
    rp0, c0 = oracle_mod.neighbors(wl.box, nb["pos"], RC, 0.0)
    out0 = oracle_mod.energy_forces(wl.model, w, wl.box, nb["pos"].astype(np.float64),
                                    nb["species"], rp0, c0)
    assert out0["energy"] == out["energy"]
    assert np.array_equal(out0["forces"], out["forces"])


def test_species_error(oracle_mod):
    wl = W.load("water648")
    nb, w, _ = _system(oracle_mod, wl)
    sp = nb["species"].copy(); sp[3] = 7
    rc = oracle_mod.energy_forces_status(wl.model, w, wl.box, nb["pos"].astype(np.float64), sp,
                                         nb["row_ptr"], nb["col_shift"])
    assert rc == oracle_mod.ERR_SPECIES


# ---- MD -------------------------------------------------------------------------------

def _md_setup(oracle_mod, scale=30.0):
    wl = W.load("water648")
    w = W.make_weights(wl.model, 2001)
    w[-wl.model.channels:] *= scale  # stiffer readout so the dynamics is not trivial
    v = W.maxwell_velocities(wl.species, wl.masses(), 300.0, 3001).astype(np.float64)
    return wl, w, v


def test_md_time_reversible(oracle_mod):
    wl, w, v = _md_setup(oracle_mod)
    a = oracle_mod.md_steps(wl.model, w, wl.box, RC, SKIN, wl.pos, v, wl.species, wl.masses(),
                            0.5, 10, 20)
    assert a["status"] == 0
    b = oracle_mod.md_steps(wl.model, w, wl.box, RC, SKIN, a["pos"], -a["vel"], a["species"],
                            wl.masses(), 0.5, 10, 20, perm_accum=a["perm_accum"], forces=a["forces"])
    assert b["status"] == 0
    L = float(wl.box[0])
    x0 = np.empty((wl.n, 3)); x0[b["perm_accum"]] = b["pos"]
    d = x0 - wl.pos.astype(np.float64)
    d -= L * np.round(d / L)
    # the second call's rebuild rounds positions to their stored fp32 values (ulp 1.9e-6 A
    # at 18.6 A); beyond that rounding the trajectory retraces itself. A first-order
    # mistake in the kicks would leave errors of order dt^2 a n ~ 1e-2 A.
    assert np.abs(d).max() < 5e-6
    v0 = np.empty((wl.n, 3)); v0[b["perm_accum"]] = -b["vel"]
    assert np.abs(v0 - v).max() < 5e-6


def test_md_energy_error_scales_dt2(oracle_mod):
    """Velocity Verlet is second order: the total-energy error over a fixed time span drops
    by ~4x when dt halves."""
    wl, w, v = _md_setup(oracle_mod, scale=300.0)
    conv = 9.648533e-3
    ms = wl.masses()

    def ke(vv, sp):
        return 0.5 * (ms[sp][:, None] * vv ** 2).sum() / conv

    nb0 = oracle_mod.build_neighbors(wl.box, wl.pos, wl.species, RC, SKIN)
    p0 = oracle_mod.energy_forces(wl.model, w, wl.box, nb0["pos"].astype(np.float64),
                                  nb0["species"], nb0["row_ptr"], nb0["col_shift"],
                                  want_forces=False)["energy"]
    etot0 = p0 + ke(v, wl.species)
    errs = []
    for dt, steps in ((0.5, 10), (0.25, 20)):
        r = oracle_mod.md_steps(wl.model, w, wl.box, RC, SKIN, wl.pos, v, wl.species, ms, dt,
                                steps, 1000)
        assert r["status"] == 0
        errs.append(abs(r["epot"][-1] + ke(r["vel"], r["species"]) - etot0))
    ratio = errs[0] / errs[1]
    assert 3.0 < ratio < 5.3, (errs, ratio)


def test_md_skin_flag(oracle_mod):
    wl, w, v = _md_setup(oracle_mod)
    r = oracle_mod.md_steps(wl.model, w, wl.box, RC, 0.01, wl.pos, v * 20, wl.species,
                            wl.masses(), 0.5, 20, 20)
    assert r["status"] == oracle_mod.ERR_SKIN


# ---- NVT (Berendsen weak coupling) and monitors -------------------------------------------
# Constants from their SI definitions (CODATA 2018), independent of the oracle's values.
KB_EV = 1.380649e-23 / 1.602176634e-19               # eV/K
AMU_A2FS2_EV = 1.66053906660e-27 * 1e10 / 1.602176634e-19  # 1 amu A^2/fs^2 in eV


def _ke_ev(vel, species, masses):
    m = masses[species]
    return 0.5 * float((m[:, None] * np.asarray(vel, np.float64) ** 2).sum()) * AMU_A2FS2_EV


def test_ke_trace_is_kinetic_energy(oracle_mod):
    wl, w, v = _md_setup(oracle_mod)
    a = oracle_mod.md_steps(wl.model, w, wl.box, RC, SKIN, wl.pos, v, wl.species, wl.masses(),
                            0.5, 6, 20)
    assert a["status"] == 0
    ke = _ke_ev(a["vel"], a["species"], wl.masses())
    assert abs(a["ke"][-1] - ke) <= 1e-7 * ke  # the oracle's 9.648533e-3 is rounded to 7 digits
    # NVE: kinetic + potential energy is conserved to the integrator's error
    etot = a["ke"] + a["epot"]
    assert np.abs(etot - etot[0]).max() < 1e-3 * np.abs(a["ke"]).max()


def test_berendsen_tau_equal_dt_reaches_target(oracle_mod):
    """With tau = dt the scale factor is sqrt(T0/T): right after the thermostat the kinetic
    energy is exactly (3N/2) k_B T0 at every step, whatever the forces did."""
    wl, w, v = _md_setup(oracle_mod)
    for T0 in (150.0, 450.0):
        a = oracle_mod.md_steps(wl.model, w, wl.box, RC, SKIN, wl.pos, v, wl.species,
                                wl.masses(), 0.5, 5, 20, thermostat=1, t_target_K=T0, tau_fs=0.5)
        assert a["status"] == 0
        target = 1.5 * wl.n * KB_EV * T0
        assert np.abs(a["ke"] / target - 1.0).max() < 1e-7
        assert abs(_ke_ev(a["vel"], a["species"], wl.masses()) / target - 1.0) < 1e-7


def test_berendsen_ideal_gas_relaxes_geometrically(oracle_mod):
    """Zero weights give zero forces (an ideal gas). Each step then sets
    T <- T + (dt/tau)(T0 - T), so T_s - T0 = (1 - dt/tau)^(s+1) (T_init - T0)."""
    wl = W.load("water648")
    w = np.zeros(W.weight_count(wl.model), np.float32)
    v = W.maxwell_velocities(wl.species, wl.masses(), 40.0, 3002).astype(np.float64)
    T_init = 2.0 * _ke_ev(v, wl.species, wl.masses()) / (3 * wl.n * KB_EV)
    T0, dt, tau, n = 25.0, 0.5, 4.0, 12
    a = oracle_mod.md_steps(wl.model, w, wl.box, RC, SKIN, wl.pos, v, wl.species, wl.masses(),
                            dt, n, 20, thermostat=1, t_target_K=T0, tau_fs=tau)
    assert a["status"] == 0
    assert np.all(a["epot"] == 0.0)
    T = 2.0 * a["ke"] / (3 * wl.n * KB_EV)
    expect = T0 + (1.0 - dt / tau) ** np.arange(1, n + 1) * (T_init - T0)
    assert np.abs(T / expect - 1.0).max() < 1e-7


def test_berendsen_arguments(oracle_mod):
    wl, w, v = _md_setup(oracle_mod)
    for kw in (dict(thermostat=1, t_target_K=300.0, tau_fs=0.25),  # tau < dt
               dict(thermostat=1, t_target_K=-1.0, tau_fs=10.0),
               dict(thermostat=2, t_target_K=300.0, tau_fs=10.0)):
        a = oracle_mod.md_steps(wl.model, w, wl.box, RC, SKIN, wl.pos, v, wl.species,
                                wl.masses(), 0.5, 2, 20, **kw)
        assert a["status"] == oracle_mod.ERR_ARG


def test_rmin_trace_brute_force(oracle_mod):
    """Shortest pair distance: every pair of the returned positions, minimum image."""
    wl, w, v = _md_setup(oracle_mod)
    a = oracle_mod.md_steps(wl.model, w, wl.box, RC, SKIN, wl.pos, v, wl.species, wl.masses(),
                            0.5, 4, 20)
    assert a["status"] == 0
    x = a["pos"]
    L = wl.box.astype(np.float64)
    d = x[:, None, :] - x[None, :, :]
    d -= L * np.round(d / L)
    r = np.sqrt((d ** 2).sum(-1))
    r[np.arange(wl.n), np.arange(wl.n)] = np.inf
    assert r.min() < RC
    assert abs(a["rmin"][-1] - r.min()) < 1e-12
