"""Write oracle expected values for the large workloads (salt60k, capsid39k, salt500k).

Only the fp64 oracle (``oracle/``) and the seeded generators are used; nothing here touches
the GPU library. Output per workload: ``tests/golden/<workload>.json`` (metadata: digest of
the inputs, weight seed, total energy, pair count, timing) and ``tests/golden/<workload>.npz``
(fp64 arrays, no pickles).

salt60k and capsid39k run the whole periodic system through the oracle and store every
atom's energy and force, indexed by original (pre-sort) atom id.

salt500k is too large for one oracle run, so the oracle runs on clusters cut around chosen
centres. A per-atom energy depends only on atoms within n_layers * r_cut (23 A) of it, and
the force on an atom only on atoms within twice that, so in a cluster of radius
R = 2 * n_layers * r_cut + DELTA (non-periodic, in a box of 4 R) the energies of every atom
within R - n_layers * r_cut of the centre and the forces of every atom within DELTA of it
equal those of the periodic system. Half of the centres lie within 2 A of one, two or three
periodic faces of the box (so their clusters cross the periodic boundary), half are random.

salt60k_md runs the oracle's velocity-Verlet integrator on the whole salt60k box (start at
50 K, readout weights scaled by 30, MD_STEPS steps inside one rebuild interval) and stores
every atom's final position and velocity and the potential-energy trace.

usage: python tests/golden/make_golden.py [salt60k capsid39k salt500k salt60k_md]
"""
from __future__ import annotations

import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from molecular_dynamics_hilbert_amd import workloads as W  # noqa: E402

WEIGHT_SEED = {"water648": 2001, "salt4k": 2002, "salt60k": 2003, "capsid39k": 2004,
               "salt500k": 2005}
N_CLUSTERS = 64   # salt500k cluster centres (half near periodic faces), all distinct
DELTA = 2.0       # A: force atoms lie within DELTA of a cluster's centre


def digest(wl, w) -> str:
    h = hashlib.sha256()
    for a in (wl.box, wl.pos, wl.species, w):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def full_system(name: str):
    wl = W.load(name)
    w = W.make_weights(wl.model, WEIGHT_SEED[name])
    t0 = time.time()
    nb = oracle.build_neighbors(wl.box, wl.pos, wl.species, wl.model.r_cut, wl.skin)
    out = oracle.energy_forces(wl.model, w, wl.box, nb["pos"].astype(np.float64), nb["species"],
                               nb["row_ptr"], nb["col_shift"])
    t1 = time.time()
    perm = np.asarray(nb["perm"])
    e_by_id = np.empty(wl.n)
    e_by_id[perm] = out["e_atom"]
    f_by_id = np.empty((wl.n, 3))
    f_by_id[perm] = out["forces"]
    meta = dict(workload=name, digest=digest(wl, w), weight_seed=WEIGHT_SEED[name],
                energy=out["energy"], n_edges=int(nb["row_ptr"][-1]),
                net_force=out["forces"].sum(0).tolist(),
                max_abs_force=float(np.abs(out["forces"]).max()),
                oracle_seconds=t1 - t0, method="full periodic system, every atom")
    arrays = dict(e_atom=e_by_id, forces=f_by_id)
    return meta, arrays


def cluster(wl, w, x, center: int, radius: float):
    """Atoms within `radius` (minimum image) of atom `center`, placed in a 4*radius box.
    Returns the selected original ids, their distances from the centre, and the oracle's
    per-atom energies and forces of the cluster (in the order of the ids)."""
    L = wl.box.astype(np.float64)
    d = x - x[center]
    d -= L * np.round(d / L)
    r2 = (d * d).sum(1)
    sel = np.where(r2 < radius * radius)[0]
    Lc = 4.0 * radius
    xc = d[sel] + Lc / 2
    box = np.full(3, Lc, np.float32)
    rp, col = oracle.neighbors(box, xc.astype(np.float32), wl.model.r_cut, wl.skin, method=1)
    out = oracle.energy_forces(wl.model, w, box, xc, wl.species[sel], rp, col)
    return sel, np.sqrt(r2[sel]), out["e_atom"], out["forces"]


def face_centres(x, L, rng, k):
    """k atom ids whose wrapped coordinates lie within 2 A of a face on 1, 2 or 3 axes
    (cycling through faces, edges and corners)."""
    near = (x < 2.0) | (x > L - 2.0)
    cnt = near.sum(1)
    out = []
    for t in range(k):
        want = 1 + t % 3
        pool = np.setdiff1d(np.where(cnt == want)[0], out)
        if pool.size == 0:  # few atoms lie near a corner: take any face atom not yet taken
            pool = np.setdiff1d(np.where(cnt >= 1)[0], out)
        out.append(int(rng.choice(pool)))
    return out


def clustered(name: str):
    wl = W.load(name)
    w = W.make_weights(wl.model, WEIGHT_SEED[name])
    T, rc = wl.model.n_layers, wl.model.r_cut
    radius = 2 * T * rc + DELTA
    r_e = radius - T * rc
    wpos, _ = oracle.wrap_keys(wl.box, wl.pos)
    x = wpos.astype(np.float64)
    L = wl.box.astype(np.float64)
    rng = np.random.default_rng(78)
    centres = face_centres(x, L, rng, N_CLUSTERS // 2)
    rest = np.setdiff1d(np.arange(wl.n), centres)
    centres += [int(c) for c in rng.choice(rest, N_CLUSTERS - len(centres), replace=False)]
    e_ids, e_vals, f_ids, f_vals, sizes = [], [], [], [], []
    seen_e, seen_f = set(), set()
    t0 = time.time()
    for k, c in enumerate(centres):
        sel, dist, ea, fa = cluster(wl, w, x, c, radius)
        sizes.append(int(sel.size))
        for a in np.where(dist < r_e)[0]:
            if int(sel[a]) not in seen_e:
                seen_e.add(int(sel[a])); e_ids.append(int(sel[a])); e_vals.append(float(ea[a]))
        for a in np.where(dist < DELTA)[0]:
            if int(sel[a]) not in seen_f:
                seen_f.add(int(sel[a])); f_ids.append(int(sel[a])); f_vals.append(fa[a])
        print("  cluster %d/%d: %d atoms, %d energies, %d forces so far, %.0f s" % (
            k + 1, len(centres), sel.size, len(e_ids), len(f_ids), time.time() - t0), flush=True)
    meta = dict(workload=name, digest=digest(wl, w), weight_seed=WEIGHT_SEED[name],
                centres=centres, cluster_sizes=sizes, radius=radius, energy_radius=r_e,
                force_radius=DELTA, oracle_seconds=time.time() - t0,
                method="clusters of radius 2*T*r_c+%.1f A around %d centres (%d within 2 A of "
                       "periodic faces): energies within R-T*r_c, forces within %.1f A of each "
                       "centre" % (DELTA, len(centres), N_CLUSTERS // 2, DELTA))
    arrays = dict(e_ids=np.array(e_ids, np.int64), e_atom=np.array(e_vals),
                  f_ids=np.array(f_ids, np.int64), forces=np.array(f_vals).reshape(-1, 3))
    return meta, arrays


MD_STEPS = 4
MD_SCALE = 30.0   # readout weights scale, as in the small MD parity runs
MD_TEMP = 50.0    # K


def md_trajectory(name: str):
    base = name[:-3]
    wl = W.load(base)
    w = W.make_weights(wl.model, WEIGHT_SEED[base])
    w[-wl.model.channels:] *= MD_SCALE
    vseed = 3000 + WEIGHT_SEED[base] % 1000
    vel = W.maxwell_velocities(wl.species, wl.masses(), MD_TEMP, vseed)
    t0 = time.time()
    o = oracle.md_steps(wl.model, w, wl.box, wl.model.r_cut, wl.skin, wl.pos, vel, wl.species,
                        wl.masses(), wl.dt_fs, MD_STEPS, 20)
    assert o["status"] == 0
    pa = np.asarray(o["perm_accum"])
    x = np.empty((wl.n, 3)); x[pa] = o["pos"]
    v = np.empty((wl.n, 3)); v[pa] = o["vel"]
    meta = dict(workload=name, digest=digest(wl, w), weight_seed=WEIGHT_SEED[base],
                readout_scale=MD_SCALE, temperature_K=MD_TEMP, velocity_seed=vseed,
                n_steps=MD_STEPS, rebuild_every=20, epot=[float(e) for e in o["epot"]],
                oracle_seconds=time.time() - t0,
                method="oracle velocity Verlet on the whole periodic box; final positions and "
                       "velocities of every atom by original id")
    return meta, dict(pos=x, vel=v, epot=np.asarray(o["epot"]))


def main(names):
    for name in names:
        t = time.time()
        if name.endswith("_md"):
            meta, arrays = md_trajectory(name)
        else:
            meta, arrays = clustered(name) if name == "salt500k" else full_system(name)
        with open(os.path.join(HERE, name + ".json"), "w") as f:
            json.dump(meta, f)
        np.savez_compressed(os.path.join(HERE, name + ".npz"), **arrays)
        print("%s: %.1f s" % (name, time.time() - t), flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["salt60k", "capsid39k", "salt500k"])
