"""Write oracle expected values for the large workloads (salt60k, capsid39k, salt500k).

Only the fp64 oracle (``oracle/``) and the seeded generators are used; nothing here touches
the GPU library. Output: ``tests/golden/<workload>.json`` with the total energy, sampled
per-atom energies and forces keyed by original (pre-sort) atom index, and a digest of the
inputs so a test can detect generator drift.

salt60k and capsid39k run the whole periodic system through the oracle. For salt500k the
oracle runs on clusters cut around sampled atoms: a per-atom energy depends only on atoms
within n_layers * r_cut (23 A), and the force on an atom only on atoms within twice that, so
a cluster of radius 25 A (energies) or 48 A (forces) in a large non-periodic box reproduces
those values exactly.

usage: python tests/golden/make_golden.py [salt60k capsid39k salt500k]
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


def digest(wl, w) -> str:
    h = hashlib.sha256()
    for a in (wl.box, wl.pos, wl.species, w):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def full_system(name: str, n_samples: int = 1024) -> dict:
    wl = W.load(name)
    w = W.make_weights(wl.model, WEIGHT_SEED[name])
    t0 = time.time()
    nb = oracle.build_neighbors(wl.box, wl.pos, wl.species, wl.model.r_cut, wl.skin)
    out = oracle.energy_forces(wl.model, w, wl.box, nb["pos"].astype(np.float64), nb["species"],
                               nb["row_ptr"], nb["col_shift"])
    t1 = time.time()
    rng = np.random.default_rng(77)
    slots = np.sort(rng.choice(wl.n, min(n_samples, wl.n), replace=False))
    orig = nb["perm"][slots]
    return dict(workload=name, digest=digest(wl, w), weight_seed=WEIGHT_SEED[name],
                energy=out["energy"], n_edges=int(nb["row_ptr"][-1]),
                sample_ids=orig.tolist(), e_atom=out["e_atom"][slots].tolist(),
                forces=out["forces"][slots].tolist(), net_force=out["forces"].sum(0).tolist(),
                max_abs_force=float(np.abs(out["forces"]).max()),
                oracle_seconds=t1 - t0, method="full periodic system")


def cluster(wl, w, center: int, radius: float):
    """Atoms within `radius` (minimum image) of atom `center`, placed in a 4*radius box."""
    L = wl.box.astype(np.float64)
    wpos, _ = oracle.wrap_keys(wl.box, wl.pos)
    x = wpos.astype(np.float64)
    d = x - x[center]
    d -= L * np.round(d / L)
    sel = np.where((d * d).sum(1) < radius * radius)[0]
    Lc = 4.0 * radius
    xc = d[sel] + Lc / 2
    box = np.full(3, Lc, np.float32)
    rp, col = oracle.neighbors(box, xc.astype(np.float32), wl.model.r_cut, wl.skin, method=1)
    out = oracle.energy_forces(wl.model, w, box, xc, wl.species[sel], rp, col)
    k = int(np.where(sel == center)[0][0])
    return out["e_atom"][k], out["forces"][k], sel.size


def clustered(name: str, n_e: int = 8, n_f: int = 2) -> dict:
    wl = W.load(name)
    w = W.make_weights(wl.model, WEIGHT_SEED[name])
    rng = np.random.default_rng(78)
    ids = rng.choice(wl.n, n_e + n_f, replace=False)
    T, rc = wl.model.n_layers, wl.model.r_cut
    e_ids, e_vals, f_ids, f_vals, sizes = [], [], [], [], []
    t0 = time.time()
    for k in ids[:n_e]:
        e, _, m = cluster(wl, w, int(k), T * rc + 2.0)
        e_ids.append(int(k)); e_vals.append(float(e)); sizes.append(m)
    for k in ids[n_e:]:
        e, f, m = cluster(wl, w, int(k), 2 * T * rc + 2.0)
        f_ids.append(int(k)); f_vals.append(np.asarray(f).tolist()); sizes.append(m)
        e_ids.append(int(k)); e_vals.append(float(e))
    return dict(workload=name, digest=digest(wl, w), weight_seed=WEIGHT_SEED[name],
                e_ids=e_ids, e_atom=e_vals, f_ids=f_ids, forces=f_vals, cluster_sizes=sizes,
                oracle_seconds=time.time() - t0,
                method="clusters of radius T*r_c+2 (energies) and 2*T*r_c+2 (forces)")


def main(names):
    for name in names:
        t = time.time()
        res = clustered(name) if name == "salt500k" else full_system(name)
        with open(os.path.join(HERE, name + ".json"), "w") as f:
            json.dump(res, f)
        print("%s: %.1f s" % (name, time.time() - t), flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["salt60k", "capsid39k", "salt500k"])
