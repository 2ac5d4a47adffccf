"""ctypes wrapper of the fp64 CPU oracle (``libtess_oracle.so``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``. The GPU library never loads it. Every function here
marshals numpy arrays into the C oracle and returns numpy arrays; no arithmetic of the
method lives in this file.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tess_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libtess_oracle.so")

OK, ERR_ARG, ERR_BOX, ERR_CAPACITY, ERR_SKIN, ERR_SPECIES = 0, -1, -2, -3, -6, -7


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (fp64, OpenMP, no FP contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(
            os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "tess_oracle.h"))):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wno-unused-function",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Model(C.Structure):
    _fields_ = [("n_species", C.c_int32), ("n_layers", C.c_int32), ("channels", C.c_int32),
                ("l_max", C.c_int32), ("n_heads", C.c_int32), ("n_rbf", C.c_int32),
                ("radial_hidden", C.c_int32), ("r_cut", C.c_float)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = C.CDLL(build())
        L = _lib
        p = C.c_void_p
        L.tor_num_threads.restype = C.c_int32
        L.tor_wrap1.restype = C.c_float
        L.tor_wrap1.argtypes = [C.c_float, C.c_double]
        L.tor_hilbert_key3.restype = C.c_uint32
        L.tor_hilbert_key3.argtypes = [C.c_uint32, C.c_uint32, C.c_uint32, C.c_int32]
        L.tor_wrap_keys.argtypes = [C.c_int32, p, p, p, p]
        L.tor_stable_argsort_u32.argtypes = [C.c_int32, p, p]
        L.tor_neighbors.restype = C.c_int32
        L.tor_neighbors.argtypes = [C.c_int32, p, p, C.c_float, C.c_float, C.c_int32, C.c_int64,
                                    p, p, p]
        L.tor_flagged_pairs.restype = C.c_int64
        L.tor_flagged_pairs.argtypes = [C.c_int32, p, p, C.c_float, C.c_float, C.c_double,
                                        C.c_int64, p, p]
        L.tor_build_neighbors.restype = C.c_int32
        L.tor_build_neighbors.argtypes = [C.c_int32, p, C.c_float, C.c_float, p, p, p, p, p,
                                          C.c_int64, p, p, p]
        L.tor_n_paths.restype = C.c_int32
        L.tor_sph.argtypes = [C.c_int32, p, p]
        L.tor_paths.argtypes = [C.c_int32, p, p, p]
        L.tor_coupling.argtypes = [C.c_int32, p]
        L.tor_weights_count.restype = C.c_int64
        L.tor_weights_count.argtypes = [p]
        L.tor_energy_forces.restype = C.c_int32
        L.tor_energy_forces.argtypes = [p, p, C.c_int32, p, p, p, p, p, p, p, p, p]
        L.tor_md_steps.restype = C.c_int32
        L.tor_md_steps.argtypes = [p, p, C.c_int32, p, C.c_float, C.c_float, p, p, p, p,
                                   C.c_double, C.c_int32, C.c_int32, p, p, C.c_int32, p, C.c_int64,
                                   C.c_int32, C.c_double, C.c_double, p, p]
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _box(box):
    return _f32(np.asarray(box).reshape(3))


def model_struct(spec) -> _Model:
    t = spec.as_tuple() if hasattr(spec, "as_tuple") else tuple(spec)
    return _Model(*[int(v) for v in t[:7]], float(t[7]))


# ---- neighbour list -------------------------------------------------------------------

def wrap1(x: float, L: float) -> np.float32:
    return np.float32(lib().tor_wrap1(float(x), float(L)))


def hilbert_key3(x: int, y: int, z: int, bits: int = 10) -> int:
    return int(lib().tor_hilbert_key3(x, y, z, bits))


def wrap_keys(box, pos):
    pos = _f32(pos).reshape(-1, 3)
    n = pos.shape[0]
    out = np.empty_like(pos)
    keys = np.empty(n, np.uint32)
    lib().tor_wrap_keys(n, _ptr(_box(box)), _ptr(pos), _ptr(out), _ptr(keys))
    return out, keys


def stable_argsort(keys):
    keys = np.ascontiguousarray(keys, dtype=np.uint32)
    perm = np.empty(keys.shape[0], np.int32)
    lib().tor_stable_argsort_u32(keys.shape[0], _ptr(keys), _ptr(perm))
    return perm


def neighbors(box, pos, r_cut, skin, method=1, cap=None):
    """CSR (row_ptr, col_shift) of the candidate list for wrapped, sorted fp32 positions."""
    pos = _f32(pos).reshape(-1, 3)
    n = pos.shape[0]
    row_ptr = np.zeros(n + 1, np.int32)
    ne = np.zeros(1, np.int64)
    rc = lib().tor_neighbors(n, _ptr(_box(box)), _ptr(pos), r_cut, skin, method, 0, _ptr(row_ptr),
                             None, _ptr(ne))
    if rc not in (OK, ERR_CAPACITY):
        raise RuntimeError("oracle neighbours failed: %d" % rc)
    cap = int(ne[0]) if cap is None else cap
    col = np.zeros(max(cap, 1), np.uint32)
    rc = lib().tor_neighbors(n, _ptr(_box(box)), _ptr(pos), r_cut, skin, method, cap,
                             _ptr(row_ptr), _ptr(col), _ptr(ne))
    if rc != OK:
        raise RuntimeError("oracle neighbours failed: %d" % rc)
    return row_ptr, col[: int(ne[0])]


def neighbors_status(box, pos, r_cut, skin, method=1, cap=0):
    pos = _f32(pos).reshape(-1, 3)
    n = pos.shape[0]
    row_ptr = np.zeros(n + 1, np.int32)
    col = np.zeros(max(cap, 1), np.uint32)
    ne = np.zeros(1, np.int64)
    rc = lib().tor_neighbors(n, _ptr(_box(box)), _ptr(pos), r_cut, skin, method, cap,
                             _ptr(row_ptr), _ptr(col), _ptr(ne))
    return int(rc), int(ne[0])


def flagged_pairs(box, pos, r_cut, skin, band=1e-5):
    pos = _f32(pos).reshape(-1, 3)
    n = pos.shape[0]
    cnt = lib().tor_flagged_pairs(n, _ptr(_box(box)), _ptr(pos), r_cut, skin, band, 0, None, None)
    fi = np.zeros(max(cnt, 1), np.int32)
    fj = np.zeros(max(cnt, 1), np.int32)
    lib().tor_flagged_pairs(n, _ptr(_box(box)), _ptr(pos), r_cut, skin, band, cnt, _ptr(fi), _ptr(fj))
    return fi[:cnt], fj[:cnt]


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(lib().tor_num_threads())


def build_neighbors(box, pos, species, r_cut, skin, vel=None):
    """Full rebuild. Returns dict(pos, species, vel, perm, keys, row_ptr, col_shift)."""
    pos = _f32(pos).reshape(-1, 3).copy()
    n = pos.shape[0]
    sp = np.ascontiguousarray(species, dtype=np.int32).copy()
    v = None if vel is None else np.ascontiguousarray(vel, dtype=np.float64).reshape(-1, 3).copy()
    perm = np.empty(n, np.int32)
    keys = np.empty(n, np.uint32)
    row_ptr = np.zeros(n + 1, np.int32)
    ne = np.zeros(1, np.int64)
    # first pass sizes the list; the rebuild is deterministic, so run it twice
    p0, s0 = pos.copy(), sp.copy()
    rc = lib().tor_build_neighbors(n, _ptr(_box(box)), r_cut, skin, _ptr(p0), _ptr(s0), None,
                                   _ptr(perm), None, 0, _ptr(row_ptr), None, _ptr(ne))
    if rc not in (OK, ERR_CAPACITY):
        raise RuntimeError("oracle rebuild failed: %d" % rc)
    cap = int(ne[0])
    col = np.zeros(max(cap, 1), np.uint32)
    rc = lib().tor_build_neighbors(n, _ptr(_box(box)), r_cut, skin, _ptr(pos), _ptr(sp), _ptr(v),
                                   _ptr(perm), _ptr(keys), cap, _ptr(row_ptr), _ptr(col), _ptr(ne))
    if rc != OK:
        raise RuntimeError("oracle rebuild failed: %d" % rc)
    return dict(pos=pos, species=sp, vel=v, perm=perm, keys=keys, row_ptr=row_ptr,
                col_shift=col[:cap])


# ---- model ----------------------------------------------------------------------------

def n_paths(l_max: int) -> int:
    return int(lib().tor_n_paths(l_max))


def sph(l_max: int, nvec):
    nv = np.ascontiguousarray(nvec, dtype=np.float64)
    Y = np.zeros(9, np.float64)
    lib().tor_sph(l_max, _ptr(nv), _ptr(Y))
    return Y[: (l_max + 1) ** 2]


def paths(l_max: int):
    P = n_paths(l_max)
    a, b, c = (np.zeros(16, np.int32) for _ in range(3))
    lib().tor_paths(l_max, _ptr(a), _ptr(b), _ptr(c))
    return list(zip(a[:P].tolist(), b[:P].tolist(), c[:P].tolist()))


def coupling(l_max: int):
    P = n_paths(l_max)
    cg = np.zeros((max(P, 1), 5, 5, 5), np.float64)
    lib().tor_coupling(l_max, _ptr(cg))
    return cg[:P]


def weights_count(spec) -> int:
    m = model_struct(spec)
    return int(lib().tor_weights_count(C.byref(m)))


def energy_forces(spec, weights, box, pos, species, row_ptr, col_shift, want_forces=True,
                  want_feats=False):
    """fp64 energy, per-atom energies and forces of positions in the CSR's order."""
    m = model_struct(spec)
    pos = np.ascontiguousarray(pos, dtype=np.float64).reshape(-1, 3)
    n = pos.shape[0]
    w = _f32(weights)
    sp = np.ascontiguousarray(species, dtype=np.int32)
    rp = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col = np.ascontiguousarray(col_shift, dtype=np.uint32)
    E = np.zeros(1, np.float64)
    ea = np.zeros(n, np.float64)
    F = np.zeros((n, 3), np.float64) if want_forces else None
    D = (spec.l_max + 1) ** 2
    feats = np.zeros((n, spec.channels, D), np.float64) if want_feats else None
    rc = lib().tor_energy_forces(C.byref(m), _ptr(w), n, _ptr(_box(box)), _ptr(pos), _ptr(sp),
                                 _ptr(rp), _ptr(col), _ptr(E), _ptr(ea), _ptr(F), _ptr(feats))
    if rc != OK:
        raise RuntimeError("oracle energy_forces failed: %d" % rc)
    out = dict(energy=float(E[0]), e_atom=ea, forces=F)
    if want_feats:
        out["feats"] = feats
    return out


def energy_forces_status(spec, weights, box, pos, species, row_ptr, col_shift):
    m = model_struct(spec)
    pos = np.ascontiguousarray(pos, dtype=np.float64).reshape(-1, 3)
    E = np.zeros(1, np.float64)
    return int(lib().tor_energy_forces(C.byref(m), _ptr(_f32(weights)), pos.shape[0],
                                       _ptr(_box(box)), _ptr(pos),
                                       _ptr(np.ascontiguousarray(species, dtype=np.int32)),
                                       _ptr(np.ascontiguousarray(row_ptr, dtype=np.int32)),
                                       _ptr(np.ascontiguousarray(col_shift, dtype=np.uint32)),
                                       _ptr(E), None, None, None))


def md_steps(spec, weights, box, r_cut, skin, pos, vel, species, masses, dt_fs, n_steps,
             rebuild_every, perm_accum=None, forces=None, cap=None, thermostat=0,
             t_target_K=0.0, tau_fs=0.0):
    m = model_struct(spec)
    pos = np.ascontiguousarray(pos, dtype=np.float64).reshape(-1, 3).copy()
    vel = np.ascontiguousarray(vel, dtype=np.float64).reshape(-1, 3).copy()
    sp = np.ascontiguousarray(species, dtype=np.int32).copy()
    n = pos.shape[0]
    pa = np.arange(n, dtype=np.int32) if perm_accum is None else np.ascontiguousarray(
        perm_accum, dtype=np.int32).copy()
    valid = forces is not None
    F = np.zeros((n, 3), np.float64) if forces is None else np.ascontiguousarray(
        forces, dtype=np.float64).reshape(-1, 3).copy()
    ep = np.zeros(max(n_steps, 1), np.float64)
    ke = np.zeros(max(n_steps, 1), np.float64)
    rmin = np.zeros(max(n_steps, 1), np.float64)
    if cap is None:
        cap = 400 * n
    ms = np.ascontiguousarray(masses, dtype=np.float64)
    rc = lib().tor_md_steps(C.byref(m), _ptr(_f32(weights)), n, _ptr(_box(box)), r_cut, skin,
                            _ptr(pos), _ptr(vel), _ptr(sp), _ptr(ms), dt_fs, n_steps,
                            rebuild_every, _ptr(pa), _ptr(F), int(valid), _ptr(ep), int(cap),
                            int(thermostat), float(t_target_K), float(tau_fs), _ptr(ke),
                            _ptr(rmin))
    return dict(status=int(rc), pos=pos, vel=vel, species=sp, perm_accum=pa, forces=F,
                epot=ep[:n_steps], ke=ke[:n_steps], rmin=rmin[:n_steps])
