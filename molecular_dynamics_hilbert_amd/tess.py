"""Thin ctypes binding of libtess.so (include/tess.h). Argument marshalling only: every step
of the hot path runs in the library's HIP kernels. torch supplies device memory and the
current stream; it is imported before the library so that both share one HIP runtime.

The library must have been built (``python -m molecular_dynamics_hilbert_amd.build`` or
``__graft_entry__.build()``); there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtess.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "tess.h")

(OK, ERR_ARG, ERR_BOX, ERR_CAPACITY, ERR_WORKSPACE, ERR_HIP, ERR_SKIN, ERR_SPECIES,
 ERR_NONFINITE, ERR_ROW, ERR_RADIAL) = (0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10)
MD_FORCES_VALID = 1
MD_GRAPH = 2


class TessError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (what, status_string(status), status))


class ModelDesc(C.Structure):
    _fields_ = [("n_species", C.c_int32), ("n_layers", C.c_int32), ("channels", C.c_int32),
                ("l_max", C.c_int32), ("n_heads", C.c_int32), ("n_rbf", C.c_int32),
                ("radial_hidden", C.c_int32), ("r_cut", C.c_float)]


THERMOSTAT_NONE, THERMOSTAT_BERENDSEN = 0, 1


class MdOptions(C.Structure):
    _fields_ = [("thermostat", C.c_int32), ("t_target_K", C.c_float), ("tau_fs", C.c_float),
                ("ke_trace", C.c_void_p), ("rmin_trace", C.c_void_p)]


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libtess.so is not built (%s); build it with "
                               "python -m molecular_dynamics_hilbert_amd.build" % LIB_PATH)
        L = C.CDLL(LIB_PATH)
        p, i32, i64, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_float
        L.tess_abi_version.restype = i32
        L.tess_status_string.restype = C.c_char_p
        L.tess_status_string.argtypes = [i32]
        L.tess_weights_count.restype = i64
        L.tess_weights_count.argtypes = [p]
        L.tess_workspace_bytes.restype = i64
        L.tess_workspace_bytes.argtypes = [p, i32, i64]
        L.tess_build_neighbors.restype = i32
        L.tess_build_neighbors.argtypes = [i32, p, f32, f32, p, p, p, p, p, p, p, p, p, i64, p, p,
                                           i64, p]
        L.tess_energy_forces.restype = i32
        L.tess_energy_forces.argtypes = [p, p, i32, p, p, p, p, p, p, i64, p, p, p, p, i64, p]
        L.tess_md_steps.restype = i32
        L.tess_md_steps.argtypes = [p, p, i32, p, f32, f32, p, p, p, p, f32, i32, i32, i32, p, p,
                                    p, p, p, p, i64, p, p, i64, p]
        L.tess_md_steps_ex.restype = i32
        L.tess_md_steps_ex.argtypes = [p, p, i32, p, f32, f32, p, p, p, p, f32, i32, i32, i32, p,
                                       p, p, p, p, p, i64, p, p, i64, p, p]
        L.tess_timing_enable.restype = i32
        L.tess_timing_enable.argtypes = [i32]
        L.tess_timing_read.restype = i32
        L.tess_timing_read.argtypes = [C.c_char_p, p, p]
        L.tess_timing_only.restype = i32
        L.tess_timing_only.argtypes = [C.c_char_p]
        L.tess_set_curve.restype = i32
        L.tess_set_curve.argtypes = [i32]
        L.tess_check_status.restype = i32
        L.tess_check_status.argtypes = [p, i64, p]
        L.tess_build_neighbors_static.restype = i32
        L.tess_build_neighbors_static.argtypes = [i32, p, f32, f32, p, p, p, p, p, p, p, p, p,
                                                  i64, p, p]
        _lib = L
    return _lib


def timing_enable(on: bool) -> None:
    lib().tess_timing_enable(1 if on else 0)


def set_curve(curve: str) -> None:
    """Atom order of later rebuilds: "hilbert" (default) or "morton" (comparison runs)."""
    st = lib().tess_set_curve({"hilbert": 0, "morton": 1}[curve])
    if st != OK:
        raise TessError(st, "tess_set_curve")


def timing_only(kernel=None) -> None:
    """Time only `kernel` (None: every instrumented kernel)."""
    lib().tess_timing_only(kernel.encode() if kernel else None)


def timing_read(kernel: str):
    """(total_ms, launches) of an instrumented kernel since timing_enable(True)."""
    ms = C.c_double(0.0)
    cnt = C.c_int64(0)
    st = lib().tess_timing_read(kernel.encode(), C.byref(ms), C.byref(cnt))
    if st != OK:
        raise TessError(st, "tess_timing_read")
    return ms.value, cnt.value


def header_functions() -> list:
    """Names of the functions include/tess.h declares."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int32_t|int64_t|const char\*)\s+(tess_\w+)\s*\(", txt, re.M)))


def status_string(s: int) -> str:
    return lib().tess_status_string(int(s)).decode()


def desc(spec) -> ModelDesc:
    t = spec.as_tuple() if hasattr(spec, "as_tuple") else tuple(spec)
    return ModelDesc(*[int(v) for v in t[:7]], float(t[7]))


def weights_count(spec) -> int:
    return int(lib().tess_weights_count(C.byref(desc(spec))))


def workspace_bytes(spec, n: int, edge_cap: int) -> int:
    d = None if spec is None else C.byref(desc(spec))
    return int(lib().tess_workspace_bytes(d, int(n), int(edge_cap)))


def _p(t):
    if t is None:
        return None
    assert t.is_cuda and t.is_contiguous(), "device, contiguous tensors required"
    return C.c_void_p(t.data_ptr())


def _box(box):
    b = (C.c_float * 3)(*[float(x) for x in box])
    return b


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def workspace(spec, n: int, edge_cap: int, device="cuda") -> torch.Tensor:
    """A workspace of tess_workspace_bytes() bytes whose device status word (its first
    word) starts at zero and whose other bytes start as 0xFF."""
    nb = workspace_bytes(spec, n, edge_cap)
    if nb < 0:
        raise TessError(ERR_ARG, "tess_workspace_bytes")
    # every byte but the status word's line starts as 0xFF (a NaN in every float), so a read of
    # anything the library did not write first shows up in the results
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device=device)
    ws[:256].zero_()
    return ws


def check_status(ws, check=True) -> int:
    """tess_check_status: synchronise the current stream, report and clear the workspace's
    device status word."""
    st = lib().tess_check_status(_p(ws), int(ws.numel()), _stream())
    if check and st != OK:
        raise TessError(st, "tess_check_status")
    return st


def build_neighbors(box, r_cut, skin, pos, species, perm, row_ptr, col_shift, ws, vel=None,
                    ref_pos=None, hkey=None, rev=None, check=True):
    """tess_build_neighbors on device tensors (pos float32[n,3], species int32[n], perm int32[n],
    row_ptr int32[n+1], col_shift uint32/int32[cap]). Returns (status, n_edges)."""
    n = int(pos.shape[0])
    ne = C.c_int64(0)
    cap = int(col_shift.numel()) if col_shift is not None else 0
    st = lib().tess_build_neighbors(n, _box(box), float(r_cut), float(skin), _p(pos), _p(species),
                                    _p(vel), _p(ref_pos), _p(perm), _p(hkey), _p(row_ptr),
                                    _p(col_shift), _p(rev), cap, C.byref(ne), _p(ws),
                                    int(ws.numel()), _stream())
    if check and st != OK:
        raise TessError(st, "tess_build_neighbors")
    return st, int(ne.value)


def build_neighbors_static(box, r_cut, skin, pos, species, perm, row_ptr, col_shift, vel=None,
                           ref_pos=None, hkey=None, rev=None, check=True):
    """tess_build_neighbors_static: build_neighbors with the library's own device scratch (no
    workspace). Returns (status, n_edges)."""
    n = int(pos.shape[0])
    ne = C.c_int64(0)
    cap = int(col_shift.numel()) if col_shift is not None else 0
    st = lib().tess_build_neighbors_static(n, _box(box), float(r_cut), float(skin), _p(pos),
                                           _p(species), _p(vel), _p(ref_pos), _p(perm),
                                           _p(hkey), _p(row_ptr), _p(col_shift), _p(rev), cap,
                                           C.byref(ne), _stream())
    if check and st != OK:
        raise TessError(st, "tess_build_neighbors_static")
    return st, int(ne.value)


def energy_forces(spec, weights, box, pos, species, row_ptr, col_shift, rev, n_edges, energy, ws,
                  e_atom=None, forces=None, check=True):
    n = int(pos.shape[0])
    st = lib().tess_energy_forces(C.byref(desc(spec)), _p(weights), n, _box(box), _p(pos),
                                  _p(species), _p(row_ptr), _p(col_shift), _p(rev), int(n_edges),
                                  _p(energy), _p(e_atom), _p(forces), _p(ws), int(ws.numel()),
                                  _stream())
    if check and st != OK:
        raise TessError(st, "tess_energy_forces")
    return st


def md_steps(spec, weights, box, r_cut, skin, pos, vel, species, mass_by_species, dt_fs, n_steps,
             rebuild_every, perm_accum, forces, row_ptr, col_shift, rev, ws, epot_trace=None,
             forces_valid=False, graph=False, check=True, thermostat=None, t_target_K=0.0,
             tau_fs=0.0, ke_trace=None, rmin_trace=None):
    """tess_md_steps, or tess_md_steps_ex when a thermostat ("berendsen") or a trace
    (ke_trace float64[n_steps], rmin_trace float32[n_steps]) is given."""
    n = int(pos.shape[0])
    ne = C.c_int64(0)
    args = [C.byref(desc(spec)), _p(weights), n, _box(box), float(r_cut), float(skin), _p(pos),
            _p(vel), _p(species), _p(mass_by_species), float(dt_fs), int(n_steps),
            int(rebuild_every),
            (MD_FORCES_VALID if forces_valid else 0) | (MD_GRAPH if graph else 0),
            _p(perm_accum), _p(forces), _p(epot_trace), _p(row_ptr), _p(col_shift), _p(rev),
            int(col_shift.numel()), C.byref(ne), _p(ws), int(ws.numel())]
    if thermostat is None and ke_trace is None and rmin_trace is None:
        st = lib().tess_md_steps(*args, _stream())
        name = "tess_md_steps"
    else:
        kinds = {None: THERMOSTAT_NONE, "none": THERMOSTAT_NONE,
                 "berendsen": THERMOSTAT_BERENDSEN}
        opt = MdOptions(kinds[thermostat] if thermostat in kinds else int(thermostat),
                        float(t_target_K), float(tau_fs), _p(ke_trace), _p(rmin_trace))
        st = lib().tess_md_steps_ex(*args, C.byref(opt), _stream())
        name = "tess_md_steps_ex"
    if check and st != OK:
        raise TessError(st, name)
    return st, int(ne.value)


class System:
    """Device-resident state of one workload: positions, species, neighbour list, workspace.
    Convenience for tests and the benchmark; all work happens in the library."""

    def __init__(self, wl, weights, edge_cap=None, device="cuda", skin=None, vel=None):
        self.wl = wl
        self.spec = wl.model
        self.box = [float(x) for x in wl.box]
        self.r_cut = float(wl.model.r_cut)
        self.skin = float(wl.skin if skin is None else skin)
        n = wl.n
        self.n = n
        self.pos = torch.from_numpy(wl.pos.copy()).to(device)
        self.species = torch.from_numpy(wl.species.copy()).to(device)
        self.vel = None if vel is None else torch.from_numpy(vel.copy()).to(device)
        self.weights = torch.from_numpy(weights).to(device)
        self.perm = torch.empty(n, dtype=torch.int32, device=device)
        self.hkey = torch.empty(n, dtype=torch.int32, device=device)
        self.row_ptr = torch.empty(n + 1, dtype=torch.int32, device=device)
        if edge_cap is None:
            # probe: one rebuild without room for pairs gives the exact count
            ws0 = workspace(None, n, 0, device)
            p0, s0 = self.pos.clone(), self.species.clone()
            st, ne = build_neighbors(self.box, self.r_cut, self.skin, p0, s0, self.perm,
                                     self.row_ptr, torch.empty(0, dtype=torch.int32, device=device),
                                     ws0, check=False)
            if st not in (OK, ERR_CAPACITY):
                raise TessError(st, "tess_build_neighbors")
            if ne > 2**31 - 1:  # beyond what the int32 row offsets can hold
                raise TessError(ERR_CAPACITY, "tess_build_neighbors (%d pairs)" % ne)
            edge_cap = max(1, int(1.15 * ne) + 64)
        self.edge_cap = edge_cap
        self.col_shift = torch.empty(edge_cap, dtype=torch.int32, device=device)
        self.rev = torch.empty(edge_cap, dtype=torch.int32, device=device)
        self.ws = workspace(self.spec, n, edge_cap, device)
        self.energy = torch.zeros(1, dtype=torch.float64, device=device)
        self.e_atom = torch.zeros(n, dtype=torch.float32, device=device)
        self.forces = torch.zeros((n, 3), dtype=torch.float32, device=device)
        self.n_edges = 0

    def rebuild(self):
        st, self.n_edges = build_neighbors(self.box, self.r_cut, self.skin, self.pos, self.species,
                                           self.perm, self.row_ptr, self.col_shift, self.ws,
                                           vel=self.vel, hkey=self.hkey, rev=self.rev)
        return self.n_edges

    def energy_forces(self, forces=True):
        energy_forces(self.spec, self.weights, self.box, self.pos, self.species, self.row_ptr,
                      self.col_shift, self.rev, self.n_edges, self.energy, self.ws,
                      e_atom=self.e_atom, forces=self.forces if forces else None)
