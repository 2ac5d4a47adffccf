"""Host-side checks of libtess.so that need no GPU: it loads next to torch on one HIP runtime,
exports every function include/tess.h declares, and rejects bad arguments, unsupported shapes,
small boxes and small workspaces before enqueueing anything."""
import ctypes as C
import re

import numpy as np
import pytest

from molecular_dynamics_hilbert_amd import workloads as W


@pytest.fixture(scope="module")
def T():
    from molecular_dynamics_hilbert_amd import tess
    tess.lib()
    return tess


def test_exports_every_declared_function(T):
    names = T.header_functions()
    assert {"tess_build_neighbors", "tess_energy_forces", "tess_md_steps"} <= set(names)
    for nm in names:
        assert hasattr(T.lib(), nm), nm


def test_single_hip_runtime(T):
    maps = open("/proc/self/maps").read()
    paths = set(re.findall(r"(\S*libamdhip64\S*)", maps))
    assert len(paths) == 1, paths


def test_counts_and_status(T):
    assert T.lib().tess_abi_version() == 2
    for wl in (W.water648(), W.salt4k()):
        assert T.weights_count(wl.model) == W.weight_count(wl.model)
    assert T.weights_count(W.big_model()) == W.weight_count(W.big_model())
    bad = W.ModelSpec(n_species=2, n_layers=1, channels=24, l_max=1, n_heads=1)
    assert T.weights_count(bad) == -1
    assert T.workspace_bytes(W.big_model(), 1000, 200000) > T.workspace_bytes(W.big_model(), 1000, 100000)
    assert T.status_string(T.ERR_CAPACITY).startswith("neighbour list")


def test_host_side_rejections(T):
    L = T.lib()
    fake = C.c_void_p(0x1000)  # never dereferenced: every call below fails host-side
    ne = C.c_int64(0)
    small = (C.c_float * 3)(13.0, 13.0, 13.0)
    ok_box = (C.c_float * 3)(30.0, 30.0, 30.0)
    assert L.tess_build_neighbors(10, small, 5.75, 1.0, fake, fake, None, None, fake, None, fake,
                                  fake, None, 100, C.byref(ne), fake, 1 << 30, None) == T.ERR_BOX
    assert L.tess_build_neighbors(10, ok_box, 5.75, 1.0, fake, fake, None, None, fake, None, fake,
                                  fake, None, 100, C.byref(ne), fake, 16, None) == T.ERR_WORKSPACE
    assert L.tess_build_neighbors(-1, ok_box, 5.75, 1.0, fake, fake, None, None, fake, None, fake,
                                  fake, None, 100, C.byref(ne), fake, 1 << 30, None) == T.ERR_ARG
    bad = T.desc(W.ModelSpec(n_species=2, n_layers=1, channels=24, l_max=1, n_heads=1))
    e = L.tess_energy_forces(C.byref(bad), fake, 10, ok_box, fake, fake, fake, fake, None, 10,
                             fake, None, None, fake, 1 << 40, None)
    assert e == T.ERR_ARG
    good = T.desc(W.water648().model)
    e = L.tess_energy_forces(C.byref(good), fake, 10, ok_box, fake, fake, fake, fake, None, 10,
                             fake, None, None, fake, 8, None)
    assert e == T.ERR_WORKSPACE


def test_md_options_rejected_host_side(T):
    """tess_md_steps_ex checks its thermostat options before enqueueing anything."""
    L = T.lib()
    fake = C.c_void_p(0x1000)
    ne = C.c_int64(0)
    box = (C.c_float * 3)(30.0, 30.0, 30.0)
    good = T.desc(W.water648().model)
    rc = float(W.water648().model.r_cut)

    def call(opt, ws_bytes=1 << 40):
        return L.tess_md_steps_ex(C.byref(good), fake, 10, box, rc, 1.0, fake, fake, fake, fake,
                                  0.5, 4, 20, 0, fake, fake, None, fake, fake, fake, 100,
                                  C.byref(ne), fake, ws_bytes, opt, None)

    for o in (T.MdOptions(T.THERMOSTAT_BERENDSEN, 300.0, 0.25, None, None),  # tau < dt
              T.MdOptions(T.THERMOSTAT_BERENDSEN, -5.0, 10.0, None, None),
              T.MdOptions(T.THERMOSTAT_BERENDSEN, float("nan"), 10.0, None, None),
              T.MdOptions(7, 300.0, 10.0, None, None)):
        assert call(C.byref(o)) == T.ERR_ARG
    # valid options reach the workspace check
    o = T.MdOptions(T.THERMOSTAT_BERENDSEN, 300.0, 10.0, None, None)
    assert call(C.byref(o), ws_bytes=8) == T.ERR_WORKSPACE
    assert call(None, ws_bytes=8) == T.ERR_WORKSPACE


def test_misaligned_weights_and_workspace_rejected(T):
    """The weights blob and the workspace are read with 16-byte loads: a pointer that is not
    16-byte aligned is refused on the host before anything is enqueued."""
    L = T.lib()
    wl = W.water648()
    d = T.desc(wl.model)
    box = (C.c_float * 3)(30.0, 30.0, 30.0)
    fake = C.c_void_p(0x1000)
    e = C.c_void_p(0x2000)

    def ef(weights, ws):
        return L.tess_energy_forces(C.byref(d), weights, 10, box, fake, fake, fake, fake, None,
                                    0, e, None, None, ws, 1 << 40, None)

    assert ef(C.c_void_p(0x1004), fake) == T.ERR_ARG
    assert ef(fake, C.c_void_p(0x1008)) == T.ERR_WORKSPACE
    ne = C.c_int64(0)
    assert L.tess_build_neighbors(10, box, 5.75, 1.0, fake, fake, None, None, fake, fake, fake,
                                  fake, None, 100, C.byref(ne), C.c_void_p(0x1001), 1 << 40,
                                  None) == T.ERR_WORKSPACE
    rc = float(wl.model.r_cut)
    assert L.tess_md_steps_ex(C.byref(d), C.c_void_p(0x100c), 10, box, rc, 1.0, fake, fake, fake,
                              fake, 0.5, 4, 20, 0, fake, fake, None, fake, fake, fake, 100,
                              C.byref(ne), fake, 1 << 40, None, None) == T.ERR_ARG
