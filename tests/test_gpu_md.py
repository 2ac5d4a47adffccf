"""GPU parity of tess_md_steps (velocity Verlet between rebuilds) against the fp64 oracle's
md_steps on the same start state. Over one 20-step interval (and over two intervals with a
rebuild between them) positions agree within 1e-4 A and velocities within 1e-5 A/fs per
component, compared per original atom id; the potential-energy trace within 1e-5 relative."""
import numpy as np
import pytest

from molecular_dynamics_hilbert_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def T():
    import torch
    assert torch.cuda.is_available()
    from molecular_dynamics_hilbert_amd import tess
    tess.lib()
    return tess


def _gpu_md(T, wl, w, vel, steps, every, skin=None, scale_v=1.0):
    import torch
    s = T.System(wl, w, skin=skin)
    dev = "cuda"
    vel_t = torch.from_numpy((vel * scale_v).astype(np.float32)).to(dev)
    masses = torch.from_numpy(wl.masses().astype(np.float32)).to(dev)
    pa = torch.arange(wl.n, dtype=torch.int32, device=dev)
    ep = torch.zeros(steps, dtype=torch.float64, device=dev)
    st, ne = T.md_steps(s.spec, s.weights, s.box, s.r_cut, s.skin, s.pos, vel_t, s.species, masses,
                        wl.dt_fs, steps, every, pa, s.forces, s.row_ptr, s.col_shift, s.rev, s.ws,
                        epot_trace=ep, check=False)
    torch.cuda.synchronize()
    return dict(status=st, pos=s.pos.cpu().numpy().astype(np.float64),
                vel=vel_t.cpu().numpy().astype(np.float64), pa=pa.cpu().numpy(),
                forces=s.forces.cpu().numpy().astype(np.float64), epot=ep.cpu().numpy())


def _compare(T, oracle_mod, wname, steps, every, wseed, scale=1.0, temp=50.0):
    """Random weights bind nothing, so at 300 K the fastest H atoms pass skin/2 within one
    20-step interval; the parity runs start at 50 K so that no interval is flagged."""
    wl = W.load(wname)
    w = W.make_weights(wl.model, wseed)
    w[-wl.model.channels:] *= scale
    vel = W.maxwell_velocities(wl.species, wl.masses(), temp, 3000 + wseed % 1000)
    g = _gpu_md(T, wl, w, vel, steps, every)
    o = oracle_mod.md_steps(wl.model, w, wl.box, wl.model.r_cut, wl.skin, wl.pos, vel, wl.species,
                            wl.masses(), wl.dt_fs, steps, every)
    assert g["status"] == o["status"] == 0
    assert np.array_equal(np.sort(g["pa"]), np.arange(wl.n))
    xg = np.empty((wl.n, 3)); xg[g["pa"]] = g["pos"]
    xo = np.empty((wl.n, 3)); xo[o["perm_accum"]] = o["pos"]
    vg = np.empty((wl.n, 3)); vg[g["pa"]] = g["vel"]
    vo = np.empty((wl.n, 3)); vo[o["perm_accum"]] = o["vel"]
    L = float(wl.box[0])
    dx = xg - xo
    dx -= L * np.round(dx / L)
    print("%s steps=%d max|dx|=%.2e max|dv|=%.2e" % (wname, steps, np.abs(dx).max(),
                                                     np.abs(vg - vo).max()), flush=True)
    assert np.abs(dx).max() <= 1e-4
    assert np.abs(vg - vo).max() <= 1e-5
    assert np.all(np.abs(g["epot"] - o["epot"]) <= 1e-5 * np.abs(o["epot"]))
    return g, o


def test_md_one_interval_water(T, oracle_mod):
    _compare(T, oracle_mod, "water648", 20, 20, 2001, scale=10.0)


def test_md_two_intervals_with_rebuild(T, oracle_mod):
    _compare(T, oracle_mod, "water648", 20, 10, 2001, scale=10.0)


def test_md_salt4k_short(T, oracle_mod):
    _compare(T, oracle_mod, "salt4k", 6, 3, 2002)


def test_md_skin_error(T, oracle_mod):
    """At 300 K some H atom passes skin/2 within the first interval: both the library and the
    oracle finish that interval and report it."""
    wl = W.load("water648")
    w = W.make_weights(wl.model, 2001)
    vel = W.maxwell_velocities(wl.species, wl.masses(), 300.0, 3001)
    g = _gpu_md(T, wl, w, vel, 40, 20)
    o = oracle_mod.md_steps(wl.model, w, wl.box, wl.model.r_cut, wl.skin, wl.pos, vel, wl.species,
                            wl.masses(), wl.dt_fs, 40, 20)
    assert g["status"] == o["status"] == T.ERR_SKIN
    xg = np.empty((wl.n, 3)); xg[g["pa"]] = g["pos"]
    xo = np.empty((wl.n, 3)); xo[o["perm_accum"]] = o["pos"]
    dx = xg - xo
    dx -= float(wl.box[0]) * np.round(dx / float(wl.box[0]))
    assert np.abs(dx).max() <= 1e-4


def test_md_graph_replay_matches_eager(T):
    """TESS_MD_GRAPH: the steps of a rebuild interval are captured into a HIP graph once and
    replayed. Two identical systems, one eager and one replayed, run three calls of two
    20-step intervals each (the first interval captures, every later one replays), with
    unrelated eager GPU work and synchronisations between the calls; after every call
    positions, velocities, forces, the permutation and the energy trace are bit-identical."""
    import torch
    wl = W.load("salt4k")
    w = W.make_weights(wl.model, 2002)
    vel = W.maxwell_velocities(wl.species, wl.masses(), 50.0, 3002).astype(np.float32)
    dev = "cuda"
    masses = torch.from_numpy(wl.masses().astype(np.float32)).to(dev)
    runs = []
    for graph in (False, True):
        s = T.System(wl, w)
        runs.append(dict(s=s, graph=graph, vel=torch.from_numpy(vel.copy()).to(dev),
                         pa=torch.arange(wl.n, dtype=torch.int32, device=dev),
                         ep=torch.zeros(40, dtype=torch.float64, device=dev)))
    other = T.System(W.load("water648"), W.make_weights(W.load("water648").model, 2001))
    other.rebuild()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()  # graphs are not captured on the NULL stream
    with torch.cuda.stream(stream):
        assert torch.cuda.current_stream().cuda_stream != 0
        _graph_calls(T, torch, wl, masses, runs, other)


def _graph_calls(T, torch, wl, masses, runs, other):
    for call in range(3):
        for r in runs:
            s = r["s"]
            st, _ = T.md_steps(s.spec, s.weights, s.box, s.r_cut, s.skin, s.pos, r["vel"],
                               s.species, masses, wl.dt_fs, 40, 20, r["pa"], s.forces, s.row_ptr,
                               s.col_shift, s.rev, s.ws, epot_trace=r["ep"],
                               forces_valid=call > 0, graph=r["graph"], check=False)
            assert st == T.OK
            torch.cuda.synchronize()
            other.energy_forces()  # eager work between replays
            torch.cuda.synchronize()
        a, b = runs[0], runs[1]
        assert torch.equal(a["s"].pos, b["s"].pos)
        assert torch.equal(a["vel"], b["vel"])
        assert torch.equal(a["s"].forces, b["s"].forces)
        assert torch.equal(a["pa"], b["pa"])
        assert torch.equal(a["ep"], b["ep"])
        print("call %d: identical, E=%.6f" % (call, float(b["ep"][-1])), flush=True)


def test_nve_energy_conservation(T):
    """Energy conservation of velocity Verlet with the library's forces (F = -dE/dx): salt4k
    at 50 K, 400 steps of 0.5 fs (200 fs, a rebuild every 20 steps). The total energy
    E_pot + E_kin at every interval boundary stays within 2e-6 eV/atom of its start and its
    linear drift is below 1e-6 eV/atom/ps (measured: 1.2e-7 and 2.4e-9). With random weights this is a smoothness and
    consistency check of the forces, not a physical drift figure."""
    import torch
    wl = W.load("salt4k")
    w = W.make_weights(wl.model, 2002)
    vel0 = W.maxwell_velocities(wl.species, wl.masses(), 50.0, 3002).astype(np.float32)
    s = T.System(wl, w)
    dev = "cuda"
    vel = torch.from_numpy(vel0).to(dev)
    m = wl.masses().astype(np.float64)
    masses = torch.from_numpy(wl.masses().astype(np.float32)).to(dev)
    pa = torch.arange(wl.n, dtype=torch.int32, device=dev)
    ep = torch.zeros(20, dtype=torch.float64, device=dev)
    conv = 9.648533e-3  # eV/A/amu -> A/fs^2
    t, etot = [], []
    for call in range(20):
        st, _ = T.md_steps(s.spec, s.weights, s.box, s.r_cut, s.skin, s.pos, vel, s.species,
                           masses, wl.dt_fs, 20, 20, pa, s.forces, s.row_ptr, s.col_shift, s.rev,
                           s.ws, epot_trace=ep, forces_valid=call > 0, check=False)
        assert st == T.OK
        v = vel.cpu().numpy().astype(np.float64)
        mm = m[wl.species[pa.cpu().numpy()]]
        ekin = 0.5 * float((mm[:, None] * v * v).sum()) / conv
        etot.append(float(ep[-1].cpu()) + ekin)
        t.append((call + 1) * 20 * wl.dt_fs * 1e-3)  # ps
    e = (np.array(etot) - etot[0]) / wl.n
    slope = np.polyfit(np.array(t), e, 1)[0]
    print("NVE salt4k: max|dE_tot|/atom = %.2e eV, drift %.2e eV/atom/ps" % (np.abs(e).max(),
                                                                            slope), flush=True)
    assert np.abs(e).max() < 2e-6
    assert abs(slope) < 1e-6
