"""tess_build_neighbors_static (the rebuild with the library's own device scratch, for callers
that cannot allocate) against tess_build_neighbors on the same inputs: every output bit for
bit, on two calls in a row (60,000 atoms, then 4,096: the second call finds the first call's
contents in the shared scratch), plus the size limit."""
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


def _outputs(T, wl, static, cap):
    import torch
    dev = "cuda"
    n = wl.n
    pos = torch.from_numpy(wl.pos.copy()).to(dev)
    sp = torch.from_numpy(wl.species.copy()).to(dev)
    vel = torch.from_numpy(np.arange(3 * n, dtype=np.float32).reshape(n, 3)).to(dev)
    ref = torch.empty((n, 3), dtype=torch.float32, device=dev)
    perm = torch.empty(n, dtype=torch.int32, device=dev)
    hkey = torch.empty(n, dtype=torch.int32, device=dev)
    rp = torch.empty(n + 1, dtype=torch.int32, device=dev)
    col = torch.full((cap,), -1, dtype=torch.int32, device=dev)
    rev = torch.full((cap,), -1, dtype=torch.int32, device=dev)
    if static:
        st, ne = T.build_neighbors_static(wl.box, wl.model.r_cut, wl.skin, pos, sp, perm, rp, col,
                                          vel=vel, ref_pos=ref, hkey=hkey, rev=rev, check=False)
    else:
        ws = T.workspace(None, n, cap)
        st, ne = T.build_neighbors(wl.box, wl.model.r_cut, wl.skin, pos, sp, perm, rp, col, ws,
                                   vel=vel, ref_pos=ref, hkey=hkey, rev=rev, check=False)
    torch.cuda.synchronize()
    assert st == T.OK
    out = dict(pos=pos, sp=sp, vel=vel, ref=ref, perm=perm, hkey=hkey, rp=rp,
               col=col[:ne], rev=rev[:ne])
    return ne, {k: v.cpu().numpy() for k, v in out.items()}


def test_static_rebuild_matches_workspace_rebuild(T):
    for name in ("salt60k", "salt4k"):  # the second call is smaller
        wl = W.load(name)
        cap = int(1.2 * 140 * wl.n)
        ne_a, a = _outputs(T, wl, False, cap)
        ne_b, b = _outputs(T, wl, True, cap)
        assert ne_a == ne_b > 0
        for k in a:
            assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), (name, k)
        print("%s: %d pairs, static rebuild identical" % (name, ne_a), flush=True)


def test_static_rebuild_limit_and_errors(T):
    import torch
    dev = "cuda"
    n = (1 << 19) + 1
    pos = torch.zeros((n, 3), dtype=torch.float32, device=dev)
    sp = torch.zeros(n, dtype=torch.int32, device=dev)
    perm = torch.empty(n, dtype=torch.int32, device=dev)
    rp = torch.empty(n + 1, dtype=torch.int32, device=dev)
    col = torch.empty(16, dtype=torch.int32, device=dev)
    st, _ = T.build_neighbors_static([200.0] * 3, 5.75, 1.0, pos, sp, perm, rp, col, check=False)
    assert st == T.ERR_WORKSPACE
    st, _ = T.build_neighbors_static([10.0] * 3, 5.75, 1.0, pos[:10], sp[:10], perm[:10],
                                     rp[:11], col, check=False)
    assert st == T.ERR_BOX
    # a capacity shortfall reports the required count, as the workspace variant does
    wl = W.load("water648")
    ne_full, _ = _outputs(T, wl, True, 200000)
    p = torch.from_numpy(wl.pos.copy()).to(dev)
    s = torch.from_numpy(wl.species.copy()).to(dev)
    st, ne = T.build_neighbors_static(wl.box, wl.model.r_cut, wl.skin, p, s, perm[:wl.n],
                                      rp[:wl.n + 1], col, check=False)
    assert st == T.ERR_CAPACITY and ne == ne_full
