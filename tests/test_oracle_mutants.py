"""The oracle's pins must be able to fail: each test here copies the oracle's C source into a
temporary directory, plants one plausible mistake in that copy (CPU only; the repository's
oracle is untouched), builds it as a separate library and checks that at least one of the
named pins rejects it. A mistake that every pin accepts would mean the part it touches is
unpinned.

Mutants:
- l2_mshift: the gated l = 2 update reads (forward) and writes (adjoint) the m-components of
  m^2 cyclically shifted. Forward and backward stay consistent (finite differences pass);
  only rotation equivariance at l_max = 2 can reject it.
- softmax_adjoint_alpha: the envelope adjoint uses alpha = u p instead of p = exp(s - M)/Z.
- jacobian_sign: one entry of the l = 2 harmonic Jacobian has the wrong sign.
- shift_sign: the image shift enters the edge vector with the wrong sign.
"""
import importlib.util
import os
import shutil
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_DIR = os.path.join(os.path.dirname(HERE), "oracle")

MUTANTS = {
    "l2_mshift": [
        ("          for (int k = 0; k < C; k++) y += Lw->Wl[l][c * C + k] * mi[k * D + d];",
         "          int dsrc = (l == 2) ? l * l + (mm + 1) % (2 * l + 1) : d;\n"
         "          for (int k = 0; k < C; k++) y += Lw->Wl[l][c * C + k] * mi[k * D + dsrc];"),
        ("          mb[k * D + d] = s2;",
         "          mb[k * D + ((l == 2) ? l * l + (mm + 1) % (2 * l + 1) : d)] = s2;"),
    ],
    "softmax_adjoint_alpha": [("    ubar += p * diff;", "    ubar += alpha * diff;")],
    "jacobian_sign": [("    J[7][0] = s15 * z; J[7][2] = s15 * x;",
                       "    J[7][0] = -s15 * z; J[7][2] = s15 * x;")],
    "shift_sign": [
        ("  for (int a = 0; a < 3; a++) rv[a] = pos[3 * j + a] - pos[3 * i + a] + (double)s[a] * L[a];",
         "  for (int a = 0; a < 3; a++) rv[a] = pos[3 * j + a] - pos[3 * i + a] - (double)s[a] * L[a];"),
    ],
}


def _mutant_module(tmp_path_factory, name):
    d = tmp_path_factory.mktemp("oracle_" + name)
    pkg = d / ("oracle_" + name)
    shutil.copytree(ORACLE_DIR, pkg, ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    src = pkg / "tess_oracle.c"
    text = src.read_text()
    for old, new in MUTANTS[name]:
        assert text.count(old) == 1, "mutation site not found: " + old
        text = text.replace(old, new)
    src.write_text(text)
    spec = importlib.util.spec_from_file_location("oracle_" + name, pkg / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod
    spec.loader.exec_module(mod)
    mod.build(force=True)
    return mod


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def test_l2_mshift_rejected(tmp_path_factory):
    from tests import test_oracle_model as TM
    mod = _mutant_module(tmp_path_factory, "l2_mshift")
    # consistent forward/backward: the finite-difference pin cannot see it ...
    assert not _fails(TM.test_forces_finite_difference, mod, "salt4k")
    # ... the l_max = 2 rotation pins do
    assert _fails(TM.test_rotation_invariance_lmax2_cluster, mod, ("salt4k", 9.0, 2002))
    assert _fails(TM.test_cube_rotations_periodic_lmax2, mod)


@pytest.mark.parametrize("name", ["softmax_adjoint_alpha", "jacobian_sign"])
def test_gradient_mutants_rejected(tmp_path_factory, name):
    from tests import test_oracle_model as TM
    mod = _mutant_module(tmp_path_factory, name)
    assert _fails(TM.test_forces_finite_difference, mod, "salt4k")


def test_shift_sign_rejected(tmp_path_factory):
    from tests import test_oracle_model as TM
    mod = _mutant_module(tmp_path_factory, "shift_sign")
    assert _fails(TM.test_energy_translation_and_permutation_invariance, mod)
