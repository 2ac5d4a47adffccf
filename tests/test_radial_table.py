"""Accuracy of the tabulated radial weights (CPU, fp64).

The HIP path evaluates each layer's radial MLP w_p(r) = sum_h W2[p][h] SiLU(sum_k W1[h][k]
b_k(r)) exactly only at 1,025 knots on [0, r_c] and interpolates every edge with the cubic
Hermite polynomial through the two neighbouring knots' values and r-derivatives (the knot
spacing and the scheme are the library's; the basis b_k is the enveloped Bessel basis of the
model: u(r) sqrt(2/r_c) sin(k pi r/r_c)/r with u the cosine envelope). This test measures the
scheme's error against the MLP at random distances for the 4-layer, 64-hidden model with the
benchmark's weights, and checks the properties the forces rely on: the interpolant matches
the function and its derivative at the knots, and is C^1 across them."""
import numpy as np

from molecular_dynamics_hilbert_amd import workloads as W

NK = 1024  # intervals of the library's table


def _layers(spec, w):
    S, C, T, R, K = spec.n_species, spec.channels, spec.n_layers, spec.radial_hidden, 8
    P = 11 if spec.l_max == 2 else 4
    G = C * (1 + spec.l_max)
    off = S * C
    out = []
    for _ in range(T):
        off += 2 * C * C
        W1 = w[off:off + R * K].reshape(R, K).astype(np.float64)
        off += R * K
        W2 = w[off:off + P * R].reshape(P, R).astype(np.float64)
        off += P * R + G * C + spec.l_max * C * C
        out.append((W1, W2))
    return out


def _mlp(r, W1, W2, rc):
    r = np.asarray(r, np.float64)[:, None]
    k = np.arange(1, 9)[None, :]
    a = k * np.pi / rc
    u = 0.5 * (np.cos(np.pi * r / rc) + 1.0)
    du = -0.5 * np.pi / rc * np.sin(np.pi * r / rc)
    pref = np.sqrt(2.0 / rc)
    with np.errstate(invalid="ignore", divide="ignore"):
        B = np.where(r > 0, pref * np.sin(a * r) / r, pref * a)
        dB = np.where(r > 0, pref * (a * np.cos(a * r) / r - np.sin(a * r) / r ** 2), 0.0)
    b, db = u * B, du * B + u * dB
    z, dz = b @ W1.T, db @ W1.T
    sg = 1.0 / (1.0 + np.exp(-z))
    return (z * sg) @ W2.T, (sg * (1.0 + z * (1.0 - sg)) * dz) @ W2.T


def _hermite(r, wk, dwk, h):
    x = r / h
    i = np.minimum(np.floor(x).astype(int), NK - 1)
    t = (x - i)[:, None]
    h00, h10 = 2 * t ** 3 - 3 * t ** 2 + 1, (t ** 3 - 2 * t ** 2 + t) * h
    h01, h11 = 3 * t ** 2 - 2 * t ** 3, (t ** 3 - t ** 2) * h
    d00, d10 = 6 * (t ** 2 - t) / h, 3 * t ** 2 - 4 * t + 1
    d11 = 3 * t ** 2 - 2 * t
    w = h00 * wk[i] + h10 * dwk[i] + h01 * wk[i + 1] + h11 * dwk[i + 1]
    dw = d00 * wk[i] + d10 * dwk[i] - d00 * wk[i + 1] + d11 * dwk[i + 1]
    return w, dw


def test_interpolation_error_below_fp32_rounding():
    spec = W.big_model()
    w = W.make_weights(spec, 2003)
    rc = float(spec.r_cut)
    h = rc / NK
    knots = np.arange(NK + 1) * h
    rs = np.random.default_rng(7).uniform(0.05, rc * (1 - 1e-7), 100000)
    for W1, W2 in _layers(spec, w):
        wk, dwk = _mlp(knots, W1, W2, rc)
        wi, dwi = _hermite(rs, wk, dwk, h)
        we, dwe = _mlp(rs, W1, W2, rc)
        assert np.abs(wi - we).max() <= 1e-9 * np.abs(we).max()
        assert np.abs(dwi - dwe).max() <= 3e-7 * np.abs(dwe).max()


def test_interpolant_is_c1_at_the_knots():
    spec = W.big_model()
    w = W.make_weights(spec, 2003)
    rc = float(spec.r_cut)
    h = rc / NK
    knots = np.arange(NK + 1) * h
    W1, W2 = _layers(spec, w)[0]
    wk, dwk = _mlp(knots, W1, W2, rc)
    # at a knot from the interval on its right (t = 0) and on its left (t -> 1)
    inner = knots[1:-1]
    wl, dwl = _hermite(inner - 1e-12, wk, dwk, h)
    wr, dwr = _hermite(inner, wk, dwk, h)
    assert np.allclose(wr, wk[1:-1], rtol=0, atol=1e-12 * np.abs(wk).max())
    assert np.allclose(dwr, dwk[1:-1], rtol=0, atol=1e-9 * np.abs(dwk).max())
    assert np.abs(wl - wr).max() <= 1e-9 * np.abs(wk).max()
    assert np.abs(dwl - dwr).max() <= 1e-6 * np.abs(dwk).max()
    # w and dw/dr vanish at r_c (envelope), so the table ends smoothly at the cutoff
    assert np.abs(wk[-1]).max() <= 1e-12 * np.abs(wk).max()


def _midpoint_deviation(W1, W2, rc):
    """The library's table guard in numpy: fp32-stored knots, Hermite at the interval
    midpoints (fp64) against the MLP; deviations relative to the midpoints' max |w|, |dw/dr|."""
    h = rc / NK
    knots = np.arange(NK + 1) * h
    mids = (np.arange(NK) + 0.5) * h
    wk, dwk = _mlp(knots, W1, W2, rc)
    wk, dwk = wk.astype(np.float32).astype(np.float64), dwk.astype(np.float32).astype(np.float64)
    wi, dwi = _hermite(mids, wk, dwk, h)
    we, dwe = _mlp(mids, W1, W2, rc)
    return np.abs(wi - we).max() / np.abs(we).max(), np.abs(dwi - dwe).max() / np.abs(dwe).max()


def test_table_guard_thresholds():
    """The guard flags a layer whose midpoint deviation exceeds 1e-6 of max|w| or 1e-4 of
    max|dw/dr|. The benchmark's weights, and the same with W1 scaled by 4 (sharper radial
    functions; the GPU parity test uses them), stay inside (the stored fp32 knots dominate:
    about 5e-8 and 1e-5); W1 scaled by 32 is flagged."""
    spec = W.big_model()
    w = W.make_weights(spec, 2003)
    rc = float(spec.r_cut)
    for scale, inside in ((1.0, True), (4.0, True), (32.0, False)):
        dev = [_midpoint_deviation(W1 * scale, W2, rc) for W1, W2 in _layers(spec, w)]
        ok = all(a <= 1e-6 and b <= 1e-4 for a, b in dev)
        assert ok == inside, (scale, dev)
