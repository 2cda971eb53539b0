"""The Winograd F(m,3) algebra the GPU path uses for its 3x3x3 convs (m = 6;
m = 2 and m = 4 are kept as options), restated on the host and checked
against direct correlation (CPU only).

Along x, with zero padding of one column on each side, output columns 2p and
2p+1 of a 3-tap correlation with taps g = (g0, g1, g2) use the inputs
d_k = x[2p-1+k], k = 0..3.  The GPU path stores
  U = (d0 - d2, d1 + d2, d2 - d1, d1 - d3)          (input transform)
  V = (g0, (g0+g1+g2)/2, (g0-g1+g2)/2, g2)          (weight transform)
multiplies them per xi (summed over channels and the (t, y) taps), and
recovers
  y[2p] = M0 + M1 + M2,  y[2p+1] = M1 - M2 - M3      (output transform).
These are the minimal-filtering identities for interpolation points
0, 1, -1 and infinity.  F(4,3) uses 0, 1, -1, 2, -2, infinity: six inputs
d_k = x[4q-1+k] give four outputs x[4q..4q+3] through
  U = (4d0-5d2+d4, -4d1-4d2+d3+d4, 4d1-4d2-d3+d4, -2d1-d2+2d3+d4,
       2d1-d2-2d3+d4, 4d1-5d3+d5)
  V = (g0/4, -(g0+g1+g2)/6, -(g0-g1+g2)/6, g0/24+g1/12+g2/6, g0/24-g1/12+g2/6, g2)
  y = (M0+M1+M2+M3+M4, M1-M2+2M3-2M4, M1+M2+4M3+4M4, M1-M2+8M3-8M4+M5).
F(6,3) uses 0, 1, -1, 1/2, -1/2, 2, -2, infinity: eight inputs d_k =
x[6q-1+k] give six outputs x[6q..6q+5].  With the rows of G scaled to the
taps' magnitude (factors 2/9, 32/45 and 2/45 moved into the output
transform):
  U = (d0-d6+21/4(d4-d2), t1+t2, t1-t2, t3+t4, t3-t4, t5+t6, t5-t6, d7-d1+21/4(d3-d5))
      t1 = d2+d6-17/4 d4, t2 = d1+d5-17/4 d3, t3 = 4d2+d6-5d4, t4 = 2d1-5/2 d3+1/2 d5,
      t5 = d2/4+d6-5/4 d4, t6 = d1/2-5/2 d3+2d5
  V = (g0, -(g0+g1+g2), -(g0-g1+g2), g0+g1/2+g2/4, g0-g1/2+g2/4, g0/4+g1/2+g2, g0/4-g1/2+g2, g2)
  with a = 2/9 (M1+M2), b = 2/9 (M1-M2), c = (M3+M4)/45, d = (M3-M4)/45,
  e = (M5+M6)/45, f = (M5-M6)/45:
  y = (M0+a+32c+2e, b+16d+4f, a+8c+8e, b+4d+16f, a+2c+32e, b+d+64f+M7).
"""
import numpy as np
import pytest


def wino_1d(x, g):
    W = x.shape[-1]
    W2 = (W + 1) // 2
    xp = np.zeros(x.shape[:-1] + (2 * W2 + 2,), x.dtype)
    xp[..., 1:W + 1] = x
    d = [xp[..., k:k + 2 * W2:2] for k in range(4)]  # d_k[p] = x[2p-1+k]
    U = [d[0] - d[2], d[1] + d[2], d[2] - d[1], d[1] - d[3]]
    g0, g1, g2 = g
    V = [g0, (g0 + g1 + g2) / 2, (g0 - g1 + g2) / 2, g2]
    M = [u * v for u, v in zip(U, V)]
    y = np.empty(x.shape[:-1] + (2 * W2,), x.dtype)
    y[..., 0::2] = M[0] + M[1] + M[2]
    y[..., 1::2] = M[1] - M[2] - M[3]
    return y[..., :W]


def wino4_1d(x, g):
    W = x.shape[-1]
    WQ = (W + 3) // 4
    xp = np.zeros(x.shape[:-1] + (4 * WQ + 2,), x.dtype)
    xp[..., 1:W + 1] = x
    d = [xp[..., k:k + 4 * WQ:4] for k in range(6)]  # d_k[q] = x[4q-1+k]
    U = [4 * d[0] - 5 * d[2] + d[4], -4 * d[1] - 4 * d[2] + d[3] + d[4], 4 * d[1] - 4 * d[2] - d[3] + d[4],
         -2 * d[1] - d[2] + 2 * d[3] + d[4], 2 * d[1] - d[2] - 2 * d[3] + d[4], 4 * d[1] - 5 * d[3] + d[5]]
    g0, g1, g2 = g
    V = [g0 / 4, -(g0 + g1 + g2) / 6, -(g0 - g1 + g2) / 6, g0 / 24 + g1 / 12 + g2 / 6,
         g0 / 24 - g1 / 12 + g2 / 6, g2]
    M = [u * v for u, v in zip(U, V)]
    y = np.empty(x.shape[:-1] + (4 * WQ,), x.dtype)
    y[..., 0::4] = M[0] + M[1] + M[2] + M[3] + M[4]
    y[..., 1::4] = M[1] - M[2] + 2 * M[3] - 2 * M[4]
    y[..., 2::4] = M[1] + M[2] + 4 * M[3] + 4 * M[4]
    y[..., 3::4] = M[1] - M[2] + 8 * M[3] - 8 * M[4] + M[5]
    return y[..., :W]


def wino6_1d(x, g):
    W = x.shape[-1]
    WQ = (W + 5) // 6
    xp = np.zeros(x.shape[:-1] + (6 * WQ + 2,), x.dtype)
    xp[..., 1:W + 1] = x
    d = [xp[..., k:k + 6 * WQ:6] for k in range(8)]  # d_k[q] = x[6q-1+k]
    t1, t2 = d[2] + d[6] - 4.25 * d[4], d[1] + d[5] - 4.25 * d[3]
    t3, t4 = 4 * d[2] + d[6] - 5 * d[4], 2 * d[1] - 2.5 * d[3] + 0.5 * d[5]
    t5, t6 = 0.25 * d[2] + d[6] - 1.25 * d[4], 0.5 * d[1] - 2.5 * d[3] + 2 * d[5]
    U = [d[0] - d[6] + 5.25 * (d[4] - d[2]), t1 + t2, t1 - t2, t3 + t4, t3 - t4, t5 + t6, t5 - t6,
         d[7] - d[1] + 5.25 * (d[3] - d[5])]
    g0, g1, g2 = g
    V = [g0, -(g0 + g1 + g2), -(g0 - g1 + g2), g0 + g1 / 2 + g2 / 4, g0 - g1 / 2 + g2 / 4,
         g0 / 4 + g1 / 2 + g2, g0 / 4 - g1 / 2 + g2, g2]
    M = [u * v for u, v in zip(U, V)]
    a, b = 2 / 9 * (M[1] + M[2]), 2 / 9 * (M[1] - M[2])
    c, dd = (M[3] + M[4]) / 45, (M[3] - M[4]) / 45
    e, f = (M[5] + M[6]) / 45, (M[5] - M[6]) / 45
    y = np.empty(x.shape[:-1] + (6 * WQ,), x.dtype)
    y[..., 0::6] = M[0] + a + 32 * c + 2 * e
    y[..., 1::6] = b + 16 * dd + 4 * f
    y[..., 2::6] = a + 8 * c + 8 * e
    y[..., 3::6] = b + 4 * dd + 16 * f
    y[..., 4::6] = a + 2 * c + 32 * e
    y[..., 5::6] = b + dd + 64 * f + M[7]
    return y[..., :W]


def direct_1d(x, g):
    W = x.shape[-1]
    xp = np.pad(x, [(0, 0)] * (x.ndim - 1) + [(1, 1)])
    return sum(g[k] * xp[..., k:k + W] for k in range(3))


@pytest.mark.parametrize("W", [1, 2, 3, 7, 16, 39, 78])
def test_f23_equals_direct_correlation(W):
    rng = np.random.default_rng(W)
    x = rng.standard_normal((5, W))
    g = rng.standard_normal(3)
    np.testing.assert_allclose(wino_1d(x, g), direct_1d(x, g), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 7, 16, 39, 78, 624])
def test_f43_equals_direct_correlation(W):
    rng = np.random.default_rng(100 + W)
    x = rng.standard_normal((5, W))
    g = rng.standard_normal(3)
    np.testing.assert_allclose(wino4_1d(x, g), direct_1d(x, g), rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("W", [1, 2, 3, 5, 6, 7, 12, 13, 39, 78, 624])
def test_f63_equals_direct_correlation(W):
    rng = np.random.default_rng(200 + W)
    x = rng.standard_normal((5, W))
    g = rng.standard_normal(3)
    np.testing.assert_allclose(wino6_1d(x, g), direct_1d(x, g), rtol=1e-10, atol=1e-10)


def test_f63_each_output_picks_its_own_window():
    # unit impulses: output column j of a group sees exactly x[j-1..j+1]
    for W in (6, 12):
        for j in range(W):
            x = np.zeros(W)
            x[j] = 1.0
            for k in range(3):
                g = np.zeros(3)
                g[k] = 1.0
                np.testing.assert_allclose(wino6_1d(x, g), direct_1d(x, g), atol=1e-12)


def test_wino_with_channel_contraction_and_other_taps():
    # A full 3x3x3 conv = sum over (dt, dy) of x-correlations; the transform
    # commutes with the channel contraction and with the (t, y) tap sum.
    rng = np.random.default_rng(7)
    Cin, Cout, T, H, W = 3, 2, 4, 3, 10
    x = rng.standard_normal((Cin, T, H, W))
    w = rng.standard_normal((Cout, Cin, 3, 3, 3))
    xp = np.pad(x, [(0, 0), (2, 0), (1, 1), (0, 0)])  # causal in t, pad 1 in y
    ref = np.zeros((Cout, T, H, W))
    win = np.zeros((Cout, T, H, W))
    for o in range(Cout):
        for i in range(Cin):
            for dt in range(3):
                for dy in range(3):
                    rows = xp[i, dt:dt + T, dy:dy + H, :]
                    ref[o] += direct_1d(rows, w[o, i, dt, dy])
                    win[o] += wino6_1d(rows, w[o, i, dt, dy])
    np.testing.assert_allclose(win, ref, rtol=1e-11, atol=1e-11)
