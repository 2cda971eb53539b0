"""The space-to-depth form of the encoder's 3x3 stride-2 down-conv (pad 1),
restated on the host and checked against direct strided correlation (CPU
only).

The input's four phase images P[py][px][Y][X] = x[2Y+py][2X+px] sit side by
side in channels (block b = 2 py + px).  Output (Y, X) of the strided conv
reads input rows 2Y-1, 2Y, 2Y+1, i.e. phase row 1 of Y-1 (kernel tap 0),
phase row 0 of Y (tap 1) and phase row 1 of Y (tap 2); the same along
columns.  So the strided conv is a 2x2 conv at offsets (a - 1, b - 1),
a, b in {0, 1}, over the 4C-channel phase tensor, with weight block
W'[a][b][block (py, px)] = w[ky][kx], where
  ky = (py == 1 ? 0 : none) for a = 0, (py == 0 ? 1 : 2) for a = 1,
and kx likewise: nine of the sixteen (tap, block) pairs carry a kernel tap,
the other seven are zero.  The down-conv's weight preparation builds exactly
these blocks and the phase-tap kernel runs the 2x2 conv.
"""
import numpy as np
import pytest


def strided_conv(x, w):
    """Direct 3x3 stride-2 correlation, zero pad 1: x [H][W][C], w [O][C][3][3]."""
    H, W, C = x.shape
    xp = np.zeros((H + 2, W + 2, C))
    xp[1:-1, 1:-1] = x
    out = np.zeros((H // 2, W // 2, w.shape[0]))
    for Y in range(H // 2):
        for X in range(W // 2):
            patch = xp[2 * Y:2 * Y + 3, 2 * X:2 * X + 3]  # rows 2Y-1..2Y+1 of x
            out[Y, X] = np.einsum("ijc,ocij->o", patch, w)
    return out


def s2d_weights(w):
    """W'[a][b] as [O][4C]: the tap mapping stated in the module docstring."""
    O, C = w.shape[:2]
    Wp = np.zeros((2, 2, O, 4 * C))
    for a in range(2):
        for b in range(2):
            for py in range(2):
                for px in range(2):
                    ky = (0 if py == 1 else None) if a == 0 else (1 if py == 0 else 2)
                    kx = (0 if px == 1 else None) if b == 0 else (1 if px == 0 else 2)
                    if ky is None or kx is None:
                        continue
                    blk = 2 * py + px
                    Wp[a, b, :, blk * C:(blk + 1) * C] = w[:, :, ky, kx]
    return Wp


def s2d_conv(x, w):
    H, W, C = x.shape
    P = np.concatenate([x[py::2, px::2] for py in range(2) for px in range(2)], axis=-1)  # [H/2][W/2][4C]
    Pp = np.zeros((H // 2 + 1, W // 2 + 1, 4 * C))
    Pp[1:, 1:] = P  # offsets -1 reach one row / column of zeros
    Wp = s2d_weights(w)
    out = np.zeros((H // 2, W // 2, w.shape[0]))
    for a in range(2):
        for b in range(2):
            out += np.einsum("yxk,ok->yxo", Pp[a:a + H // 2, b:b + W // 2], Wp[a, b])
    return out


@pytest.mark.parametrize("H,W,C,O", [(4, 6, 3, 5), (8, 8, 2, 2), (6, 10, 4, 7)])
def test_space_to_depth_equals_strided_conv(H, W, C, O):
    rng = np.random.default_rng(H * 100 + W * 10 + C)
    x = rng.standard_normal((H, W, C))
    w = rng.standard_normal((O, C, 3, 3))
    ref = strided_conv(x, w)
    got = s2d_conv(x, w)
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_nine_of_sixteen_blocks_carry_a_tap():
    w = np.arange(1, 10, dtype=float).reshape(1, 1, 3, 3)
    Wp = s2d_weights(w)
    nonzero = sorted(int(v) for v in Wp.reshape(-1) if v != 0)
    assert nonzero == list(range(1, 10))  # every kernel tap exactly once
    assert np.count_nonzero(Wp) == 9


def test_mapping_breaks_if_a_tap_is_misplaced():
    """A plausible slip (offset 0 reading tap 0 of the odd phase) is caught."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((6, 6, 2))
    w = rng.standard_normal((3, 2, 3, 3))
    ref = strided_conv(x, w)
    Wp = s2d_weights(w)
    bad = Wp.copy()
    C = 2
    bad[1, 1, :, 3 * C:4 * C] = w[:, :, 0, 0]  # block (1, 1) at offset (0, 0) should be tap (2, 2)
    H, W = 6, 6
    P = np.concatenate([x[py::2, px::2] for py in range(2) for px in range(2)], axis=-1)
    Pp = np.zeros((H // 2 + 1, W // 2 + 1, 4 * C))
    Pp[1:, 1:] = P
    out = np.zeros_like(ref)
    for a in range(2):
        for b in range(2):
            out += np.einsum("yxk,ok->yxo", Pp[a:a + H // 2, b:b + W // 2], bad[a, b])
    assert np.abs(out - ref).max() > 1e-3
