"""Error bound of the device SiLU and exponential (the hardware exp2 of
t * log2(e) and the hardware reciprocal, which every norm-SiLU prologue and
the attention softmax use), against float64 references, through
wvd_math_probe.  The norm-SiLU issue ("Prototype evidence and limits") asks
that such fast exp / sqrt lowering be reviewed.

Bounds (relative error, t the input):
  SiLU, |t| <= 40:        |err| <= 4 * 2^-24 + |t| * 2^-23   (<= 4.8e-6 at |t| = 40)
  exp,  -87 <= t <= 0:    |err| <= 4 * 2^-24 + |t| * 2^-23   (<= 1.1e-5 at t = -87)
The |t| term is the rounding of t * log2(e) before the exp2; both bounds sit
far below the fp16 rounding (2^-11 relative) of every value the decoder
stores.  Inputs: SiLU's range covers the normalised activations (|x / ||x||
* sqrt(C) * gamma| stays well below 40), exp's the softmax's max-subtracted
logits down to where e^t leaves the normal fp32 range.
"""
import numpy as np
import pytest

from tests.gpu_util import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

EPS = 2.0 ** -24


def probe(x: np.ndarray):
    import torch

    from video_diffusion_vae_amd import wvd
    xt = torch.from_numpy(x.astype(np.float32)).cuda()
    s = torch.empty_like(xt)
    e = torch.empty_like(xt)
    wvd.wvd_math_probe(xt.data_ptr(), s.data_ptr(), e.data_ptr(), xt.numel(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return s.cpu().numpy().astype(np.float64), e.cpu().numpy().astype(np.float64)


def grid(lo, hi, n, seed):
    rng = np.random.default_rng(seed)
    x = np.concatenate([np.linspace(lo, hi, n), rng.uniform(lo, hi, n)]).astype(np.float32)
    return x


def test_silu_error_bound():
    x = grid(-40.0, 40.0, 1 << 20, 1)
    x = np.concatenate([x, np.float32([0.0, -0.0, 1e-30, -1e-30, 1e-6, -1e-6, 40.0, -40.0])])
    s, _ = probe(x)
    t = x.astype(np.float64)
    ref = t / (1.0 + np.exp(-t))
    rel = np.abs(s - ref) / np.maximum(np.abs(ref), 1e-300)
    bound = 4 * EPS + np.abs(t) * 2 * EPS
    worst = np.argmax(rel / bound)
    print(f"SiLU: max rel err {rel.max():.3e}; worst vs bound {rel[worst]:.3e} / {bound[worst]:.3e} at t={t[worst]}")
    assert (rel <= bound).all()
    assert s[np.float32(x) == 0].tolist() == [0.0, 0.0]


def test_exp_error_bound():
    x = grid(-87.0, 0.0, 1 << 20, 2)
    _, e = probe(x)
    t = x.astype(np.float64)
    ref = np.exp(t)
    rel = np.abs(e - ref) / ref
    bound = 4 * EPS + np.abs(t) * 2 * EPS
    worst = np.argmax(rel / bound)
    print(f"exp: max rel err {rel.max():.3e}; worst vs bound {rel[worst]:.3e} / {bound[worst]:.3e} at t={t[worst]}")
    assert (rel <= bound).all()


def test_nan_passes_through():
    s, e = probe(np.float32([np.nan, np.inf, -np.inf]))
    assert np.isnan(s[0]) and np.isnan(e[0])
    assert s[1] == np.inf and e[1] == np.inf and e[2] == 0.0


# ---- the fp16 packing and the norm scale (wvd_f16_probe) ----------------

F16_MAX = 0x7BFF  # 65504


def f16_probe(x: np.ndarray):
    import torch

    from video_diffusion_vae_amd import wvd
    x = np.concatenate([x.astype(np.float32), np.zeros((-x.size) % 8, np.float32)])
    xt = torch.from_numpy(x).cuda()
    h = torch.empty(x.size, dtype=torch.int16, device="cuda")
    rs = torch.empty_like(xt)
    wvd.range_flags(clear=True)
    wvd.wvd_f16_probe(xt.data_ptr(), h.data_ptr(), rs.data_ptr(), x.size, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    flags = wvd.range_flags(clear=True)
    return x, h.cpu().numpy().view(np.uint16), rs.cpu().numpy(), flags


def test_f16_packing_is_round_to_nearest_even():
    """Every fp16 value the kernels store goes through this packing: it must
    equal IEEE round-to-nearest-even (numpy's float32 -> float16) bit for bit
    over the whole finite range, ties and subnormals included."""
    rng = np.random.default_rng(3)
    mag = np.exp2(rng.uniform(-27.0, 15.999, 1 << 20))
    x = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    # exact midpoints between neighbouring fp16 values (normal and subnormal)
    b = rng.integers(0, 0x7BFF, 1 << 18, dtype=np.uint16)
    lo = b.view(np.float16).astype(np.float32)
    hi = (b + 1).view(np.float16).astype(np.float32)
    mid = ((lo.astype(np.float64) + hi.astype(np.float64)) / 2).astype(np.float32)
    assert np.all(mid.astype(np.float64) == (lo.astype(np.float64) + hi.astype(np.float64)) / 2)
    edges = np.float32([0.0, -0.0, 65504.0, -65504.0, 6.1035156e-05, 5.9604645e-08, 2.9802322e-08,
                        2.9802326e-08, 1.0, -1.0, 0.33333334])
    x = np.concatenate([x, mid, -mid, edges])
    x, h, _, flags = f16_probe(x)
    ref = x.astype(np.float16).view(np.uint16)
    bad = np.flatnonzero(h != ref)
    assert bad.size == 0, [(float(x[i]), hex(h[i]), hex(ref[i])) for i in bad[:8]]
    assert flags == 0


def test_f16_packing_saturates_and_keeps_nan():
    from video_diffusion_vae_amd import wvd
    sat = np.float32([65504.004, 65519.996, 65520.0, 1e6, np.inf, -65505.0, -1e30, -np.inf])
    mixed = np.float32([1e6, 1.5, 1.5, 1.5, 1.5, 1.5, 1.5, -3.0])
    x, h, _, flags = f16_probe(np.concatenate([sat, mixed]))
    assert h[:8].tolist() == [F16_MAX] * 5 + [F16_MAX | 0x8000] * 3
    # the in-range values of a group that takes the rare path keep their value
    assert h[8:16].tolist() == [F16_MAX] + [0x3E00] * 6 + [0xC200]
    assert flags == wvd.WVD_RANGE_SATURATED
    x, h, _, flags = f16_probe(np.float32([np.nan, 2.0, -np.nan, 0.5]))
    assert (h[0] & 0x7C00) == 0x7C00 and (h[0] & 0x3FF) != 0
    assert (h[2] & 0x7C00) == 0x7C00 and (h[2] & 0x3FF) != 0
    assert h[1] == 0x4000 and h[3] == 0x3800
    assert flags == wvd.WVD_RANGE_NAN


def test_norm_scale_error_bound():
    """The Winograd input transforms' 1 / max(||v||, 1e-12) from the channel
    sum of squares: one hardware rsqrt, within 2^-22 relative of the exact
    value over every sum a column of fp16 values can give (0, and 2^-48 up to
    1024 channels of 65504^2)."""
    rng = np.random.default_rng(4)
    ss = np.exp2(rng.uniform(-48.0, 42.0, 1 << 20)).astype(np.float32)
    ss = np.concatenate([ss, np.float32([0.0, 1e-30, 1e-24, 1.0, 4.0, 2.0 ** 42])])
    ss, _, rs, _ = f16_probe(ss)
    ref = 1.0 / np.maximum(np.sqrt(ss.astype(np.float64)), 1e-12)
    rel = np.abs(rs.astype(np.float64) - ref) / ref
    print(f"norm scale: max rel err {rel.max():.3e}")
    assert rel.max() <= 2.0 ** -22
