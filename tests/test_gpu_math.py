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
