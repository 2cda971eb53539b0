"""Numeric edge cases of the GPU decoder, through the C ABI.

* Clamp edge: the head's bias pushed to +-1 (and +-1.25, +-0.75), so that a
  large share of the pre-clamp values lie beyond [-1, 1] and many sit right
  at the edge; the clamped video must still match the oracle (the
  Wan2.2 page, "Correctness", requires every output in [-1, 1]).
* Out-of-range values are visible: latents far beyond the fp16 range
  saturate the first stored activations, and the device range flags say so;
  a NaN in one latent frame reaches the video as NaN (the final clamp does
  not turn it into a number), only in the video frames that latent frame
  feeds (causality), and the flags record it.
"""
import numpy as np
import pytest

from tests.gpu_util import assert_range_clean, gpu_available, rel_l2
from video_diffusion_vae_amd import synth

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

MAX_ABS = 3e-2
REL_L2 = 1e-2


def clamp_edge_weights(cfg):
    """The config's weights with the head bias moved to the clamp's edges:
    +-1 (half of each channel's values then lie beyond [-1, 1]), +-1.25
    (mostly clamped) and +-0.75 (mostly not), alternating in sign over the 12
    channels (all exact in bf16)."""
    W = synth.make_weights(cfg.c, seed=0, bf16=cfg.weights_bf16)
    mag = np.array([1.0, 1.0, 1.25, 0.75] * 3, np.float32)
    sign = np.where(np.arange(12) % 2 == 0, 1.0, -1.0).astype(np.float32)
    W["head.conv.bias"] = (mag * sign).astype(np.float32)
    return W


@pytest.mark.parametrize("cfg_name", ["tiny_c16_T2_4x6", "c64_T3_352x624"])
def test_clamp_edge_matches_oracle(cfg_name):
    import torch

    from oracle import decoder as O
    from video_diffusion_vae_amd import wvd
    cfg = synth.config_by_name(cfg_name)
    W = clamp_edge_weights(cfg)
    z = synth.make_latents(cfg.T, cfg.h, cfg.w, seed=0, bf16=cfg.weights_bf16)
    ref = O.decode(z, W, cfg.c)
    clamped = float(np.mean(np.abs(ref) == 1.0))
    print(f"{cfg_name}: share of oracle outputs at +-1: {clamped:.3f}", flush=True)
    assert 0.1 < clamped < 0.9  # the clamp engages, and not everywhere
    dt = torch.bfloat16 if cfg.weights_bf16 else torch.float32
    dec = wvd.Decoder({k: torch.from_numpy(v).to(dt) for k, v in W.items()}, cfg.c, cfg.h, cfg.w)
    zt = torch.from_numpy(z).cuda().to(dt)
    for P in sorted(set(cfg.passes)):
        print(f"case clamp edge {cfg_name} P={P}", flush=True)
        got = dec.decode(zt, frames_per_pass=P).float().cpu().numpy()
        assert_range_clean()
        assert np.isfinite(got).all() and np.abs(got).max() <= 1.0
        d = np.abs(got.astype(np.float64) - ref)
        r = rel_l2(got, ref)
        print(f"clamp edge {cfg_name} P={P}: max_abs={d.max():.3e} rel_l2={r:.3e}", flush=True)
        assert d.max() <= MAX_ABS and r <= REL_L2
        # where the oracle is clamped well past the edge, so is the GPU, exactly
        far = np.abs(ref) == 1.0
        assert np.mean(np.abs(got[far]) == 1.0) > 0.95


def _tiny_decoder():
    import torch

    from video_diffusion_vae_amd import wvd
    cfg = synth.config_by_name("tiny_c16_T2_4x6")
    W = synth.make_weights(cfg.c, seed=0, bf16=False)
    dec = wvd.Decoder({k: torch.from_numpy(v) for k, v in W.items()}, cfg.c, cfg.h, cfg.w)
    return cfg, dec


def test_saturation_is_flagged():
    import torch

    from video_diffusion_vae_amd import wvd
    cfg, dec = _tiny_decoder()
    assert_range_clean()
    z = synth.make_latents(cfg.T, cfg.h, cfg.w, seed=0, bf16=False) * np.float32(1e6)
    print("case tiny c16 latents x 1e6", flush=True)
    out = dec.decode(torch.from_numpy(z).cuda(), frames_per_pass=1)
    torch.cuda.synchronize()
    flags = wvd.range_flags(clear=True)
    assert flags & wvd.WVD_RANGE_SATURATED, flags
    assert not flags & wvd.WVD_RANGE_NAN, flags
    v = out.float()
    assert bool(torch.isfinite(v).all()) and float(v.abs().max()) <= 1.0


def test_nan_reaches_the_video_and_is_flagged():
    import torch

    from video_diffusion_vae_amd import wvd
    cfg, dec = _tiny_decoder()
    assert_range_clean()
    z = synth.make_latents(cfg.T, cfg.h, cfg.w, seed=0, bf16=False)
    z[0, 5, 1, 2, 3] = np.nan  # one value of latent frame 1
    for P in (1, 2):
        print(f"case tiny c16 NaN latent P={P}", flush=True)
        out = dec.decode(torch.from_numpy(z).cuda(), frames_per_pass=P).float().cpu().numpy()
        flags = wvd.range_flags(clear=True)
        assert flags & wvd.WVD_RANGE_NAN, flags
        assert np.isfinite(out[:, :, 0]).all()        # video frame 0 reads latent frame 0 only
        assert np.isnan(out[:, :, 1:]).any()          # frames 1..4 read latent frame 1
    assert_range_clean()
