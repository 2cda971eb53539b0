"""The c=256 decoder at 704x1248 (latents 44x78), in the launch configuration
the benchmark times (frames_per_pass=4 unless swept).

* Elementwise parity at full size: by causality the first 4k-3 video frames
  of any clip are the decode of its first k latent frames.  The oracle
  decodes the first two latent frames in full (5 video frames, 3 x 5 x 704 x
  1248 outputs: frame 0 plus the first four frames that pass through both
  time_convs and read real history in every temporal tap), and the GPU must
  match them within the tolerances in the 13- and 49-latent-frame decodes at
  frames_per_pass 4 and in a 2-latent-frame decode at frames_per_pass 1 (two
  passes, so the second reads every history ring at full size).  The same
  for the deep (110-tensor) variant.
* Properties that hold at any size, bit-exact on the device: identical video
  for frames_per_pass 2, 4, 8 and 16 on the 121-latent-frame clip, whose
  first 49 frames equal the 13-latent-frame decode (causal prefix), as do
  the first 49 frames of the 49-frame clip; the 13-frame clip streamed in
  chunks of 5 and 8 latent frames equal to its whole-clip decode; every
  element finite and in [-1, 1], and no fp16 store out of range.
"""
import numpy as np
import pytest

from tests.gpu_util import assert_range_clean, gpu_available, oracle_video, rel_l2
from video_diffusion_vae_amd import synth

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

MAX_ABS = 3e-2
REL_L2 = 1e-2
PREFIX_T = 2  # latent frames the oracle decodes in full: video frames 0..4


@pytest.fixture(scope="module")
def dec():
    import torch

    from video_diffusion_vae_amd import wvd
    cfg = synth.config_by_name("c256_T49_704x1248")
    W = synth.make_weights(cfg.c, seed=0)
    d = wvd.Decoder({k: torch.from_numpy(v).to(torch.bfloat16) for k, v in W.items()}, cfg.c, cfg.h, cfg.w)
    yield d
    d.release_workspace()
    torch.cuda.empty_cache()


def decode(dec, T, P):
    import torch
    z = torch.from_numpy(synth.make_latents(T, 44, 78, seed=0)).cuda().to(torch.bfloat16)
    out = dec.decode(z, frames_per_pass=P)
    torch.cuda.synchronize()
    assert_range_clean()
    return out


def check_range(out):
    import torch
    assert bool(torch.isfinite(out).all()) and float(out.abs().max()) <= 1.0


def check_prefix(out, ref, name):
    """The first frames of `out` against the oracle's prefix video `ref`,
    frame by frame and over the whole prefix."""
    nf = ref.shape[2]
    got = out[:, :, :nf].float().cpu().numpy()
    for f in range(nf):
        d = np.abs(got[:, :, f].astype(np.float64) - ref[:, :, f])
        print(f"{name} frame {f}: max_abs={d.max():.3e} rel_l2={rel_l2(got[:, :, f], ref[:, :, f]):.3e}", flush=True)
    d = np.abs(got.astype(np.float64) - ref)
    r = rel_l2(got, ref)
    print(f"{name} frames 0..{nf - 1}: max_abs={d.max():.3e} rel_l2={r:.3e}", flush=True)
    assert d.max() <= MAX_ABS and r <= REL_L2, (name, d.max(), r)


def test_prefix_matches_oracle(dec):
    ref = oracle_video(synth.config_by_name("c256_T13_704x1248"), seed=0, T=PREFIX_T)  # [1,3,5,704,1248]
    assert ref.shape == (1, 3, 5, 704, 1248)
    for T, P in ((13, 4), (49, 4), (PREFIX_T, 1)):
        print(f"case full-size prefix T={T} P={P}", flush=True)
        out = decode(dec, T, P)
        check_range(out)
        check_prefix(out, ref, f"T={T} P={P}")
        del out


def test_causal_prefix_bit_identical(dec):
    import torch
    print("case full-size causal prefix T=13 vs T=49", flush=True)
    short = decode(dec, 13, 4)
    full = decode(dec, 49, 4)
    assert full.shape[2] == 193 and short.shape[2] == 49
    assert torch.equal(full[:, :, :49], short)


def test_chunked_stream_bit_identical(dec):
    import torch
    print("case full-size T=13 streamed as chunks 5 + 8, P=4", flush=True)
    z = torch.from_numpy(synth.make_latents(13, 44, 78, seed=0)).cuda().to(torch.bfloat16)
    whole = dec.decode(z, frames_per_pass=4).clone()
    st = dec.stream()
    a = st.decode(z[:, :, :5], frames_per_pass=4)
    b = st.decode(z[:, :, 5:], frames_per_pass=4)
    torch.cuda.synchronize()
    assert_range_clean()
    assert a.shape[2] == 17 and b.shape[2] == 32
    assert torch.equal(torch.cat([a, b], dim=2), whole)
    del a, b, whole, st


def test_frames_per_pass_sweep_bit_identical(dec):
    """The 481-frame clip at frames_per_pass 2, 4, 8, 16: one video, whose
    first 49 frames are the 13-latent-frame decode (tied to the oracle by
    test_prefix_matches_oracle)."""
    import torch
    print("case full-size T=13 P=4 (prefix of the T=121 clip)", flush=True)
    short = decode(dec, 13, 4).cpu()
    print("case full-size T=121 P=4", flush=True)
    ref = decode(dec, 121, 4)
    check_range(ref)
    assert torch.equal(ref[:, :, :49].cpu(), short)
    del short
    for P in (2, 8, 16):
        print(f"case full-size T=121 P={P}", flush=True)
        dec.release_workspace()
        torch.cuda.empty_cache()
        out = decode(dec, 121, P)
        assert torch.equal(out, ref), f"P={P}"
        del out


def test_deep_variant_prefix_matches_oracle():
    """The 110-tensor decoder at full size: the first five video frames of a
    5-latent-frame decode (frames_per_pass 4, so a full and a partial pass)
    and of a 2-latent-frame decode at frames_per_pass 1, against the oracle's
    decode of the first two latent frames."""
    import torch

    from video_diffusion_vae_amd import wvd
    cfg = synth.config_by_name("deep_c256_T49_704x1248")
    ref = oracle_video(cfg, seed=0, T=PREFIX_T)
    W = synth.make_weights(cfg.c, seed=0, deep=True)
    d = wvd.Decoder({k: torch.from_numpy(v).to(torch.bfloat16) for k, v in W.items()}, cfg.c, cfg.h, cfg.w)
    for T, P in ((5, 4), (PREFIX_T, 1)):
        print(f"case deep full-size prefix T={T} P={P}", flush=True)
        out = decode(d, T, P)
        check_range(out)
        check_prefix(out, ref, f"deep T={T} P={P}")
        del out
    del d
    torch.cuda.empty_cache()
