"""GPU encoder (the decoder's mirror image) against the CPU encoder oracle,
through the C ABI (wvd_encoder_prepare / wvd_encode).

Tolerances on the fp32 latents, as for the decoder's video: max |gpu -
oracle| <= 3e-2 and rel-L2 <= 1e-2 (fp16 storage of every stored activation,
fp32 accumulation; the latents' RMS is about 0.2-0.3).  The GPU latents must
be bit-identical across frames_per_pass and across causal prefixes (the
first k latent frames of a clip equal the encode of its first 4k-3 video
frames).  At 704x1248 the oracle encodes the first five video frames (two
latent frames) in full.
"""
import hashlib
import os

import numpy as np
import pytest

from tests.gpu_util import CACHE, ROOT, assert_range_clean, gpu_available, rel_l2
from video_diffusion_vae_amd import synth_encoder as SE

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

MAX_ABS = 3e-2
REL_L2 = 1e-2


def _src_hash() -> str:
    h = hashlib.sha256()
    for p in ("oracle/decoder.py", "oracle/encoder.py", "video_diffusion_vae_amd/synth.py",
              "video_diffusion_vae_amd/synth_encoder.py"):
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def oracle_latents(cfg, T: int) -> np.ndarray:
    """The oracle's latents of the first 4T-3 video frames (cached on disk)."""
    from oracle import encoder as OE
    path = os.path.join(CACHE, f"{cfg.name}_T{T}_{_src_hash()}.npy")
    if os.path.exists(path):
        return np.load(path)
    W = SE.make_encoder_weights(cfg.c, seed=0, bf16=cfg.weights_bf16)
    v = SE.make_video(T, cfg.h, cfg.w, seed=0, bf16=cfg.weights_bf16)
    z = OE.encode(v, W, cfg.c)
    os.makedirs(CACHE, exist_ok=True)
    np.save(path + ".tmp.npy", z)
    os.replace(path + ".tmp.npy", path)
    return z


_encoders = {}


def encoder_for(cfg):
    import torch

    from video_diffusion_vae_amd import wvd
    key = (cfg.c, cfg.h, cfg.w, cfg.weights_bf16)
    if key not in _encoders:
        _encoders.clear()
        W = SE.make_encoder_weights(cfg.c, seed=0, bf16=cfg.weights_bf16)
        dt = torch.bfloat16 if cfg.weights_bf16 else torch.float32
        _encoders[key] = wvd.Encoder({k: torch.from_numpy(v).to(dt) for k, v in W.items()}, cfg.c, cfg.h, cfg.w)
    return _encoders[key]


def encode_gpu(cfg, T: int, P: int) -> np.ndarray:
    import torch
    enc = encoder_for(cfg)
    v = torch.from_numpy(SE.make_video(T, cfg.h, cfg.w, seed=0, bf16=cfg.weights_bf16)).cuda()
    if cfg.weights_bf16:
        v = v.to(torch.bfloat16)
    z = enc.encode(v, frames_per_pass=P)
    torch.cuda.synchronize()
    assert_range_clean()
    return z.cpu().numpy()


def check_close(got, ref, name):
    d = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    r = rel_l2(got, ref)
    print(f"{name}: max_abs={d.max():.3e} rel_l2={r:.3e} (oracle rms {np.sqrt(np.mean(ref ** 2)):.3f})", flush=True)
    assert np.isfinite(got).all()
    assert d.max() <= MAX_ABS, (name, d.max())
    assert r <= REL_L2, (name, r)


# The full-width (c=256) encoder at a tiny latent size.
ENC_C256_SMALL = SE.EncoderConfig("enc_c256_T3_2x3", 256, 3, 2, 3, (1, 3))


@pytest.mark.parametrize("cfg", [SE.encoder_config_by_name("enc_tiny_c16_T2_4x6"),
                                 SE.encoder_config_by_name("enc_c64_T3_352x624"), ENC_C256_SMALL],
                         ids=lambda c: c.name)
def test_encode_matches_oracle_and_is_pass_invariant(cfg):
    ref = oracle_latents(cfg, cfg.T)
    outs = {}
    for P in sorted(set(cfg.passes) | {1, cfg.T}):
        print(f"case {cfg.name} P={P}", flush=True)
        outs[P] = encode_gpu(cfg, cfg.T, P)
        assert outs[P].shape == cfg.latent_shape
        check_close(outs[P], ref, f"{cfg.name} P={P}")
    first = next(iter(outs.values()))
    for P, z in outs.items():
        assert np.array_equal(z, first), f"P={P} differs"


def test_encode_causal_prefix_bit_identical():
    cfg = SE.encoder_config_by_name("enc_c64_T3_352x624")
    full = encode_gpu(cfg, 3, 2)
    for k in (1, 2):
        print(f"case encoder prefix k={k}", flush=True)
        assert np.array_equal(encode_gpu(cfg, k, 2), full[:, :, :k])


def test_full_size_encoder_prefix_matches_oracle():
    """c=256 at 704x1248: the oracle's latents of the first five video frames
    against a 2-latent-frame encode at frames_per_pass 1 (two passes: the
    history rings at full size) and the first two latent frames of the
    13-latent-frame encode at frames_per_pass 4; the latter bit-identical at
    frames_per_pass 4 and 13."""
    import torch
    cfg = SE.encoder_config_by_name("enc_c256_T13_704x1248")
    ref = oracle_latents(cfg, 2)
    print("case full-size encoder T=2 P=1", flush=True)
    check_close(encode_gpu(cfg, 2, 1), ref, "encoder T=2 P=1")
    print("case full-size encoder T=13 P=4", flush=True)
    z4 = encode_gpu(cfg, 13, 4)
    check_close(z4[:, :, :2], ref, "encoder T=13 P=4 frames 0..1")
    encoder_for(cfg).release_workspace()
    torch.cuda.empty_cache()
    print("case full-size encoder T=13 P=13", flush=True)
    assert np.array_equal(encode_gpu(cfg, 13, 13), z4)
    _encoders.clear()
    torch.cuda.empty_cache()
