"""wvd_decode_static (the decode that allocates nothing: its workspace is a
static device array inside the library) against wvd_decode with a
caller-owned workspace, through the C ABI: bit-identical video on two calls
in a row, the second with a smaller input, for two decoder widths."""
import numpy as np
import pytest

from tests.gpu_util import assert_range_clean, gpu_available
from video_diffusion_vae_amd import synth

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _decoder(cfg):
    import torch

    from video_diffusion_vae_amd import wvd
    W = synth.make_weights(cfg.c, seed=0, bf16=cfg.weights_bf16)
    dt = torch.bfloat16 if cfg.weights_bf16 else torch.float32
    return wvd.Decoder({k: torch.from_numpy(v).to(dt) for k, v in W.items()}, cfg.c, cfg.h, cfg.w), dt


def _static(dec, z, P):
    import torch

    from video_diffusion_vae_amd import wvd
    T = int(z.shape[2])
    out = torch.full((1, 3, 4 * T - 3, 16 * dec.h, 16 * dec.w), float("nan"), dtype=torch.bfloat16, device="cuda")
    zdt = wvd.WVD_DTYPE_F32 if z.dtype == torch.float32 else wvd.WVD_DTYPE_BF16
    wvd.wvd_decode_static(dec.plan, z.data_ptr(), zdt, T, P, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    return out


@pytest.mark.parametrize("cfg,calls", [
    (synth.Config("tiny_c16_T4_4x6", 16, 4, 4, 6, (1,), weights_bf16=False), [(4, 4), (2, 1)]),
    (synth.Config("c256_T3_2x3", 256, 3, 2, 3, (1,)), [(3, 3), (1, 1)]),
])
def test_static_decode_matches_workspace_decode(cfg, calls):
    import torch

    from video_diffusion_vae_amd import wvd
    dec, dt = _decoder(cfg)
    z_all = torch.from_numpy(synth.make_latents(cfg.T, cfg.h, cfg.w, seed=0, bf16=cfg.weights_bf16)).cuda().to(dt)
    for T, P in calls:
        assert dec.workspace_bytes(T, P) <= wvd.WVD_STATIC_WORKSPACE_BYTES
        print(f"case {cfg.name} static T={T} P={P}", flush=True)
        z = z_all[:, :, :T].contiguous()
        got = _static(dec, z, P)
        ref = dec.decode(z, frames_per_pass=P)
        torch.cuda.synchronize()
        assert_range_clean()
        assert got.shape == ref.shape
        assert bool(torch.isfinite(got.float()).all())
        assert torch.equal(got, ref), (cfg.name, T, P)
    del dec
    torch.cuda.empty_cache()


def test_static_decode_rejects_a_workspace_beyond_the_static_array():
    import torch

    from video_diffusion_vae_amd import wvd
    cfg = synth.config_by_name("c64_T3_352x624")
    dec, dt = _decoder(cfg)
    assert dec.workspace_bytes(3, 3) > wvd.WVD_STATIC_WORKSPACE_BYTES
    z = torch.from_numpy(synth.make_latents(3, cfg.h, cfg.w, seed=0)).cuda().to(dt)
    out = torch.zeros(cfg.video_shape, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(wvd.WvdError) as e:
        wvd.wvd_decode_static(dec.plan, z.data_ptr(), wvd.WVD_DTYPE_BF16, 3, 3, out.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
    assert e.value.status == wvd.WVD_ENOSPACE and "static workspace" in str(e.value)
    torch.cuda.synchronize()
    assert not bool(out.any())  # nothing was enqueued
