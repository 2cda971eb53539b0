"""Seeded input generator: determinism, inventory and bf16 rounding."""
import numpy as np
import torch

from video_diffusion_vae_amd import synth


def test_inventory_count_and_shapes():
    for c in (16, 64, 256):
        specs = synth.weight_specs(c)
        assert len(specs) == 84
        names = [s.name for s in specs]
        assert len(set(names)) == 84
        d = {s.name: s.shape for s in specs}
        assert d["conv_in.weight"] == (4 * c, 48, 3, 3, 3)
        assert d["mid.attn.qkv.weight"] == (12 * c, 4 * c)
        assert d["up2.res0.shortcut.weight"] == (2 * c, 4 * c, 1, 1, 1)
        assert d["up3.res0.shortcut.weight"] == (c, 2 * c, 1, 1, 1)
        assert d["up1.time_conv.weight"] == (8 * c, 4 * c, 3, 1, 1)
        assert d["up2.up_conv.weight"] == (2 * c, 2 * c, 3, 3)
        assert d["head.conv.weight"] == (12, c, 3, 3, 3)
        assert "up3.up_conv.weight" not in d and "up2.time_conv.weight" not in d


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-8, 8, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 65504.0], np.float32)]).astype(np.float32)
    ours = synth.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(ours, ref)
    bits = synth.bf16_bits(ours)
    np.testing.assert_array_equal(bits, torch.from_numpy(ours).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_weights_deterministic_and_law():
    a = synth.make_weights(16, seed=5)
    b = synth.make_weights(16, seed=5)
    assert list(a) == synth.weight_names(16)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    w = synth.make_weights(16, seed=5, bf16=False)["up3.res1.conv1.weight"]
    bound = 1 / np.sqrt(16 * 27)
    assert np.abs(w).max() <= bound and np.abs(w).max() > 0.95 * bound
    g = synth.make_weights(64, seed=5, bf16=False)["mid.res0.norm1.gamma"]
    assert abs(g.mean() - 1) < 0.03 and abs(g.std() - 0.1) < 0.02


def test_latents_prefix_property():
    z5 = synth.make_latents(5, 4, 6, seed=2)
    z3 = synth.make_latents(3, 4, 6, seed=2)
    np.testing.assert_array_equal(z5[:, :, :3], z3)
    assert z5.shape == (1, 48, 5, 4, 6)
    np.testing.assert_array_equal(synth.bf16_round(z5), z5)
