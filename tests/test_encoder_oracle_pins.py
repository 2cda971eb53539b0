"""Pins of the encoder oracle (oracle/encoder.py) against things other than
itself: torch CPU routines (pixel_unshuffle, strided conv2d, conv3d), brute
force, closed forms, causality and pass invariance.  The layer functions it
shares with the decoder oracle are pinned in tests/test_oracle_pins.py."""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

from oracle import decoder as OD
from oracle import encoder as OE
from video_diffusion_vae_amd import synth_encoder as SE

C_TINY = 4


def rnd(rng, *shape, scale=1.0):
    return (scale * rng.standard_normal(shape)).astype(np.float32)


def test_patchify_matches_torch_and_inverts_the_pixel_shuffle():
    rng = np.random.default_rng(0)
    v = rnd(rng, 3, 4, 6, 10)
    p = OE.patchify(v)
    assert p.shape == (4, 3, 5, 12)
    ref = Fnn.pixel_unshuffle(torch.from_numpy(v).permute(1, 0, 2, 3), 2)  # [F, 12, H, W]
    np.testing.assert_array_equal(p, ref.permute(0, 2, 3, 1).numpy())
    np.testing.assert_array_equal(OD.pixel_shuffle_video(p), v)
    # channel 4k + 2dy + dx holds pixel (2Y + dy, 2X + dx) of colour k
    for k, dy, dx in itertools.product(range(3), range(2), range(2)):
        np.testing.assert_array_equal(p[..., 4 * k + 2 * dy + dx], v[k, :, dy::2, dx::2])


def test_down_conv_matches_torch_and_brute_force():
    rng = np.random.default_rng(1)
    x = rnd(rng, 2, 6, 8, 3)
    w = rnd(rng, 5, 3, 3, 3)
    b = rnd(rng, 5)
    got = OE.down_conv(x, w, b)
    assert got.shape == (2, 3, 4, 5)
    xt = torch.from_numpy(x).permute(0, 3, 1, 2).double()
    ref = Fnn.conv2d(xt, torch.from_numpy(w).double(), torch.from_numpy(b).double(), stride=2, padding=1)
    np.testing.assert_allclose(got, ref.permute(0, 2, 3, 1).numpy(), rtol=1e-5, atol=1e-5)
    brute = np.zeros(got.shape, np.float64)
    for f, Y, X, o in itertools.product(range(2), range(3), range(4), range(5)):
        acc = float(b[o])
        for i, dy, dx in itertools.product(range(3), range(3), range(3)):
            yy, xx = 2 * Y + dy - 1, 2 * X + dx - 1
            if 0 <= yy < 6 and 0 <= xx < 8:
                acc += float(w[o, i, dy, dx]) * float(x[f, yy, xx, i])
        brute[f, Y, X, o] = acc
    np.testing.assert_allclose(got, brute, rtol=1e-5, atol=1e-5)


def test_time_downsample_rule():
    """Frame 0 passes; output frame s+1 = b + sum_dt W[:, :, dt] . pair[s+dt-2]
    with pair s = [x(2s+1), x(2s+2)] along channels and zero pairs in front."""
    rng = np.random.default_rng(2)
    C, H, W = 3, 2, 3
    x = rnd(rng, 7, H, W, C)                   # frames 0..6 -> 4 frames
    w = rnd(rng, C, 2 * C, 3, 1, 1)
    b = rnd(rng, C)
    y = OE.time_downsample(x, w, b, "t", OD.Cache())
    assert y.shape == (4, H, W, C)
    np.testing.assert_array_equal(y[0], x[0])
    pairs = [np.concatenate([x[2 * s + 1], x[2 * s + 2]], axis=-1).astype(np.float64) for s in range(3)]
    for s in range(3):
        acc = np.broadcast_to(b.astype(np.float64), (H, W, C)).copy()
        for dt in range(3):
            j = s + dt - 2
            if j >= 0:
                acc += pairs[j] @ w[:, :, dt, 0, 0].T.astype(np.float64)
        np.testing.assert_allclose(y[s + 1], acc, rtol=1e-5, atol=1e-5)
    # the same with torch: conv3d over the pair sequence with two zero pairs in front
    pt = torch.from_numpy(np.stack(pairs)).permute(3, 0, 1, 2)[None]
    ref = Fnn.conv3d(Fnn.pad(pt, (0, 0, 0, 0, 2, 0)), torch.from_numpy(w).double(), torch.from_numpy(b).double())
    np.testing.assert_allclose(y[1:], ref[0].permute(1, 2, 3, 0).numpy(), rtol=1e-5, atol=1e-5)


def test_time_downsample_chunks_carry_pairs():
    """A later chunk (starting on an odd frame) continues from the previous
    chunk's last two pairs: chunked output equals the whole-clip output."""
    rng = np.random.default_rng(3)
    x = rnd(rng, 9, 2, 2, 2)
    w = rnd(rng, 2, 4, 3, 1, 1)
    b = rnd(rng, 2)
    whole = OE.time_downsample(x, w, b, "t", OD.Cache())
    for cut in (1, 3, 5, 7):
        cache = OD.Cache()
        a = OE.time_downsample(x[:cut], w, b, "t", cache)
        cache.first_chunk = False
        c = OE.time_downsample(x[cut:], w, b, "t", cache)
        np.testing.assert_array_equal(np.concatenate([a, c]), whole)


@pytest.fixture(scope="module")
def tiny():
    W = SE.make_encoder_weights(C_TINY, seed=3, bf16=False)
    v = SE.make_video(3, 2, 3, seed=3, bf16=False)   # [1, 3, 9, 32, 48]
    return W, v


def test_encoder_shape_law(tiny):
    W, v = tiny
    for T in (1, 2, 3):
        z = OE.encode(v[:, :, :4 * T - 3], W, C_TINY)
        assert z.shape == (1, 48, T, 2, 3)
        assert np.isfinite(z).all()


def test_encoder_causality(tiny):
    """Latent frames from the first 4k-3 video frames do not change when later
    frames are appended (bit-exact)."""
    W, v = tiny
    full = OE.encode(v, W, C_TINY)
    for k in (1, 2):
        np.testing.assert_array_equal(OE.encode(v[:, :, :4 * k - 3], W, C_TINY), full[:, :, :k])


@pytest.mark.parametrize("P", [1, 2])
def test_encoder_frames_per_pass_invariance(tiny, P):
    W, v = tiny
    np.testing.assert_array_equal(OE.encode(v, W, C_TINY, frames_per_pass=P), OE.encode(v, W, C_TINY))


def test_encoder_zero_weights_closed_form(tiny):
    """All conv weights 0: every conv emits its bias, so the latents are the
    head bias at every position and frame."""
    W, v = tiny
    W0 = {k: (np.zeros_like(val) if k.endswith(".weight") else val) for k, val in W.items()}
    z = OE.encode(v[:, :, :5], W0, C_TINY)
    np.testing.assert_array_equal(z, np.broadcast_to(W["head.conv.bias"][None, :, None, None, None], z.shape))


def test_encoder_matches_torch_composition(tiny):
    """The encoder restated with torch CPU routines (pixel_unshuffle, conv3d
    with front padding, strided conv2d, scaled_dot_product_attention) in
    float64."""
    W, v = tiny
    Wt = {k: torch.from_numpy(val).double() for k, val in W.items()}

    def cconv(x, name):  # x [C, F, H, W]
        w = Wt[name + ".weight"]
        kt, kh, kw = w.shape[2:]
        xp = Fnn.pad(x[None], (kw // 2, kw // 2, kh // 2, kh // 2, kt - 1, 0))
        return Fnn.conv3d(xp, w, Wt[name + ".bias"])[0]

    def norm(x, g):
        return Fnn.normalize(x, dim=0) * math.sqrt(x.shape[0]) * g[:, None, None, None]

    def rb(x, n):
        h = cconv(Fnn.silu(norm(x, Wt[n + ".norm1.gamma"])), n + ".conv1")
        h = cconv(Fnn.silu(norm(h, Wt[n + ".norm2.gamma"])), n + ".conv2")
        if n + ".shortcut.weight" in Wt:
            x = cconv(x, n + ".shortcut")
        return x + h

    vt = torch.from_numpy(v[0]).double()                                   # [3, F, H, W]
    x = Fnn.pixel_unshuffle(vt.permute(1, 0, 2, 3), 2).permute(1, 0, 2, 3)  # [12, F, H/2, W/2]
    x = cconv(x, "conv_in")
    for s in range(4):
        x = rb(x, f"down{s}.res0")
        x = rb(x, f"down{s}.res1")
        if s < 3:
            y = Fnn.conv2d(x.permute(1, 0, 2, 3), Wt[f"down{s}.down_conv.weight"],
                           Wt[f"down{s}.down_conv.bias"], stride=2, padding=1)
            x = y.permute(1, 0, 2, 3)
        if s in (1, 2):
            C = x.shape[0]
            pairs = torch.cat([x[:, 1::2], x[:, 2::2]], dim=0)               # [2C, (F-1)/2, H, W]
            x = torch.cat([x[:, :1], cconv(pairs, f"down{s}.time_conv")], dim=1)
    x = rb(x, "mid.res0")
    C, Fr, H, Wd = x.shape
    xn = norm(x, Wt["mid.attn.norm.gamma"]).permute(1, 2, 3, 0).reshape(Fr, H * Wd, C)
    qkv = Fnn.linear(xn, Wt["mid.attn.qkv.weight"], Wt["mid.attn.qkv.bias"])
    q, k, vv = qkv.split(C, dim=-1)
    o = Fnn.scaled_dot_product_attention(q, k, vv)
    o = Fnn.linear(o, Wt["mid.attn.proj.weight"], Wt["mid.attn.proj.bias"])
    x = x + o.reshape(Fr, H, Wd, C).permute(3, 0, 1, 2)
    x = rb(x, "mid.res1")
    ref = cconv(Fnn.silu(norm(x, Wt["head.norm.gamma"])), "head.conv")     # [48, T, h, w]
    got = OE.encode(v, W, C_TINY)
    assert got.shape == (1,) + tuple(ref.shape)
    np.testing.assert_allclose(got[0], ref.numpy(), rtol=1e-4, atol=1e-4 * float(ref.abs().max()))


def test_encoder_weight_inventory():
    names = SE.encoder_weight_names(16)
    assert len(names) == SE.NUM_WEIGHTS_ENCODER == 84 and len(set(names)) == 84
    specs = {s.name: s.shape for s in SE.encoder_weight_specs(16)}
    assert specs["conv_in.weight"] == (16, 12, 3, 3, 3)
    assert specs["down1.res0.shortcut.weight"] == (32, 16, 1, 1, 1)
    assert specs["down2.time_conv.weight"] == (64, 128, 3, 1, 1)
    assert specs["down0.down_conv.weight"] == (16, 16, 3, 3)
    assert specs["head.conv.weight"] == (48, 64, 3, 3, 3)
    assert "down0.time_conv.weight" not in specs and "down3.down_conv.weight" not in specs


def test_encoder_flop_count_brute():
    """encoder_flops against a count that walks the layer shapes of a tiny
    encode (every conv's output voxels x Cout x Cin x taps)."""
    c, T, h, w = 4, 3, 2, 3
    W = SE.make_encoder_weights(c, seed=0, bf16=False)
    F = {"x": 4 * T - 3}
    res = {"r": 64 * h * w}
    total = 0.0

    def conv_cost(frames, px, wt):
        return 2.0 * frames * px * wt.shape[0] * int(np.prod(wt.shape[1:]))

    total += conv_cost(F["x"], res["r"], W["conv_in.weight"])
    frames, px = F["x"], res["r"]
    for s in range(4):
        for k in range(2):
            n = f"down{s}.res{k}"
            total += conv_cost(frames, px, W[n + ".conv1.weight"]) + conv_cost(frames, px, W[n + ".conv2.weight"])
            if n + ".shortcut.weight" in W:
                total += conv_cost(frames, px, W[n + ".shortcut.weight"])
        if s < 3:
            px //= 4
            total += conv_cost(frames, px, W[f"down{s}.down_conv.weight"])
        if s in (1, 2):
            frames = (frames + 1) // 2
            total += conv_cost(frames - 1, px, W[f"down{s}.time_conv.weight"])
    for n in ("mid.res0", "mid.res1"):
        total += conv_cost(frames, px, W[n + ".conv1.weight"]) + conv_cost(frames, px, W[n + ".conv2.weight"])
    C = 4 * c
    total += 2.0 * frames * px * (3 * C * C + C * C) + 2.0 * frames * 2 * px * px * C
    total += conv_cost(frames, px, W["head.conv.weight"])
    assert (frames, px) == (T, h * w)
    assert OE.encoder_flops(c, T, h, w) == pytest.approx(total, rel=1e-12)
