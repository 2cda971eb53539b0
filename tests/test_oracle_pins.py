"""Pins of the CPU oracle against things other than itself.

Each layer function is checked against a torch CPU library routine (a
different implementation of the same definition), a brute-force loop on tiny
inputs, a closed form or an invariant, so that a dropped term, a wrong sign,
a wrong index or a transposed operand fails at least one test.
"""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

from oracle import decoder as O
from video_diffusion_vae_amd import synth

RTOL = 1e-5
ATOL = 1e-5


def rnd(rng, *shape, scale=1.0):
    return (scale * rng.standard_normal(shape)).astype(np.float32)


def torch_causal_conv3d(x, w, b, history=None):
    """torch reference: pad kt-1 frames in front (zeros or history), pad
    spatially by (k-1)/2, then F.conv3d (cross-correlation)."""
    kt, kh, kw = w.shape[2:]
    xt = torch.from_numpy(x).permute(3, 0, 1, 2)[None]  # [1, Cin, F, H, W]
    if history is None:
        xt = Fnn.pad(xt, (kw // 2, kw // 2, kh // 2, kh // 2, kt - 1, 0))
    else:
        ht = torch.from_numpy(history).permute(3, 0, 1, 2)[None]
        xt = torch.cat([ht, xt], dim=2)
        xt = Fnn.pad(xt, (kw // 2, kw // 2, kh // 2, kh // 2, 0, 0))
    y = Fnn.conv3d(xt.double(), torch.from_numpy(w).double(), torch.from_numpy(b).double())
    return y[0].permute(1, 2, 3, 0).numpy()


@pytest.mark.parametrize("k", [(3, 3, 3), (1, 1, 1), (3, 1, 1), (1, 3, 3)])
def test_causal_conv3d_matches_torch(k):
    rng = np.random.default_rng(1)
    x = rnd(rng, 4, 5, 6, 3)
    w = rnd(rng, 5, 3, *k)
    b = rnd(rng, 5)
    got = O.causal_conv3d(x, w, b)
    ref = torch_causal_conv3d(x, w, b)
    np.testing.assert_allclose(got, ref, rtol=RTOL, atol=ATOL)


def test_causal_conv3d_brute_force():
    """Seven nested loops straight from the definition out[o,f,y,x] = b[o] +
    sum_{i,dt,dy,dx} w[o,i,dt,dy,dx] * x[i, f+dt-2, y+dy-1, x+dx-1]."""
    rng = np.random.default_rng(2)
    Fr, H, W, Ci, Co = 3, 3, 4, 2, 3
    x = rnd(rng, Fr, H, W, Ci)
    w = rnd(rng, Co, Ci, 3, 3, 3)
    b = rnd(rng, Co)
    ref = np.zeros((Fr, H, W, Co), np.float64)
    for o, f, y, xx in itertools.product(range(Co), range(Fr), range(H), range(W)):
        s = float(b[o])
        for i, dt, dy, dx in itertools.product(range(Ci), range(3), range(3), range(3)):
            fi, yi, xi = f + dt - 2, y + dy - 1, xx + dx - 1
            if 0 <= fi < Fr and 0 <= yi < H and 0 <= xi < W:
                s += float(w[o, i, dt, dy, dx]) * float(x[fi, yi, xi, i])
        ref[f, y, xx, o] = s
    np.testing.assert_allclose(O.causal_conv3d(x, w, b), ref, rtol=RTOL, atol=ATOL)


def test_causal_conv3d_history_is_prefix():
    """Conv over [a; b] restricted to b's frames == conv over b with a's last
    two frames as history (causality + locality in time)."""
    rng = np.random.default_rng(3)
    a = rnd(rng, 3, 4, 5, 3)
    bb = rnd(rng, 2, 4, 5, 3)
    w = rnd(rng, 4, 3, 3, 3, 3)
    bias = rnd(rng, 4)
    full = O.causal_conv3d(np.concatenate([a, bb]), w, bias)
    part = O.causal_conv3d(bb, w, bias, history=a[-2:])
    np.testing.assert_array_equal(full[3:], part)
    ref = torch_causal_conv3d(bb, w, bias, history=a[-2:])
    np.testing.assert_allclose(part, ref, rtol=RTOL, atol=ATOL)


def test_conv2d_matches_torch():
    rng = np.random.default_rng(4)
    x = rnd(rng, 2, 5, 7, 3)
    w = rnd(rng, 4, 3, 3, 3)
    b = rnd(rng, 4)
    ref = Fnn.conv2d(torch.from_numpy(x).permute(0, 3, 1, 2).double(),
                     torch.from_numpy(w).double(), torch.from_numpy(b).double(), padding=1)
    np.testing.assert_allclose(O.conv2d(x, w, b), ref.permute(0, 2, 3, 1).numpy(), rtol=RTOL, atol=ATOL)


def test_rms_norm_closed_forms():
    rng = np.random.default_rng(5)
    x = rnd(rng, 2, 3, 4, 16, scale=3.0)
    one = np.ones(16, np.float32)
    y = O.rms_norm(x, one)
    # gamma = 1: every voxel's channel RMS is exactly 1.
    np.testing.assert_allclose(np.sqrt(np.mean(y.astype(np.float64) ** 2, axis=-1)), 1.0, rtol=1e-6)
    # scale invariance for alpha > 0; odd symmetry.
    np.testing.assert_allclose(O.rms_norm(7.5 * x, one), y, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(O.rms_norm(-x, one), -y, rtol=1e-6, atol=1e-7)
    # gamma scales channel-wise.
    g = rnd(rng, 16)
    np.testing.assert_allclose(O.rms_norm(x, g), y * g, rtol=1e-5, atol=1e-6)
    # torch library routine: F.normalize(x) * sqrt(C) * gamma.
    ref = Fnn.normalize(torch.from_numpy(x).double(), dim=-1) * math.sqrt(16) * torch.from_numpy(g).double()
    np.testing.assert_allclose(O.rms_norm(x, g), ref.numpy(), rtol=1e-5, atol=1e-6)


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 2001).astype(np.float32)
    ref = Fnn.silu(torch.from_numpy(x).double()).numpy()
    np.testing.assert_allclose(O.silu(x), ref, rtol=1e-6, atol=1e-7)
    assert O.silu(np.array([0.0], np.float32))[0] == 0.0


def test_upsample_matches_torch():
    rng = np.random.default_rng(6)
    x = rnd(rng, 2, 3, 5, 4)
    ref = Fnn.interpolate(torch.from_numpy(x).permute(0, 3, 1, 2), scale_factor=2, mode="nearest")
    np.testing.assert_array_equal(O.upsample_nearest2x(x), ref.permute(0, 2, 3, 1).numpy())


def _attn_weights(rng, C):
    return {
        "a.norm.gamma": (1 + 0.1 * rng.standard_normal(C)).astype(np.float32),
        "a.qkv.weight": rnd(rng, 3 * C, C, scale=1 / math.sqrt(C)),
        "a.qkv.bias": rnd(rng, 3 * C, scale=0.1),
        "a.proj.weight": rnd(rng, C, C, scale=1 / math.sqrt(C)),
        "a.proj.bias": rnd(rng, C, scale=0.1),
    }


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(7)
    C = 8
    x = rnd(rng, 2, 3, 4, C)
    W = _attn_weights(rng, C)
    got = O.attention(x, W, "a")
    xt = torch.from_numpy(x).double().reshape(2, 12, C)
    xn = Fnn.normalize(xt, dim=-1) * math.sqrt(C) * torch.from_numpy(W["a.norm.gamma"]).double()
    qkv = Fnn.linear(xn, torch.from_numpy(W["a.qkv.weight"]).double(), torch.from_numpy(W["a.qkv.bias"]).double())
    q, k, v = qkv.split(C, dim=-1)
    o = Fnn.scaled_dot_product_attention(q[:, None], k[:, None], v[:, None])[:, 0]
    ref = xt + Fnn.linear(o, torch.from_numpy(W["a.proj.weight"]).double(), torch.from_numpy(W["a.proj.bias"]).double())
    np.testing.assert_allclose(got, ref.reshape(2, 3, 4, C).numpy(), rtol=1e-5, atol=1e-5)


def test_attention_closed_forms():
    rng = np.random.default_rng(8)
    C = 8
    W = _attn_weights(rng, C)
    # One token: softmax over one key is 1, so O = V.
    x1 = rnd(rng, 1, 1, 1, C)
    xn = O.rms_norm(x1.reshape(1, C), W["a.norm.gamma"])
    v = xn @ W["a.qkv.weight"][2 * C:].T + W["a.qkv.bias"][2 * C:]
    ref = x1.reshape(1, C) + v @ W["a.proj.weight"].T + W["a.proj.bias"]
    np.testing.assert_allclose(O.attention(x1, W, "a").reshape(1, C), ref, rtol=1e-5, atol=1e-6)
    # Identical tokens: uniform softmax, O = V for every token.
    xs = np.broadcast_to(x1, (1, 2, 3, C)).copy()
    np.testing.assert_allclose(O.attention(xs, W, "a").reshape(6, C), np.repeat(ref, 6, 0), rtol=1e-5, atol=1e-6)
    # Zero projection: the block is the identity.
    W0 = dict(W, **{"a.proj.weight": np.zeros((C, C), np.float32), "a.proj.bias": np.zeros(C, np.float32)})
    xr = rnd(rng, 1, 2, 3, C)
    np.testing.assert_array_equal(O.attention(xr, W0, "a"), xr)


def test_pixel_shuffle_matches_torch():
    rng = np.random.default_rng(9)
    y = rnd(rng, 2, 3, 4, 12)
    ref = Fnn.pixel_shuffle(torch.from_numpy(y).permute(0, 3, 1, 2), 2)  # [F, 3, 2H, 2W]
    np.testing.assert_array_equal(O.pixel_shuffle_video(y), ref.permute(1, 0, 2, 3).numpy())


def test_time_upsample_rule():
    """Frame 0 passes through; time_conv sees [0, 0, x1], [0, x1, x2], ...;
    channels [0, C) of step s become frame 2s+1 and [C, 2C) frame 2s+2."""
    rng = np.random.default_rng(10)
    C = 3
    x = rnd(rng, 3, 2, 2, C)
    w = rnd(rng, 2 * C, C, 3, 1, 1)
    b = rnd(rng, 2 * C)
    y = O.time_upsample(x, w, b, "tc", O.Cache())
    assert y.shape == (5, 2, 2, C)
    np.testing.assert_array_equal(y[0], x[0])
    tc = torch_causal_conv3d(x[1:], w, b)  # zero history in front of x1
    np.testing.assert_allclose(y[1], tc[0, ..., :C], rtol=RTOL, atol=ATOL)
    np.testing.assert_allclose(y[2], tc[0, ..., C:], rtol=RTOL, atol=ATOL)
    np.testing.assert_allclose(y[3], tc[1, ..., :C], rtol=RTOL, atol=ATOL)
    np.testing.assert_allclose(y[4], tc[1, ..., C:], rtol=RTOL, atol=ATOL)
    # Frame 1 depends on x1 only through the current-frame tap: explicit sum.
    ref = b[:C] + np.einsum("oi,yxi->yxo", w[:C, :, 2, 0, 0], x[1])
    np.testing.assert_allclose(y[1], ref, rtol=RTOL, atol=ATOL)


def test_resblock_closed_forms():
    rng = np.random.default_rng(11)
    Ci, Co = 4, 6
    x = rnd(rng, 2, 3, 3, Ci)
    W = {
        "r.norm1.gamma": np.ones(Ci, np.float32), "r.conv1.weight": rnd(rng, Co, Ci, 3, 3, 3),
        "r.conv1.bias": rnd(rng, Co), "r.norm2.gamma": np.ones(Co, np.float32),
        "r.conv2.weight": np.zeros((Co, Co, 3, 3, 3), np.float32), "r.conv2.bias": np.zeros(Co, np.float32),
        "r.shortcut.weight": rnd(rng, Co, Ci, 1, 1, 1), "r.shortcut.bias": rnd(rng, Co),
    }
    # conv2 = 0: the block returns the 1x1x1 shortcut of the raw input.
    sc = np.einsum("oi,fyxi->fyxo", W["r.shortcut.weight"][:, :, 0, 0, 0], x) + W["r.shortcut.bias"]
    np.testing.assert_allclose(O.resblock(x, W, "r", O.Cache()), sc, rtol=RTOL, atol=ATOL)
    # Same channels, conv2 = 0: identity.
    W2 = {k: v for k, v in W.items() if "shortcut" not in k}
    W2["r.conv1.weight"] = rnd(rng, Ci, Ci, 3, 3, 3)
    W2["r.conv1.bias"] = rnd(rng, Ci)
    W2["r.norm2.gamma"] = np.ones(Ci, np.float32)
    W2["r.conv2.weight"] = np.zeros((Ci, Ci, 3, 3, 3), np.float32)
    W2["r.conv2.bias"] = np.zeros(Ci, np.float32)
    np.testing.assert_array_equal(O.resblock(x, W2, "r", O.Cache()), x)
    # conv2 = delta on the current frame/centre tap: x + SiLU(norm(conv1 out)).
    W3 = dict(W2)
    d = np.zeros((Ci, Ci, 3, 3, 3), np.float32)
    d[np.arange(Ci), np.arange(Ci), 2, 1, 1] = 1.0
    W3["r.conv2.weight"] = d
    h = torch_causal_conv3d(O.silu(O.rms_norm(x, W2["r.norm1.gamma"])).astype(np.float32),
                            W2["r.conv1.weight"], W2["r.conv1.bias"])
    ref = x + Fnn.silu(Fnn.normalize(torch.from_numpy(h), dim=-1) * 2.0).numpy()
    np.testing.assert_allclose(O.resblock(x, W3, "r", O.Cache()), ref, rtol=1e-4, atol=1e-5)


# ---------------------------------------------------------------------------
# Whole decoder
# ---------------------------------------------------------------------------

C_TINY = 4


@pytest.fixture(scope="module")
def tiny():
    W = synth.make_weights(C_TINY, seed=3, bf16=False)
    z = synth.make_latents(4, 2, 3, seed=3, bf16=False)
    return W, z


def test_decoder_shape_law_and_range(tiny):
    W, z = tiny
    for T in (1, 2, 3):
        v = O.decode(z[:, :, :T], W, C_TINY)
        assert v.shape == (1, 3, 4 * T - 3, 32, 48)
        assert np.isfinite(v).all() and v.min() >= -1.0 and v.max() <= 1.0


def test_decoder_causality(tiny):
    """Video frames from the first k latent frames do not change when later
    latent frames are appended (bit-exact: per-frame arithmetic is identical)."""
    W, z = tiny
    full = O.decode(z, W, C_TINY)
    for k in (1, 2, 3):
        np.testing.assert_array_equal(O.decode(z[:, :, :k], W, C_TINY), full[:, :, :4 * k - 3])


@pytest.mark.parametrize("P", [1, 2, 3])
def test_decoder_frames_per_pass_invariance(tiny, P):
    W, z = tiny
    np.testing.assert_array_equal(O.decode(z, W, C_TINY, frames_per_pass=P), O.decode(z, W, C_TINY))


def test_decoder_zero_weights_closed_form(tiny):
    """All conv weights 0: every conv emits its bias; the head's bias then
    decides the video: video[k, f, 2Y+dy, 2X+dx] = clamp(b[4k+2dy+dx])."""
    W, z = tiny
    W0 = {k: (np.zeros_like(v) if k.endswith(".weight") else v) for k, v in W.items()}
    b = (4.0 * synth.make_weights(C_TINY, seed=9, bf16=False)["head.conv.bias"] / 0.01 * 0.3).astype(np.float32)
    W0["head.conv.bias"] = b  # spread over (-1.5, 1.5) so the clamp engages
    v = O.decode(z[:, :, :2], W0, C_TINY)
    for k, dy, dx in itertools.product(range(3), range(2), range(2)):
        expect = np.clip(b[4 * k + 2 * dy + dx], -1, 1)
        np.testing.assert_array_equal(v[0, k, :, dy::2, dx::2], np.float32(expect))
    assert (np.abs(b) > 1).any()


def test_decoder_matches_torch_composition(tiny):
    """The decoder restated with torch CPU routines (conv3d, interpolate,
    pixel_shuffle, scaled_dot_product_attention) in float64."""
    W, z = tiny
    T = z.shape[2]
    Wt = {k: torch.from_numpy(v).double() for k, v in W.items()}

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

    x = cconv(torch.from_numpy(z[0]).double(), "conv_in")
    x = rb(x, "mid.res0")
    C, Fr, H, Wd = x.shape
    xn = norm(x, Wt["mid.attn.norm.gamma"]).permute(1, 2, 3, 0).reshape(Fr, H * Wd, C)
    qkv = Fnn.linear(xn, Wt["mid.attn.qkv.weight"], Wt["mid.attn.qkv.bias"])
    q, k, v = qkv.split(C, dim=-1)
    o = Fnn.scaled_dot_product_attention(q, k, v)
    o = Fnn.linear(o, Wt["mid.attn.proj.weight"], Wt["mid.attn.proj.bias"])
    x = x + o.reshape(Fr, H, Wd, C).permute(3, 0, 1, 2)
    x = rb(x, "mid.res1")
    for s in range(4):
        x = rb(x, f"up{s}.res0")
        x = rb(x, f"up{s}.res1")
        if s < 2:
            C = x.shape[0]
            tc = cconv(x[:, 1:], f"up{s}.time_conv")
            inter = torch.stack([tc[:C], tc[C:]], dim=2).reshape(C, -1, *x.shape[2:])
            x = torch.cat([x[:, :1], inter], dim=1)
        if s < 3:
            u = Fnn.interpolate(x.permute(1, 0, 2, 3), scale_factor=2, mode="nearest")
            u = Fnn.conv2d(u, Wt[f"up{s}.up_conv.weight"], Wt[f"up{s}.up_conv.bias"], padding=1)
            x = u.permute(1, 0, 2, 3)
    y = cconv(Fnn.silu(norm(x, Wt["head.norm.gamma"])), "head.conv")
    ref = Fnn.pixel_shuffle(y.permute(1, 0, 2, 3), 2).permute(1, 0, 2, 3).clamp(-1, 1)
    got = O.decode(z, W, C_TINY)
    assert got.shape == (1,) + tuple(ref.shape)
    np.testing.assert_allclose(got[0], ref.numpy(), rtol=1e-4, atol=2e-5)
    assert T == 4


def test_flop_count_brute():
    """conv_flops against a per-layer count of the layer list for c=4."""
    c, T, h, w = 4, 3, 2, 3
    c4, F0, F1, F2 = 4 * c, T, 2 * T - 1, 4 * T - 3
    r0, r1, r2, r3 = h * w, 4 * h * w, 16 * h * w, 64 * h * w
    macs = 0
    macs += F0 * r0 * 48 * c4 * 27
    macs += 4 * F0 * r0 * c4 * c4 * 27                # mid res0/res1
    macs += F0 * (r0 * 4 * c4 * c4 + 2 * r0 * r0 * c4)  # qkv, proj, QK^T, PV
    macs += 4 * F0 * r0 * c4 * c4 * 27                # up0
    macs += (F0 - 1) * r0 * 2 * c4 * c4 * 3             # up0 time_conv
    macs += F1 * r1 * c4 * c4 * 9                      # up0 up_conv
    macs += 4 * F1 * r1 * c4 * c4 * 27                # up1
    macs += (F1 - 1) * r1 * 2 * c4 * c4 * 3
    macs += F2 * r2 * c4 * c4 * 9
    macs += F2 * r2 * (2 * c * c4 * 27 + 3 * 2 * c * 2 * c * 27 + 2 * c * c4)  # up2 (+ shortcut)
    macs += F2 * r3 * 2 * c * 2 * c * 9                # up2 up_conv
    macs += F2 * r3 * (c * 2 * c * 27 + 3 * c * c * 27 + c * 2 * c)            # up3 (+ shortcut)
    macs += F2 * r3 * 12 * c * 27
    assert O.conv_flops(c, T, h, w) == 2.0 * macs
    # deep: + the 48x48 latent conv and one more same-width ResBlock (two
    # 3x3x3 convs) per stage at that stage's resolution and frame count
    extra = F0 * r0 * 48 * 48
    for cs, Fr, px in ((c4, F0, r0), (c4, F1, r1), (2 * c, F2, r2), (c, F2, r3)):
        extra += 2 * Fr * px * cs * cs * 27
    assert O.conv_flops(c, T, h, w, deep=True) == 2.0 * (macs + extra)


def test_deep_variant_reduces_to_the_base_decoder(tiny):
    """Deep variant (110 tensors): with pre_conv = identity and the third
    ResBlock of every stage silenced (conv2 = 0, so the block is x + 0), the
    decode equals the 84-tensor decoder with the same shared weights; a
    nonzero third block changes the video, so the blocks are wired in."""
    W, z = tiny
    Wd = synth.make_weights(C_TINY, seed=5, bf16=False, deep=True)
    assert len(Wd) == synth.NUM_WEIGHTS_DEEP and len(W) == synth.NUM_WEIGHTS
    for k, v in W.items():
        Wd[k] = v
    Wd["pre_conv.weight"] = np.eye(48, dtype=np.float32)[:, :, None, None, None]
    Wd["pre_conv.bias"] = np.zeros(48, np.float32)
    live = dict(Wd)
    for s in range(4):
        Wd[f"up{s}.res2.conv2.weight"] = np.zeros_like(Wd[f"up{s}.res2.conv2.weight"])
        Wd[f"up{s}.res2.conv2.bias"] = np.zeros_like(Wd[f"up{s}.res2.conv2.bias"])
    base = O.decode(z[:, :, :2], W, C_TINY)
    np.testing.assert_array_equal(O.decode(z[:, :, :2], Wd, C_TINY), base)
    assert not np.array_equal(O.decode(z[:, :, :2], live, C_TINY), base)


def test_deep_pre_conv_is_a_per_voxel_matrix(tiny):
    """pre_conv is a 1x1x1 conv: scaling its weight and shifting its bias is
    the same as scaling and shifting the latents fed to a pre_conv-free
    decoder (it has no temporal or spatial taps)."""
    W, z = tiny
    Wd = synth.make_weights(C_TINY, seed=6, bf16=False, deep=True)
    rng = np.random.default_rng(4)
    A = rng.uniform(-0.3, 0.3, (48, 48)).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, 48).astype(np.float32)
    Wd["pre_conv.weight"] = A[:, :, None, None, None]
    Wd["pre_conv.bias"] = b
    zz = z[:, :, :2]
    zpre = (np.einsum("oi,itxy->otxy", A.astype(np.float64), zz[0].astype(np.float64)) +
            b[:, None, None, None]).astype(np.float32)[None]
    Wn = {k: v for k, v in Wd.items() if not k.startswith("pre_conv")}
    np.testing.assert_allclose(O.decode(zz, Wd, C_TINY), O.decode(zpre, Wn, C_TINY), rtol=1e-5, atol=1e-5)
