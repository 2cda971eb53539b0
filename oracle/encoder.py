"""CPU oracle of the Wan-style causal video VAE encoder (test infrastructure).

Test infrastructure only, like oracle/decoder.py (whose layer functions it
uses): only the test suite and the benchmark's CPU-baseline leg import it.
Plain float32 with per-frame, per-tap loops; activations are
[frames, height, width, channels].

The pages say only that the decoder's encoder stays native (the TensorRT-LLM
norm-SiLU issue, "Feature, motivation and proposed scope").  The encoder
computed here is the decoder's mirror image, read as follows (each point is
a reading, also listed with the design notes):
  * patchify: the inverse of the decoder's 2x2 pixel shuffle,
  * conv_in 12 -> c, down stages [c, 2c, 4c, 4c] of two ResBlocks,
  * spatial down-conv after stages 0-2: Conv2d 3x3, stride 2, zero pad 1,
  * temporal down-conv after the down-convs of stages 1 and 2: the clip's
    first frame is kept single; later frames pair up as (2s+1, 2s+2), their
    channels are concatenated, and a causal 3x1x1 conv 2C -> C runs over the
    pairs with zero history in front (the inverse of the decoder's time_conv
    interleave),
  * mid block (ResBlock, attention, ResBlock), head RMSNorm + SiLU + causal
    3x3x3 conv 4c -> 48.
Video [1, 3, 4T-3, 16h, 16w] -> latents [1, 48, T, h, w].  Chunked encoding
carries two history frames per temporal conv (pairs, for the temporal
down-convs) and gives the same latents as a whole-clip encode.

Parity status: every function is pinned by tests/test_encoder_oracle_pins.py
(torch CPU routines, brute force, closed forms, causality, pass invariance).
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from oracle.decoder import F32, Cache, attention, causal_conv3d, resblock, rms_norm, silu


def patchify(video: np.ndarray) -> np.ndarray:
    """[3, F, 2H, 2W] -> [F, H, W, 12] with channel 4k + 2dy + dx holding
    video[k, f, 2Y + dy, 2X + dx] (the inverse of the 2x2 pixel shuffle)."""
    K, Fr, H2, W2 = video.shape
    assert K == 3 and H2 % 2 == 0 and W2 % 2 == 0
    v = video.reshape(3, Fr, H2 // 2, 2, W2 // 2, 2)   # k, f, Y, dy, X, dx
    v = v.transpose(1, 2, 4, 0, 3, 5)                    # f, Y, X, k, dy, dx
    return np.ascontiguousarray(v.reshape(Fr, H2 // 2, W2 // 2, 12)).astype(F32)


def down_conv(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Per-frame Conv2d 3x3, stride 2, zero padding 1 (reading):
    out[f, Y, X, o] = b[o] + sum_{i,dy,dx} w[o, i, dy, dx] x[f, 2Y+dy-1, 2X+dx-1, i].
    x [F, H, W, C] with even H, W -> [F, H/2, W/2, Cout]."""
    Fr, H, W, C = x.shape
    Cout = w.shape[0]
    assert w.shape == (Cout, C, 3, 3) and H % 2 == 0 and W % 2 == 0
    Ho, Wo = H // 2, W // 2
    xp = np.pad(x.astype(F32), ((0, 0), (1, 1), (1, 1), (0, 0)))
    out = np.empty((Fr, Ho, Wo, Cout), F32)
    for f in range(Fr):
        acc = np.zeros((Ho * Wo, Cout), F32)
        for dy in range(3):
            for dx in range(3):
                patch = np.ascontiguousarray(xp[f, dy:dy + 2 * Ho:2, dx:dx + 2 * Wo:2, :]).reshape(Ho * Wo, C)
                acc += patch @ np.ascontiguousarray(w[:, :, dy, dx].T.astype(F32))
        out[f] = (acc + b.astype(F32)).reshape(Ho, Wo, Cout)
    return out


def time_downsample(x: np.ndarray, w: np.ndarray, b: np.ndarray, name: str, cache: Cache) -> np.ndarray:
    """Temporal down-conv over the clip: F frames -> (F + 1) / 2 (reading).

    The clip's first frame passes through unchanged and is never history.
    Later frames pair up as (2s+1, 2s+2); pair s is their channels
    concatenated (2C), and tc = causal 3x1x1 conv 2C -> C over the pairs
    (zero pairs in front, or the previous chunk's last two pairs) gives
    output frame s + 1.  A later chunk starts on an odd frame, so its frames
    pair up from its first one.
    """
    parts = []
    seq = x
    if cache.first_chunk:
        parts.append(x[:1])
        seq = x[1:]
    Fs = seq.shape[0]
    assert Fs % 2 == 0, "frames after the first come in pairs"
    if Fs > 0:
        pairs = np.concatenate([seq[0::2], seq[1::2]], axis=-1)  # [Fs/2, H, W, 2C]
        parts.append(cache.conv(name, pairs, w, b))
    return np.concatenate(parts, axis=0)


def encode_chunk(v: np.ndarray, W: Dict[str, np.ndarray], c: int, cache: Cache) -> np.ndarray:
    """One chunk of video frames [3, F, 16h, 16w] -> latents [F0, h, w, 48]."""
    x = patchify(v)
    x = cache.conv("conv_in", x, W["conv_in.weight"], W["conv_in.bias"])
    for s in range(4):
        x = resblock(x, W, f"down{s}.res0", cache)
        x = resblock(x, W, f"down{s}.res1", cache)
        if s < 3:
            x = down_conv(x, W[f"down{s}.down_conv.weight"], W[f"down{s}.down_conv.bias"])
        if s in (1, 2):
            x = time_downsample(x, W[f"down{s}.time_conv.weight"], W[f"down{s}.time_conv.bias"],
                                f"down{s}.time_conv", cache)
    x = resblock(x, W, "mid.res0", cache)
    x = attention(x, W, "mid.attn")
    x = resblock(x, W, "mid.res1", cache)
    hn = silu(rms_norm(x, W["head.norm.gamma"]))
    y = cache.conv("head.conv", hn, W["head.conv.weight"], W["head.conv.bias"])
    cache.first_chunk = False
    return y


def encode(video: np.ndarray, W: Dict[str, np.ndarray], c: int,
           frames_per_pass: Optional[int] = None) -> np.ndarray:
    """Encode video [1, 3, 4T-3, 16h, 16w] into latents [1, 48, T, h, w].

    frames_per_pass=None encodes the whole clip at once; otherwise pass k
    covers latent frames [kP, kP + P): video frames [0, 4P-3) for the first
    pass and [4kP-3, 4(k+1)P-3) after it, with every temporal conv carrying
    its history from pass to pass.
    """
    assert video.ndim == 5 and video.shape[0] == 1 and video.shape[1] == 3
    Fv = video.shape[2]
    assert Fv % 4 == 1, "4T-3 video frames"
    T = (Fv + 3) // 4
    P = T if frames_per_pass is None else int(frames_per_pass)
    assert P >= 1
    v = video[0].astype(F32)
    cache = Cache()
    outs = []
    for t0 in range(0, T, P):
        t1 = min(T, t0 + P)
        a = 0 if t0 == 0 else 4 * t0 - 3
        outs.append(encode_chunk(v[:, a:4 * t1 - 3], W, c, cache))
    z = np.concatenate(outs, axis=0)                       # [T, h, w, 48]
    return np.ascontiguousarray(z.transpose(3, 0, 1, 2))[None]


def encoder_flops(c: int, T: int, h: int, w: int) -> float:
    """Multiply-add FLOPs (2 per MAC) of the encoder as the oracle computes it."""
    c4 = 4 * c
    F0, F1, F2 = T, 2 * T - 1, 4 * T - 3
    r = [h * w, 4 * h * w, 16 * h * w, 64 * h * w]      # r[3] is the patchified level
    widths = [c, 2 * c, 4 * c, 4 * c]
    frames = [F2, F2, F1, F0]
    res = [r[3], r[2], r[1], r[0]]
    fl = F2 * r[3] * c * 12 * 27
    prev = c
    for s in range(4):
        cs, Fr, px = widths[s], frames[s], res[s]
        fl += Fr * px * cs * prev * 27 + 3 * Fr * px * cs * cs * 27
        if prev != cs:
            fl += Fr * px * cs * prev
        if s < 3:
            Fn = Fr
            fl += Fn * res[s + 1] * cs * cs * 9
        if s in (1, 2):
            fl += (frames[s + 1] - 1) * res[s + 1] * cs * 2 * cs * 3
        prev = cs
    fl += 2 * (2 * F0 * r[0] * c4 * c4 * 27)
    fl += F0 * r[0] * (3 * c4 * c4 + c4 * c4) + F0 * 2 * r[0] * r[0] * c4
    fl += F0 * r[0] * 48 * c4 * 27
    return 2.0 * fl
