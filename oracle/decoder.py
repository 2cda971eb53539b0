"""CPU oracle of the Wan-style causal video VAE decoder (test infrastructure).

This module is test infrastructure.  Only the test suite, the smoke check and
the CPU-baseline leg of the benchmark import it; the product path never calls
it.  It shares no code with the GPU library: it reads only numpy arrays made
by the seeded generator (video_diffusion_vae_amd.synth).

Everything is float32 (storage and accumulation) with plain per-frame,
per-tap loops; the one library primitive is numpy's matrix product, used for
the channel contraction of a single tap on a single frame.  Activations use
the layout [frames, height, width, channels].

Sources: the Wan2.2 VAE decoder page (FastVideo "wan22_vae_decode" README)
fixes the input/output law (latents [1,48,T,h,w] -> video [1,3,4T-3,16h,16w],
introduction), the numerics (two-byte bf16 storage, with sums and the norm's
statistics kept in fp32; "Limits"), that cutting the clip into passes does
not change the video ("Performance and memory") and that every output lies
in [-1, 1] ("Correctness").  The TensorRT-LLM issue "Opt-in BF16 norm-SiLU fusion for Wan
VAE decoding" (description) names the decoder's residual norm1/norm2 and
norm_out as channel normalization + affine scale + SiLU, and its temporal
caching.  The layer list itself (see synth.weight_specs) and the readings
where the pages are silent are documented with the design notes; each is
marked "reading" below.

Parity status: every function is pinned by tests/test_oracle_pins.py against
torch CPU library routines, brute-force loops, closed forms or invariants.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

F32 = np.float32
# Reading: the pages give the norm as x / ||x|| * sqrt(C) * gamma without an
# epsilon; 1e-12 on the norm only matters for an all-zero channel vector.
NORM_EPS = 1e-12


# ---------------------------------------------------------------------------
# Layer functions
# ---------------------------------------------------------------------------

def rms_norm(x: np.ndarray, gamma: np.ndarray) -> np.ndarray:
    """Channel RMSNorm per voxel: x / ||x||_C * sqrt(C) * gamma.

    Statistics in fp32 (Wan2.2 VAE decoder page, "Limits": fp32 RMS-norm
    statistics; TensorRT-LLM norm-SiLU issue, description: channel
    normalization and affine scaling).
    """
    x = x.astype(F32, copy=False)
    C = x.shape[-1]
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=F32))
    n = np.maximum(n, F32(NORM_EPS))
    return (x / n) * F32(np.sqrt(C)) * gamma.astype(F32)


def silu(x: np.ndarray) -> np.ndarray:
    """SiLU(v) = v / (1 + exp(-v)) (the "SiLU" of the norm-SiLU issue)."""
    with np.errstate(over="ignore"):
        return (x / (F32(1.0) + np.exp(-x))).astype(F32)


def causal_conv3d(x: np.ndarray, w: np.ndarray, b: np.ndarray,
                  history: Optional[np.ndarray] = None) -> np.ndarray:
    """Causal 3D convolution (cross-correlation), stride 1.

    x: [F, H, W, Cin]; w: [Cout, Cin, kt, kh, kw] with odd kh, kw;
    b: [Cout].  Output frame f reads input frames f - (kt-1) .. f: the tap
    dt = kt-1 hits the current frame.  Frames before the first one are the
    kt-1 frames of `history` (the last input frames of the previous chunk)
    or zero when history is None; spatial padding is zero, (k-1)/2 per side.
    Reading of "temporal caching" (TensorRT-LLM norm-SiLU issue, description)
    and of chunked decode leaving the video unchanged (Wan2.2 VAE decoder
    page, "Performance and memory").
    """
    Fr, H, W, Cin = x.shape
    Cout, Cin_w, kt, kh, kw = w.shape
    assert Cin_w == Cin and kh % 2 == 1 and kw % 2 == 1
    ph, pw = (kh - 1) // 2, (kw - 1) // 2
    if history is None:
        history = np.zeros((kt - 1, H, W, Cin), F32)
    assert history.shape == (kt - 1, H, W, Cin)
    seq = np.concatenate([history.astype(F32), x.astype(F32)], axis=0)
    seq = np.pad(seq, ((0, 0), (ph, ph), (pw, pw), (0, 0)))
    out = np.empty((Fr, H, W, Cout), F32)
    for f in range(Fr):
        acc = np.zeros((H * W, Cout), F32)
        for dt in range(kt):
            src = seq[f + dt]  # input frame f + dt - (kt-1), shifted by the history
            for dy in range(kh):
                for dx in range(kw):
                    patch = np.ascontiguousarray(src[dy:dy + H, dx:dx + W, :]).reshape(H * W, Cin)
                    wt = np.ascontiguousarray(w[:, :, dt, dy, dx].T.astype(F32))  # [Cin, Cout]
                    acc += patch @ wt
        out[f] = (acc + b.astype(F32)).reshape(H, W, Cout)
    return out


def conv2d(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Per-frame 2D convolution with zero padding (k-1)/2: w [Cout, Cin, kh, kw]."""
    return causal_conv3d(x, w[:, :, None, :, :], b)


def upsample_nearest2x(x: np.ndarray) -> np.ndarray:
    """Nearest-neighbour 2x spatial upsampling: U[Y, X] = x[Y // 2, X // 2]."""
    return np.repeat(np.repeat(x, 2, axis=1), 2, axis=2)


class Cache:
    """Per-conv history store for chunked decoding: name -> last input frames."""

    def __init__(self) -> None:
        self.frames: Dict[str, np.ndarray] = {}
        self.first_chunk = True

    def conv(self, name: str, x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
        kt = w.shape[2]
        hist = self.frames.get(name)
        y = causal_conv3d(x, w, b, hist)
        if kt > 1:
            prev = hist if hist is not None else np.zeros((kt - 1,) + x.shape[1:], F32)
            self.frames[name] = np.concatenate([prev, x], axis=0)[-(kt - 1):].copy()
        return y


def resblock(x: np.ndarray, W: Dict[str, np.ndarray], name: str, cache: Cache) -> np.ndarray:
    """ResBlock: RMSNorm -> SiLU -> CausalConv3d -> RMSNorm -> SiLU ->
    CausalConv3d, plus x (or a 1x1x1 conv of the raw x when the channel count
    changes; reading: the shortcut sees the un-normalised input and has a
    bias like every conv)."""
    h = silu(rms_norm(x, W[name + ".norm1.gamma"]))
    h = cache.conv(name + ".conv1", h, W[name + ".conv1.weight"], W[name + ".conv1.bias"])
    h = silu(rms_norm(h, W[name + ".norm2.gamma"]))
    h = cache.conv(name + ".conv2", h, W[name + ".conv2.weight"], W[name + ".conv2.bias"])
    sc = name + ".shortcut.weight"
    if sc in W:
        x = causal_conv3d(x, W[sc], W[name + ".shortcut.bias"])
    return x + h


def attention(x: np.ndarray, W: Dict[str, np.ndarray], name: str) -> np.ndarray:
    """Per-frame single-head spatial self-attention with a residual.

    Xn = RMSNorm(x) (no SiLU: the norm-SiLU issue leaves attention
    normalization native); [Q;K;V] = Wqkv Xn + b (contiguous thirds);
    S = Q K^T / sqrt(C) over the h*w tokens of the frame; softmax over keys
    (max-subtracted); O = softmax(S) V; out = x + Wp O + bp.  Reading: scale
    1/sqrt(C), one head of width C.
    """
    Fr, H, W_, C = x.shape
    L = H * W_
    out = np.empty_like(x, dtype=F32)
    wqkv = W[name + ".qkv.weight"].astype(F32)
    bqkv = W[name + ".qkv.bias"].astype(F32)
    wp = W[name + ".proj.weight"].astype(F32)
    bp = W[name + ".proj.bias"].astype(F32)
    for f in range(Fr):
        xf = x[f].reshape(L, C).astype(F32)
        xn = rms_norm(xf, W[name + ".norm.gamma"])
        qkv = xn @ np.ascontiguousarray(wqkv.T) + bqkv
        q, k, v = qkv[:, :C], qkv[:, C:2 * C], qkv[:, 2 * C:]
        s = (q @ np.ascontiguousarray(k.T)) / F32(np.sqrt(C))
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True, dtype=F32)
        o = p @ v
        out[f] = (xf + o @ np.ascontiguousarray(wp.T) + bp).reshape(H, W_, C)
    return out


def time_upsample(x: np.ndarray, w: np.ndarray, b: np.ndarray, name: str,
                  cache: Cache) -> np.ndarray:
    """time_conv temporal upsampling: F frames -> 2F - 1 (over the whole clip).

    Reading: the first frame of the clip is kept single and is neither
    convolved nor history; the causal 3x1x1 conv C -> 2C runs over the later
    frames S_s = x[s+1] with zero frames in front; output frame 2s+1 takes
    channels [0, C) of tc[s] and frame 2s+2 channels [C, 2C).
    """
    C = x.shape[-1]
    parts: List[np.ndarray] = []
    seq = x
    if cache.first_chunk:
        parts.append(x[:1])
        seq = x[1:]
    if seq.shape[0] > 0:
        tc = cache.conv(name, seq, w, b)
        Fs = seq.shape[0]
        inter = np.empty((2 * Fs,) + tc.shape[1:3] + (C,), F32)
        inter[0::2] = tc[..., :C]
        inter[1::2] = tc[..., C:]
        parts.append(inter)
    return np.concatenate(parts, axis=0)


def pixel_shuffle_video(y: np.ndarray) -> np.ndarray:
    """2x2 unpatchify of 12 channels to 3 colours: video[k, f, 2Y+dy, 2X+dx]
    = y[f, Y, X, 4k + 2dy + dx] (reading: PixelShuffle channel order)."""
    Fr, H, W_, C = y.shape
    assert C == 12
    v = y.reshape(Fr, H, W_, 3, 2, 2)            # f, Y, X, k, dy, dx
    v = v.transpose(3, 0, 1, 4, 2, 5)             # k, f, Y, dy, X, dx
    return np.ascontiguousarray(v.reshape(3, Fr, 2 * H, 2 * W_))


# ---------------------------------------------------------------------------
# Whole decoder
# ---------------------------------------------------------------------------

def decode_chunk(z: np.ndarray, W: Dict[str, np.ndarray], c: int, cache: Cache) -> np.ndarray:
    """One chunk of latent frames z [F, h, w, 48] -> video [3, F', 16h, 16w].

    The deep variant (its weights hold "pre_conv") first applies the 48 -> 48
    1x1x1 conv to the latents and has three ResBlocks per up stage (the
    Wan2.2 page's 110 decoder tensors, "Use")."""
    if "pre_conv.weight" in W:
        z = causal_conv3d(z, W["pre_conv.weight"], W["pre_conv.bias"])
    x = cache.conv("conv_in", z, W["conv_in.weight"], W["conv_in.bias"])
    x = resblock(x, W, "mid.res0", cache)
    x = attention(x, W, "mid.attn")
    x = resblock(x, W, "mid.res1", cache)
    for s in range(4):
        k = 0
        while f"up{s}.res{k}.norm1.gamma" in W:
            x = resblock(x, W, f"up{s}.res{k}", cache)
            k += 1
        if s < 2:
            x = time_upsample(x, W[f"up{s}.time_conv.weight"], W[f"up{s}.time_conv.bias"],
                              f"up{s}.time_conv", cache)
        if s < 3:
            x = conv2d(upsample_nearest2x(x), W[f"up{s}.up_conv.weight"], W[f"up{s}.up_conv.bias"])
    h = silu(rms_norm(x, W["head.norm.gamma"]))
    y = cache.conv("head.conv", h, W["head.conv.weight"], W["head.conv.bias"])
    cache.first_chunk = False
    return np.clip(pixel_shuffle_video(y), F32(-1.0), F32(1.0))


def decode(z: np.ndarray, W: Dict[str, np.ndarray], c: int,
           frames_per_pass: Optional[int] = None) -> np.ndarray:
    """Decode latents [1, 48, T, h, w] into video [1, 3, 4T-3, 16h, 16w].

    frames_per_pass=None decodes the whole clip at once; otherwise the clip is
    cut into chunks of that many latent frames and every temporal conv carries
    its last two input frames from chunk to chunk (the pages' frames_per_pass,
    whose value must not change the video).
    """
    assert z.ndim == 5 and z.shape[0] == 1 and z.shape[1] == 48
    T = z.shape[2]
    zt = np.ascontiguousarray(z[0].transpose(1, 2, 3, 0)).astype(F32)  # [T, h, w, 48]
    P = T if frames_per_pass is None else int(frames_per_pass)
    assert P >= 1
    cache = Cache()
    outs = []
    for t0 in range(0, T, P):
        outs.append(decode_chunk(zt[t0:t0 + P], W, c, cache))
    return np.concatenate(outs, axis=1)[None]


def conv_flops(c: int, T: int, h: int, w: int, deep: bool = False) -> float:
    """Multiply-add FLOPs (2 per MAC) of the decoder as the oracle computes it
    (up-convs as 3x3 convs on the upsampled frames); deep adds the 48 -> 48
    1x1x1 conv and a third ResBlock per up stage."""
    c4 = 4 * c
    F0, F1, F2 = T, 2 * T - 1, 4 * T - 3
    r = [h * w, 4 * h * w, 16 * h * w, 64 * h * w]
    fl = 0.0
    if deep:
        fl += F0 * r[0] * 48 * 48
    fl += F0 * r[0] * c4 * 48 * 27
    fl += 2 * (2 * F0 * r[0] * c4 * c4 * 27)
    fl += F0 * r[0] * (3 * c4 * c4 + c4 * c4) + F0 * 2 * r[0] * r[0] * c4
    widths = [c4, c4, 2 * c, c]
    frames = [F0, F1, F2, F2]
    prev = c4
    for s in range(4):
        cs, Fr, px = widths[s], frames[s], r[s]
        fl += Fr * px * cs * prev * 27 + Fr * px * cs * cs * 27
        if prev != cs:
            fl += Fr * px * cs * prev
        fl += (4 if deep else 2) * Fr * px * cs * cs * 27
        if s < 2:
            fl += (Fr - 1) * px * 2 * cs * cs * 3
        if s < 3:
            Fn = frames[s + 1]
            fl += Fn * r[s + 1] * cs * cs * 9
        prev = cs
    fl += F2 * r[3] * 12 * c * 27
    return 2.0 * fl
