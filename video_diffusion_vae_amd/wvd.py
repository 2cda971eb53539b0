"""ctypes binding of libwvd.so (the C ABI in include/wvd.h).

Argument marshalling only: every step of the decoder runs in the HIP library.
PyTorch provides device memory and the current stream.  Importing this module
loads the library and raises if it has not been built
(python -m video_diffusion_vae_amd.csrc.build).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence, Union

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwvd.so")

WVD_OK = 0
WVD_EINVAL = -1
WVD_ESHAPE = -2
WVD_ENOSPACE = -3
WVD_EUNSUPPORTED = -4
WVD_EHIP = -5
NUM_WEIGHTS = 84
NUM_WEIGHTS_DEEP = 110  # deep variant: pre_conv + three ResBlocks per up stage
NUM_WEIGHTS_ENCODER = 84
WVD_RANGE_SATURATED = 1
WVD_RANGE_NAN = 2
WVD_DTYPE_BF16 = 0
WVD_DTYPE_F32 = 1
PROFILE_CLASSES = ("conv3x3x3_main", "conv_other", "attention_gemm", "norm_stats", "copies", "wino_transforms")


class WvdError(RuntimeError):
    def __init__(self, status: int, where: str):
        detail = ""
        if status == WVD_EHIP:
            detail = " " + _lib.wvd_last_error().decode()
        super().__init__(f"{where}: {status} ({status_string(status)}){detail}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run: python -m video_diffusion_vae_amd.csrc.build")
    lib = ctypes.CDLL(LIB_PATH)
    sz = ctypes.c_size_t
    vp = ctypes.c_void_p
    i = ctypes.c_int
    lib.wvd_prepared_bytes.argtypes = [i, i, i, ctypes.POINTER(sz)]
    lib.wvd_prepared_bytes.restype = i
    lib.wvd_prepared_bytes_n.argtypes = [i, i, i, i, ctypes.POINTER(sz)]
    lib.wvd_prepared_bytes_n.restype = i
    lib.wvd_prepare.argtypes = [i, i, i, ctypes.POINTER(vp), i, i, vp, sz, vp, ctypes.POINTER(vp)]
    lib.wvd_prepare.restype = i
    lib.wvd_workspace_bytes.argtypes = [vp, i, i, ctypes.POINTER(sz)]
    lib.wvd_workspace_bytes.restype = i
    lib.wvd_decode.argtypes = [vp, vp, i, i, i, vp, vp, sz, vp]
    lib.wvd_decode.restype = i
    lib.wvd_decode_static.argtypes = [vp, vp, i, i, i, vp, vp]
    lib.wvd_decode_static.restype = i
    lib.wvd_state_bytes.argtypes = [vp, ctypes.POINTER(sz)]
    lib.wvd_state_bytes.restype = i
    lib.wvd_chunk_workspace_bytes.argtypes = [vp, i, i, ctypes.POINTER(sz)]
    lib.wvd_chunk_workspace_bytes.restype = i
    lib.wvd_decode_chunk.argtypes = [vp, vp, i, i, i, i, vp, sz, vp, vp, sz, vp]
    lib.wvd_decode_chunk.restype = i
    lib.wvd_encoder_prepared_bytes.argtypes = [i, i, i, ctypes.POINTER(sz)]
    lib.wvd_encoder_prepared_bytes.restype = i
    lib.wvd_encoder_prepare.argtypes = [i, i, i, ctypes.POINTER(vp), i, i, vp, sz, vp, ctypes.POINTER(vp)]
    lib.wvd_encoder_prepare.restype = i
    lib.wvd_encode_workspace_bytes.argtypes = [vp, i, i, ctypes.POINTER(sz)]
    lib.wvd_encode_workspace_bytes.restype = i
    lib.wvd_encode.argtypes = [vp, vp, i, i, i, vp, vp, sz, vp]
    lib.wvd_encode.restype = i
    lib.wvd_destroy.argtypes = [vp]
    lib.wvd_destroy.restype = None
    lib.wvd_status_string.argtypes = [i]
    lib.wvd_status_string.restype = ctypes.c_char_p
    lib.wvd_last_error.argtypes = []
    lib.wvd_last_error.restype = ctypes.c_char_p
    lib.wvd_set_dry_run.argtypes = [i]
    lib.wvd_set_dry_run.restype = None
    lib.wvd_last_launch_count.argtypes = [vp]
    lib.wvd_last_launch_count.restype = ctypes.c_longlong
    lib.wvd_math_probe.argtypes = [vp, vp, vp, ctypes.c_longlong, vp]
    lib.wvd_math_probe.restype = i
    lib.wvd_f16_probe.argtypes = [vp, vp, vp, ctypes.c_longlong, vp]
    lib.wvd_f16_probe.restype = i
    lib.wvd_range_flags.argtypes = [vp, i, ctypes.POINTER(ctypes.c_uint)]
    lib.wvd_range_flags.restype = i
    lib.wvd_profile_enable.argtypes = [vp, i]
    lib.wvd_profile_enable.restype = i
    lib.wvd_profile_read.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_longlong), i]
    lib.wvd_profile_read.restype = i
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def status_string(status: int) -> str:
    return _lib.wvd_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != WVD_OK:
        raise WvdError(status, where)


# ---- raw entry points (same names as the C ABI) ----

def wvd_prepared_bytes_n(c: int, h: int, w: int, n_weights: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.wvd_prepared_bytes_n(c, h, w, n_weights, ctypes.byref(n)), "wvd_prepared_bytes_n")
    return n.value


def wvd_prepared_bytes(c: int, h: int, w: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.wvd_prepared_bytes(c, h, w, ctypes.byref(n)), "wvd_prepared_bytes")
    return n.value


def wvd_prepare(c: int, h: int, w: int, weight_ptrs: Sequence[int], weight_dtype: int, prepared_ptr: int,
                prepared_bytes: int, stream_ptr: int) -> int:
    arr = (ctypes.c_void_p * len(weight_ptrs))(*weight_ptrs)
    plan = ctypes.c_void_p(0)
    _check(_lib.wvd_prepare(c, h, w, arr, len(weight_ptrs), weight_dtype, prepared_ptr, prepared_bytes, stream_ptr,
                            ctypes.byref(plan)), "wvd_prepare")
    return plan.value


def wvd_workspace_bytes(plan: int, T: int, frames_per_pass: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.wvd_workspace_bytes(plan, T, frames_per_pass, ctypes.byref(n)), "wvd_workspace_bytes")
    return n.value


def wvd_decode(plan: int, z_ptr: int, z_dtype: int, T: int, frames_per_pass: int, out_ptr: int, ws_ptr: int,
               ws_bytes: int, stream_ptr: int) -> None:
    _check(_lib.wvd_decode(plan, z_ptr, z_dtype, T, frames_per_pass, out_ptr, ws_ptr, ws_bytes, stream_ptr),
           "wvd_decode")


WVD_STATIC_WORKSPACE_BYTES = 32 << 20


def wvd_decode_static(plan: int, z_ptr: int, z_dtype: int, T: int, frames_per_pass: int, out_ptr: int,
                      stream_ptr: int) -> None:
    """wvd_decode with the library's static workspace (no allocation)."""
    st = _lib.wvd_decode_static(plan, z_ptr, z_dtype, T, frames_per_pass, out_ptr, stream_ptr)
    if st == WVD_ENOSPACE:
        raise WvdError(st, "wvd_decode_static: " + _lib.wvd_last_error().decode())
    _check(st, "wvd_decode_static")


def wvd_state_bytes(plan: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.wvd_state_bytes(plan, ctypes.byref(n)), "wvd_state_bytes")
    return n.value


def wvd_chunk_workspace_bytes(plan: int, T: int, frames_per_pass: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.wvd_chunk_workspace_bytes(plan, T, frames_per_pass, ctypes.byref(n)), "wvd_chunk_workspace_bytes")
    return n.value


def wvd_decode_chunk(plan: int, z_ptr: int, z_dtype: int, T: int, t_begin: int, frames_per_pass: int,
                     state_ptr: int, state_bytes: int, out_ptr: int, ws_ptr: int, ws_bytes: int,
                     stream_ptr: int) -> None:
    _check(_lib.wvd_decode_chunk(plan, z_ptr, z_dtype, T, t_begin, frames_per_pass, state_ptr, state_bytes, out_ptr,
                                 ws_ptr, ws_bytes, stream_ptr), "wvd_decode_chunk")


def wvd_encoder_prepared_bytes(c: int, h: int, w: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.wvd_encoder_prepared_bytes(c, h, w, ctypes.byref(n)), "wvd_encoder_prepared_bytes")
    return n.value


def wvd_encoder_prepare(c: int, h: int, w: int, weight_ptrs: Sequence[int], weight_dtype: int, prepared_ptr: int,
                        prepared_bytes: int, stream_ptr: int) -> int:
    arr = (ctypes.c_void_p * len(weight_ptrs))(*weight_ptrs)
    plan = ctypes.c_void_p(0)
    _check(_lib.wvd_encoder_prepare(c, h, w, arr, len(weight_ptrs), weight_dtype, prepared_ptr, prepared_bytes,
                                    stream_ptr, ctypes.byref(plan)), "wvd_encoder_prepare")
    return plan.value


def wvd_encode_workspace_bytes(plan: int, T: int, frames_per_pass: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.wvd_encode_workspace_bytes(plan, T, frames_per_pass, ctypes.byref(n)), "wvd_encode_workspace_bytes")
    return n.value


def wvd_encode(plan: int, video_ptr: int, video_dtype: int, T: int, frames_per_pass: int, latents_ptr: int,
               ws_ptr: int, ws_bytes: int, stream_ptr: int) -> None:
    _check(_lib.wvd_encode(plan, video_ptr, video_dtype, T, frames_per_pass, latents_ptr, ws_ptr, ws_bytes,
                           stream_ptr), "wvd_encode")


def video_frames(t: int) -> int:
    """Video frames of the first t latent frames."""
    return 4 * t - 3 if t > 0 else 0


def wvd_range_flags(stream_ptr: int, clear: bool) -> int:
    """Range flags of the fp16 stores on the current device (bit 0 saturated,
    bit 1 NaN); waits for `stream_ptr`, then clears them if asked."""
    f = ctypes.c_uint(0)
    _check(_lib.wvd_range_flags(stream_ptr, 1 if clear else 0, ctypes.byref(f)), "wvd_range_flags")
    return f.value


def wvd_math_probe(x_ptr: int, silu_ptr: int, exp_ptr: int, n: int, stream_ptr: int) -> None:
    _check(_lib.wvd_math_probe(x_ptr, silu_ptr, exp_ptr, n, stream_ptr), "wvd_math_probe")


def wvd_f16_probe(x_ptr: int, h_ptr: int, rs_ptr: int, n: int, stream_ptr: int) -> None:
    _check(_lib.wvd_f16_probe(x_ptr, h_ptr, rs_ptr, n, stream_ptr), "wvd_f16_probe")


def range_flags(clear: bool = True) -> int:
    """wvd_range_flags on torch's current stream of the current device."""
    import torch
    return wvd_range_flags(torch.cuda.current_stream().cuda_stream, clear)


def wvd_destroy(plan: int) -> None:
    _lib.wvd_destroy(plan)


def wvd_set_dry_run(on: bool) -> None:
    _lib.wvd_set_dry_run(1 if on else 0)


def wvd_last_launch_count(plan: int) -> int:
    return int(_lib.wvd_last_launch_count(plan))


def wvd_profile_enable(plan: int, on: bool) -> None:
    _check(_lib.wvd_profile_enable(plan, 1 if on else 0), "wvd_profile_enable")


def wvd_profile_read(plan: int) -> Dict[str, Dict[str, float]]:
    n = len(PROFILE_CLASSES)
    ms = (ctypes.c_double * n)()
    fl = (ctypes.c_double * n)()
    cnt = (ctypes.c_longlong * n)()
    _check(_lib.wvd_profile_read(plan, ms, fl, cnt, n), "wvd_profile_read")
    return {k: {"ms": ms[i], "flops": fl[i], "launches": int(cnt[i])} for i, k in enumerate(PROFILE_CLASSES)}


# ---- torch-facing wrapper ----

class Decoder:
    """Prepared decoder for base width c at latent size h x w on the current
    CUDA (HIP) device.  `weights` are the 84 tensors in canonical order (a
    sequence, or a dict in that order), as numpy arrays or tensors; float32
    weights are handed over as fp32 and any other float type as bf16.  They
    are copied to the device for preparation and may be dropped after."""

    def __init__(self, weights: Union[Sequence, Dict[str, object]], c: int, h: int, w: int, device=None):
        import torch

        self.torch = torch
        self.c, self.h, self.w = int(c), int(h), int(w)
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        ws = list(weights.values()) if isinstance(weights, dict) else list(weights)
        if len(ws) not in (NUM_WEIGHTS, NUM_WEIGHTS_DEEP):
            raise WvdError(WVD_EINVAL, f"Decoder: expected {NUM_WEIGHTS} or {NUM_WEIGHTS_DEEP} weights, got {len(ws)}")
        ts = [torch.as_tensor(t) for t in ws]
        f32 = all(t.dtype == torch.float32 for t in ts)
        dt = torch.float32 if f32 else torch.bfloat16
        self.weight_dtype = WVD_DTYPE_F32 if f32 else WVD_DTYPE_BF16
        dev_ws = [t.to(device=self.device, dtype=dt).contiguous() for t in ts]
        nbytes = wvd_prepared_bytes_n(self.c, self.h, self.w, len(ws))
        self.prepared = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        stream = torch.cuda.current_stream(self.device)
        self.plan = wvd_prepare(self.c, self.h, self.w, [t.data_ptr() for t in dev_ws], self.weight_dtype,
                                self.prepared.data_ptr(), nbytes, stream.cuda_stream)
        stream.synchronize()  # the input copies may be freed after this
        del dev_ws
        self._ws = None

    def workspace_bytes(self, T: int, frames_per_pass: int) -> int:
        return wvd_workspace_bytes(self.plan, T, frames_per_pass)

    def decode(self, z, frames_per_pass: int = 4, out=None, workspace=None):
        torch = self.torch
        if z.dim() != 5 or tuple(z.shape[:2]) != (1, 48) or tuple(z.shape[3:]) != (self.h, self.w):
            raise WvdError(WVD_ESHAPE, f"decode: latents of shape {tuple(z.shape)}")
        zdt = torch.float32 if z.dtype == torch.float32 else torch.bfloat16
        z = z.to(device=self.device, dtype=zdt).contiguous()
        T = int(z.shape[2])
        shape = (1, 3, 4 * T - 3, 16 * self.h, 16 * self.w)
        if out is None:
            out = torch.empty(shape, dtype=torch.bfloat16, device=self.device)
        elif tuple(out.shape) != shape or out.dtype != torch.bfloat16 or not out.is_contiguous():
            raise WvdError(WVD_ESHAPE, f"decode: out must be contiguous bf16 {shape}")
        workspace = self._workspace(self.workspace_bytes(T, frames_per_pass), workspace)
        stream = torch.cuda.current_stream(self.device)
        wvd_decode(self.plan, z.data_ptr(), WVD_DTYPE_F32 if zdt == torch.float32 else WVD_DTYPE_BF16, T,
                   int(frames_per_pass), out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                   stream.cuda_stream)
        return out

    def _workspace(self, need: int, workspace):
        if workspace is None:
            if self._ws is None or self._ws.numel() < need:
                self._ws = None
                self._ws = self.torch.empty(need, dtype=self.torch.uint8, device=self.device)
            workspace = self._ws
        return workspace

    def stream(self) -> "DecodeStream":
        """A clip decoded chunk by chunk (see DecodeStream)."""
        return DecodeStream(self)

    def release_workspace(self) -> None:
        self._ws = None

    def profile(self, on: bool = True) -> None:
        wvd_profile_enable(self.plan, on)

    def profile_read(self) -> Dict[str, Dict[str, float]]:
        return wvd_profile_read(self.plan)

    def __del__(self):
        plan = getattr(self, "plan", None)
        if plan:
            wvd_destroy(plan)
            self.plan = None


class DecodeStream:
    """One clip decoded as its latents arrive: each decode(z_chunk) returns the
    video frames of those latent frames, continuing the causal history from the
    previous chunks (kept in a device state buffer).  The concatenated chunks
    are bit-identical to Decoder.decode of the whole clip."""

    def __init__(self, dec: Decoder):
        torch = dec.torch
        self.dec = dec
        self.state = torch.empty(wvd_state_bytes(dec.plan), dtype=torch.uint8, device=dec.device)
        self.t = 0  # latent frames decoded so far

    def decode(self, z, frames_per_pass: int = 4, out=None, workspace=None):
        dec, torch = self.dec, self.dec.torch
        if z.dim() != 5 or tuple(z.shape[:2]) != (1, 48) or tuple(z.shape[3:]) != (dec.h, dec.w):
            raise WvdError(WVD_ESHAPE, f"decode_chunk: latents of shape {tuple(z.shape)}")
        zdt = torch.float32 if z.dtype == torch.float32 else torch.bfloat16
        z = z.to(device=dec.device, dtype=zdt).contiguous()
        T = int(z.shape[2])
        V = video_frames(self.t + T) - video_frames(self.t)
        shape = (1, 3, V, 16 * dec.h, 16 * dec.w)
        if out is None:
            out = torch.empty(shape, dtype=torch.bfloat16, device=dec.device)
        elif tuple(out.shape) != shape or out.dtype != torch.bfloat16 or not out.is_contiguous():
            raise WvdError(WVD_ESHAPE, f"decode_chunk: out must be contiguous bf16 {shape}")
        workspace = dec._workspace(wvd_chunk_workspace_bytes(dec.plan, T, frames_per_pass), workspace)
        stream = torch.cuda.current_stream(dec.device)
        wvd_decode_chunk(dec.plan, z.data_ptr(), WVD_DTYPE_F32 if zdt == torch.float32 else WVD_DTYPE_BF16, T, self.t,
                         int(frames_per_pass), self.state.data_ptr(), self.state.numel(), out.data_ptr(),
                         workspace.data_ptr(), workspace.numel(), stream.cuda_stream)
        self.t += T
        return out


class Encoder:
    """Prepared encoder (the decoder's mirror image) for base width c at
    latent size h x w on the current CUDA (HIP) device.  `weights` are its 84
    tensors in canonical order (video_diffusion_vae_amd.synth_encoder), as
    numpy arrays or tensors; float32 weights are handed over as fp32, any
    other float type as bf16."""

    def __init__(self, weights: Union[Sequence, Dict[str, object]], c: int, h: int, w: int, device=None):
        import torch

        self.torch = torch
        self.c, self.h, self.w = int(c), int(h), int(w)
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        ws = list(weights.values()) if isinstance(weights, dict) else list(weights)
        if len(ws) != NUM_WEIGHTS_ENCODER:
            raise WvdError(WVD_EINVAL, f"Encoder: expected {NUM_WEIGHTS_ENCODER} weights, got {len(ws)}")
        ts = [torch.as_tensor(t) for t in ws]
        f32 = all(t.dtype == torch.float32 for t in ts)
        dt = torch.float32 if f32 else torch.bfloat16
        dev_ws = [t.to(device=self.device, dtype=dt).contiguous() for t in ts]
        nbytes = wvd_encoder_prepared_bytes(self.c, self.h, self.w)
        self.prepared = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        stream = torch.cuda.current_stream(self.device)
        self.plan = wvd_encoder_prepare(self.c, self.h, self.w, [t.data_ptr() for t in dev_ws],
                                        WVD_DTYPE_F32 if f32 else WVD_DTYPE_BF16, self.prepared.data_ptr(), nbytes,
                                        stream.cuda_stream)
        stream.synchronize()
        del dev_ws
        self._ws = None

    def workspace_bytes(self, T: int, frames_per_pass: int) -> int:
        return wvd_encode_workspace_bytes(self.plan, T, frames_per_pass)

    def encode(self, video, frames_per_pass: int = 4, out=None, workspace=None):
        """video [1, 3, 4T-3, 16h, 16w] (bf16 or fp32) -> fp32 latents [1, 48, T, h, w]."""
        torch = self.torch
        if (video.dim() != 5 or tuple(video.shape[:2]) != (1, 3) or tuple(video.shape[3:]) != (16 * self.h, 16 * self.w)
                or video.shape[2] % 4 != 1):
            raise WvdError(WVD_ESHAPE, f"encode: video of shape {tuple(video.shape)}")
        vdt = torch.float32 if video.dtype == torch.float32 else torch.bfloat16
        video = video.to(device=self.device, dtype=vdt).contiguous()
        T = (int(video.shape[2]) + 3) // 4
        shape = (1, 48, T, self.h, self.w)
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=self.device)
        elif tuple(out.shape) != shape or out.dtype != torch.float32 or not out.is_contiguous():
            raise WvdError(WVD_ESHAPE, f"encode: out must be contiguous fp32 {shape}")
        need = self.workspace_bytes(T, frames_per_pass)
        if workspace is None:
            if self._ws is None or self._ws.numel() < need:
                self._ws = None
                self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
            workspace = self._ws
        stream = torch.cuda.current_stream(self.device)
        wvd_encode(self.plan, video.data_ptr(), WVD_DTYPE_F32 if vdt == torch.float32 else WVD_DTYPE_BF16, T,
                   int(frames_per_pass), out.data_ptr(), workspace.data_ptr(), workspace.numel(), stream.cuda_stream)
        return out

    def release_workspace(self) -> None:
        self._ws = None

    def profile(self, on: bool = True) -> None:
        wvd_profile_enable(self.plan, on)

    def profile_read(self) -> Dict[str, Dict[str, float]]:
        return wvd_profile_read(self.plan)

    def __del__(self):
        plan = getattr(self, "plan", None)
        if plan:
            wvd_destroy(plan)
            self.plan = None
