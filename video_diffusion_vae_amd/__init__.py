"""wvd: an MI355X-native Wan-style causal video VAE decoder.

The decoder runs in a HIP library (libwvd.so, gfx950) behind a C ABI; this
package holds the ctypes binding (video_diffusion_vae_amd.wvd) and the seeded
synthetic input generator (video_diffusion_vae_amd.synth).  Importing the
package does not load the library; `from video_diffusion_vae_amd import wvd`
does, and fails loudly when it is not built.
"""
__all__ = ["synth", "wvd"]
