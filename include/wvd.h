/*
 * wvd.h -- C ABI of the MI355X (gfx950) Wan-style causal video VAE decoder.
 *
 * The decoder turns latents [1, 48, T, h, w] into video
 * [1, 3, 4T-3, 16h, 16w] for any T >= 1 (Wan2.2 VAE decoder page,
 * introduction: 48 latent channels, 16x16 spatial and 4x temporal
 * compression).  Weights are prepared once (layout and phase transforms;
 * same page, "Use": the decoder prepares the weights once and its raw entry
 * points are destination-passing on the current stream); decoding writes into
 * a caller-owned bf16 video buffer on the caller's stream.  Arithmetic: the
 * pages' kernel stores weights and activations in two-byte bf16 and keeps its
 * sums and norm statistics in fp32 (same page, "Limits"); this library keeps
 * the two-byte storage and MFMA operand width but in fp16 (which gfx950
 * multiplies at the bf16 rate and into which every bf16 weight of normal
 * range converts exactly), with fp32 accumulation and fp32 norm statistics.
 * A stored value beyond the fp16 range saturates to +-65504 and a NaN is
 * stored as NaN; both are recorded in the device's range flags
 * (wvd_range_flags).  Each pass carries frames_per_pass latent frames through
 * the whole decoder: a larger value needs more workspace and runs faster, and
 * the video is bit-identical for every value (same page, "Performance and
 * memory").
 *
 * Memory ownership: the caller owns every device buffer (weights, prepared
 * buffer, workspace, latents, video).  A plan refers to the prepared buffer
 * but does not own it.  All device pointers are HIP device addresses on the
 * device current at the call; all work is enqueued on `stream` (NULL = the
 * default stream) and nothing synchronises the host.
 *
 * Errors: every entry point validates its arguments on the host before it
 * enqueues anything; on an error it returns a negative wvd_status, enqueues
 * nothing and leaves the output untouched.  A HIP launch failure returns
 * WVD_EHIP (work enqueued before it may have run).  No C++ exception crosses
 * this ABI.
 */
#ifndef WVD_H
#define WVD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct wvd_plan wvd_plan; /* opaque; read-only after wvd_prepare */

enum wvd_status {
  WVD_OK = 0,
  WVD_EINVAL = -1,      /* null pointer, bad count, T < 1, frames_per_pass < 1 */
  WVD_ESHAPE = -2,      /* shape inconsistent with the plan */
  WVD_ENOSPACE = -3,    /* prepared buffer or workspace smaller than required */
  WVD_EUNSUPPORTED = -4,/* c not a positive multiple of 16, h or w out of range */
  WVD_EHIP = -5         /* a HIP call failed */
};

/* Number of weight tensors in the canonical order (see wvd_prepare). */
#define WVD_NUM_WEIGHTS 84
/* The deep variant: a 48 -> 48 1x1x1 conv on the latents before conv_in and
 * three ResBlocks per up stage (the 110 decoder tensors of the Wan2.2 page,
 * "Use"). */
#define WVD_NUM_WEIGHTS_DEEP 110

/* Element type of the weights and latents handed to wvd_prepare/wvd_decode. */
enum wvd_dtype { WVD_DTYPE_BF16 = 0, WVD_DTYPE_F32 = 1 };

/* Bytes of the prepared-weights buffer for base width c at latent size h x w.
 * c: positive multiple of 16; 1 <= h, w <= 4096.  Writes *bytes.
 * wvd_prepared_bytes is the 84-tensor decoder; wvd_prepared_bytes_n takes the
 * tensor count (WVD_NUM_WEIGHTS or WVD_NUM_WEIGHTS_DEEP). */
int wvd_prepared_bytes(int c, int h, int w, size_t* bytes);
int wvd_prepared_bytes_n(int c, int h, int w, int n_weights, size_t* bytes);

/* One-time weight preparation (Wan2.2 VAE decoder page, "Use": layout and
 * phase transforms of the weights, done once).
 *   weights:  WVD_NUM_WEIGHTS device pointers to tensors of weight_dtype
 *             (WVD_DTYPE_BF16 or WVD_DTYPE_F32), contiguous, in
 *             the canonical order and PyTorch layouts: conv_in (weight
 *             [4c,48,3,3,3], bias); mid.res0 (norm1.gamma, conv1.weight,
 *             conv1.bias, norm2.gamma, conv2.weight, conv2.bias); mid.attn
 *             (norm.gamma [4c], qkv.weight [12c,4c], qkv.bias, proj.weight
 *             [4c,4c], proj.bias); mid.res1; then for stage s = 0..3 with
 *             widths [4c,4c,2c,c]: res0 (+ shortcut.weight [Cs,Cprev,1,1,1],
 *             shortcut.bias when the width changes), res1, time_conv (weight
 *             [2Cs,Cs,3,1,1], bias; s < 2), up_conv (weight [Cs,Cs,3,3],
 *             bias; s < 3); head (norm.gamma [c], conv.weight [12,c,3,3,3],
 *             conv.bias).
 *   n_weights: WVD_NUM_WEIGHTS, or WVD_NUM_WEIGHTS_DEEP for the deep
 *             variant, whose list starts with pre_conv (weight
 *             [48,48,1,1,1], bias) and has res0, res1, res2 in every stage.
 *   prepared: caller-owned device buffer of wvd_prepared_bytes_n(c, h, w,
 *             n_weights) bytes.
 * The input weights may be freed once the enqueued work has completed.  On
 * success *plan_out receives a host object to release with wvd_destroy. */
int wvd_prepare(int c, int h, int w, const void* const* weights, int n_weights,
                int weight_dtype, void* prepared, size_t prepared_bytes, void* stream,
                wvd_plan** plan_out);

/* Workspace bytes wvd_decode needs for T latent frames at frames_per_pass.
 * Depends on min(T, frames_per_pass) only. */
int wvd_workspace_bytes(const wvd_plan* plan, int T, int frames_per_pass, size_t* bytes);

/* Decode latents into video (destination-passing, on `stream`).
 *   z:   device [1, 48, T, h, w] of z_dtype (WVD_DTYPE_BF16 or WVD_DTYPE_F32),
 *        contiguous (the plan's h, w).
 *   out: device bf16 [1, 3, 4T-3, 16h, 16w], contiguous; every element is
 *        written, finite and in [-1, 1].
 *   workspace: device buffer of at least wvd_workspace_bytes(plan, T, P).
 * The output is bit-identical for every frames_per_pass >= 1, and its first
 * 4k-3 frames are bit-identical to the decode of the first k latent frames.
 * Concurrent decodes with one plan need separate workspaces. */
int wvd_decode(const wvd_plan* plan, const void* z, int z_dtype, int T, int frames_per_pass,
               void* out, void* workspace, size_t workspace_bytes, void* stream);

/* wvd_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same decode into the caller's `out`, with the workspace taken from a static
 * device array of WVD_STATIC_WORKSPACE_BYTES inside the library (one per
 * device, held until the process ends; 32 MiB fits e.g. the c=16 decoder at
 * 4 x 6 latents for frames_per_pass <= 10, or c=256 at 2 x 3 for <= 3).
 * It calls no hipMalloc, hipFree or other allocating routine.
 *   Same arguments, video and bit-identity as wvd_decode without the
 *   workspace.  WVD_ENOSPACE (with the sizes in wvd_last_error) when
 *   wvd_workspace_bytes(plan, T, frames_per_pass) exceeds the static size;
 *   nothing is enqueued then.
 * Every call on a device shares that device's array and leaves its contents
 * behind (no decode depends on them): calls on one device whose work overlaps
 * in time (several host threads, or several streams) race and corrupt each
 * other's video.  Serialise them on one stream. */
#define WVD_STATIC_WORKSPACE_BYTES ((size_t)32 << 20)
int wvd_decode_static(const wvd_plan* plan, const void* z, int z_dtype, int T, int frames_per_pass, void* out,
                      void* stream);

/* Streaming decode (the temporal caching of the norm-SiLU issue, "Feature,
 * motivation and proposed scope"; the segment-wise generation of the Wan2.2
 * page's introduction): latents arrive in chunks and each chunk's video is
 * produced as soon as it arrives.  The causal history (the last two raw input
 * frames of every temporal conv) is carried between calls in a caller-owned
 * state buffer.
 *
 * wvd_state_bytes: bytes of that state for the plan (independent of T and of
 * frames_per_pass).
 * wvd_chunk_workspace_bytes: workspace bytes wvd_decode_chunk needs for a
 * chunk of T latent frames at frames_per_pass (the state is not part of it).
 *
 * wvd_decode_chunk decodes latent frames [t_begin, t_begin + T) of a clip:
 *   z:       device [1, 48, T, h, w] of z_dtype, contiguous: those frames only.
 *   t_begin: latent frames of this clip already decoded into `state`; 0
 *            starts a new clip (the state's contents are then ignored).
 *   state:   device buffer of state_bytes >= wvd_state_bytes(plan), 16-byte
 *            aligned, owned by the caller.  Read (t_begin > 0) and rewritten
 *            by the call; it must hold the state the previous chunk of the
 *            same clip left (that chunk ending at t_begin), on the same plan.
 *            One state per clip: concurrent chunks of one clip are invalid.
 *   out:     device bf16 [1, 3, V, 16h, 16w], contiguous, with
 *            V = v(t_begin + T) - v(t_begin), v(t) = (t > 0 ? 4t - 3 : 0):
 *            the clip's video frames [v(t_begin), v(t_begin + T)).
 *   workspace: at least wvd_chunk_workspace_bytes(plan, T, frames_per_pass).
 * The video of a clip decoded in chunks of any sizes, at any frames_per_pass,
 * is bit-identical to wvd_decode of the whole clip.  Errors as wvd_decode;
 * WVD_ENOSPACE also for a short state. */
int wvd_state_bytes(const wvd_plan* plan, size_t* bytes);
int wvd_chunk_workspace_bytes(const wvd_plan* plan, int T, int frames_per_pass, size_t* bytes);
int wvd_decode_chunk(const wvd_plan* plan, const void* z, int z_dtype, int T, int t_begin, int frames_per_pass,
                     void* state, size_t state_bytes, void* out, void* workspace, size_t workspace_bytes,
                     void* stream);

/* ---- The encoder: video [1, 3, 4T-3, 16h, 16w] -> latents [1, 48, T, h, w].
 * The pages say only that the decoder's encoder stays native (the norm-SiLU
 * issue, "Feature, motivation and proposed scope"); this one is the decoder's
 * mirror image: a 2x2 patchify into 12 channels (channel 4k+2dy+dx = pixel
 * (2Y+dy, 2X+dx) of colour k), conv_in 12 -> c, four down stages of widths
 * [c, 2c, 4c, 4c] with two ResBlocks each, a 3x3 stride-2 (zero pad 1)
 * down-conv after stages 0-2, a temporal down-conv after those of stages 1
 * and 2 (the clip's first frame kept single; later frames in pairs (2s+1,
 * 2s+2), channels concatenated, causal 3x1x1 conv 2C -> C), a mid block
 * (ResBlock, attention, ResBlock) and a head (RMSNorm, SiLU, causal 3x3x3
 * conv 4c -> 48).  Same numerics as the decoder (fp16 storage, fp32
 * accumulation), fp32 latents.
 *
 * wvd_encoder_prepared_bytes / wvd_encoder_prepare: as wvd_prepared_bytes /
 *   wvd_prepare for the encoder's WVD_NUM_WEIGHTS_ENCODER tensors in their
 *   canonical order and PyTorch layouts: conv_in (weight [c,12,3,3,3],
 *   bias); for stage s = 0..3 of width Cs: res0 (norm1.gamma, conv1.weight,
 *   conv1.bias, norm2.gamma, conv2.weight, conv2.bias, + shortcut.weight
 *   [Cs,Cprev,1,1,1], shortcut.bias when the width changes), res1,
 *   down_conv (weight [Cs,Cs,3,3], bias; s < 3), time_conv (weight
 *   [Cs,2Cs,3,1,1], bias; s = 1, 2); mid.res0; mid.attn (norm.gamma,
 *   qkv.weight [12c,4c], qkv.bias, proj.weight [4c,4c], proj.bias);
 *   mid.res1; head (norm.gamma [4c], conv.weight [48,4c,3,3,3], conv.bias).
 *   The plan serves only the wvd_encode* calls (the decoder calls return
 *   WVD_EINVAL on it, and these on a decoder plan).
 * wvd_encode_workspace_bytes: workspace for T latent frames at
 *   frames_per_pass (depends on min(T, frames_per_pass)).
 * wvd_encode: video: device [1, 3, 4T-3, 16h, 16w] of video_dtype
 *   (WVD_DTYPE_BF16 or WVD_DTYPE_F32), contiguous; latents: device fp32
 *   [1, 48, T, h, w], contiguous, every element written.  Pass k covers
 *   latent frames [kP, kP+P) (video frames [0, 4P-3), then [4kP-3,
 *   4(k+1)P-3)); the latents are bit-identical for every frames_per_pass and
 *   their first k frames to the encode of the first 4k-3 video frames.
 *   Errors as wvd_decode. */
#define WVD_NUM_WEIGHTS_ENCODER 84
int wvd_encoder_prepared_bytes(int c, int h, int w, size_t* bytes);
int wvd_encoder_prepare(int c, int h, int w, const void* const* weights, int n_weights, int weight_dtype,
                        void* prepared, size_t prepared_bytes, void* stream, wvd_plan** plan_out);
int wvd_encode_workspace_bytes(const wvd_plan* plan, int T, int frames_per_pass, size_t* bytes);
int wvd_encode(const wvd_plan* plan, const void* video, int video_dtype, int T, int frames_per_pass, float* latents,
               void* workspace, size_t workspace_bytes, void* stream);

/* Release a plan (host memory only; the prepared buffer stays the caller's).
 * NULL is ignored. */
void wvd_destroy(wvd_plan* plan);

/* Static description of a status code. */
const char* wvd_status_string(int status);

/* Text naming the launch and HIP error behind the last WVD_EHIP returned on
 * the calling thread (and the sizes behind a WVD_ENOSPACE of
 * wvd_decode_static); "" if none.  Valid until the next call on the thread. */
const char* wvd_last_error(void);

/* Range events of the values stored as fp16 on the current device since the
 * last clear, by every decode on that device: *flags gets bit 0
 * (WVD_RANGE_SATURATED) when a finite value beyond +-65504 was stored
 * (saturated there) and bit 1 (WVD_RANGE_NAN) when a NaN was stored; 0 for a
 * decode whose every stored value was in range.  Waits for the work enqueued
 * on `stream`; with clear != 0 then resets the flags.  The flags are shared by
 * all plans and streams of the device: read them when no other decode on it
 * is in flight.  WVD_EINVAL on a null `flags`; in dry-run mode *flags = 0. */
#define WVD_RANGE_SATURATED 1u
#define WVD_RANGE_NAN 2u
int wvd_range_flags(void* stream, int clear, unsigned int* flags);

/* Math self-test: for n fp32 inputs x (device, n <= 2^31) writes the SiLU
 * (t / (1 + e^-t)) and the exponential e^t exactly as the decoder's kernels
 * evaluate them (the hardware exp2 and reciprocal; the norm-SiLU issue,
 * "Prototype evidence and limits", asks that such fast exp/sqrt lowering be
 * reviewed) into silu_out and exp_out (device, n floats each), on `stream`.
 * A test bounds their error against an exact reference over the input ranges
 * the decoder feeds them.  WVD_EINVAL on null buffers or a bad n. */
int wvd_math_probe(const float* x, float* silu_out, float* exp_out, long long n, void* stream);

/* Conversion self-test: for n fp32 inputs x (device; n a multiple of 8,
 * n <= 2^31; x, h_out and rs_out 16-byte aligned) writes, on `stream`:
 *   h_out[i]  = the fp16 bit pattern the kernels store for x[i], packed eight
 *               values at a time as every kernel packs them (round to
 *               nearest even; a finite value beyond +-65504 saturates there
 *               and a NaN stays NaN, each raising its range flag);
 *   rs_out[i] = the norm scale 1 / max(sqrt(x[i]), 1e-12) as the Winograd
 *               input transforms compute it from a channel sum of squares
 *               x[i] >= 0 (one hardware reciprocal square root).
 * The RMSNorm the decoder's residual blocks use is the Wan2.2 VAE decoder
 * page's; a test compares h_out with IEEE round-to-nearest-even bit for bit
 * and bounds rs_out against an exact reference.  WVD_EINVAL on null or
 * misaligned buffers or a bad n. */
int wvd_f16_probe(const float* x, unsigned short* h_out, float* rs_out, long long n, void* stream);

/* Host-validation mode for testing without a GPU: with on != 0, every entry
 * point validates its arguments and walks the full launch schedule (all
 * per-launch checks included) but enqueues no GPU work and dereferences no
 * device pointer.  Process-wide; not for use while decodes are in flight. */
void wvd_set_dry_run(int on);

/* Kernel launches the last wvd_decode on this plan made (or would have made in
 * dry-run mode); -1 for a null plan. */
long long wvd_last_launch_count(const wvd_plan* plan);

/* Enables (1) or disables (0) HIP-event timing of every kernel wvd_decode
 * launches on the plan (events recorded on the decode's stream around each
 * launch).  wvd_profile_read synchronises on the last recorded event and
 * returns, per kernel class, the summed milliseconds, the summed FLOPs (2 per
 * multiply-add each launch performs: for the Winograd-domain GEMMs that is
 * 4/9 of the direct 3x3x3 count, F(6,3) along x) and the number of launches since the
 * previous read, then clears the record.
 * Classes: 0 the dominant conv kernel (the Winograd-domain GEMM of the
 * norm-SiLU 3x3x3 convs; the direct 3x3x3 kernel for widths it does not
 * cover), 1 other convs (conv_in, head, time_conv, up-conv, shortcut blocks),
 * 2 attention GEMMs, 3 RMS statistics and the head's norm-SiLU, 4 copies /
 * layout / softmax, 5 Winograd input and output transforms.
 * Profiling is not thread-safe.  WVD_EINVAL on a null plan or array. */
int wvd_profile_enable(wvd_plan* plan, int on);
int wvd_profile_read(const wvd_plan* plan, double* ms, double* flops, long long* launches, int n_classes);

#ifdef __cplusplus
}
#endif

#endif /* WVD_H */
