// Internal interfaces between the wvd host scheduler and its HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wvd_common.h"

namespace wvd {

// Output tile: TF frames x TH rows x kTileW columns of output voxels (the M
// dimension of the implicit GEMM); TF * TH * kTileW == kTileM.
constexpr int kTileW = 16;
constexpr int kTileM = 256;
constexpr int kMaxHaloItemsPerTap = 4;  // 16-byte halo items per thread per tap
constexpr int kMaxCin = 1024;           // largest norm input width kept in LDS
constexpr int kEncInC = 32;             // encoder input channels: 12 patch channels + zero padding
constexpr int kWinoTF = 2;              // frames per tile of the Winograd-domain GEMM
constexpr int kWinoM = 6;               // Winograd F(m,3) along x: output columns per group
constexpr int kWinoN = kWinoM + 2;      // transformed planes (xi) per group
constexpr int kWinoInRun = 4;           // column groups per thread of the input transform
// LDS bytes the Winograd and up-conv epilogues stage in one halo buffer:
// 8 waves x 32 positions x (32 fp32 channels + 16 bytes of pad), or 4 waves
// x 32 x (64 channels + pad), whichever is larger.
constexpr int kSwapEpiBytes = 8 * 32 * (32 * 4 + 16);
// The head's epilogue (x taps in the output columns) stages 256 rows of 44
// fp32 partial sums in one halo buffer.
constexpr int kHeadXEpiBytes = 256 * 44 * 4;

enum Prologue { PRO_RAW = 0, PRO_NORM = 1, PRO_NORM_SILU = 2 };
enum Epilogue {
  EPI_H16 = 0,     // channels-last fp16 (+ bias, + optional residual)
  EPI_F32 = 1,     // fp32 (scaled), e.g. attention logits
  EPI_TIME = 2,    // time_conv: channels [0,C) -> frame 2s+base, [C,2C) -> 2s+1+base
  EPI_PHASE = 3,   // up-conv phase (py,px): voxel (y,x) -> (2y+py, 2x+px)
  EPI_VIDEO = 4,   // head: 2x2 pixel shuffle of 12 channels, clamp, NCTHW video
  EPI_WINO = 5,    // Winograd-domain product M[xi] (fp16, no bias): out + xi * out_pstride
  EPI_LATENT = 6   // encoder head: fp32 NCTHW latents, channel n of frame f -> [n][out_base + f]
                   // of a clip of video_T frames (generic kernel only)
};

// Spatial tap codes of a K segment (ConvSeg::KS).
enum SpatialTaps {
  KS_1x1 = 1,    // 1x1
  KS_PHASE = 2,  // 2x2 phase taps of an up-conv
  KS_3x3 = 3,    // 3x3, pad 1
  KS_3x1 = 4     // 3 rows x 1 column, row pad 1 (the Winograd-domain GEMM along x)
};

// One K segment of the implicit GEMM: a (possibly normalised) input tensor,
// its temporal history and the weights that contract it.
struct ConvSeg {
  const h16_t* x;           // input frame 0 of this pass, voxel stride lda
  const h16_t* ring;        // [2][H][W][Cin] previous input frames (raw) or null
  const float* rs;          // [2+F][H][W] per-voxel 1/||x|| (slot 2+f = frame f)
  const float* gamma;       // [Cin] gamma * sqrt(Cin) (norm prologues)
  const h16_t* w;           // wfrag: prepared fragment-major weights; else row-major [rows][ldw]
  long long x_fstride;      // elements per input frame
  long long w_tap_stride;   // elements per tap
  long long w_frame_stride; // per-frame weight offset (attention GEMMs), else 0
  int lda, ldw, Cin;
  int KT;                   // temporal taps: 1 or 3 (causal, history frames first)
  int KS;                   // spatial taps (SpatialTaps)
  int n_hist;               // valid history frames in ring (0..2)
  int prologue;             // Prologue
  int wfrag;                // 1: w is in MFMA fragment order (see launch_prep_frag)
  long long w_bytes;        // bytes of w (fragment order: bounds of the buffer loads)
  long long x_pstride;      // per-phase input offset (Winograd xi planes), else 0
  int stride;               // spatial stride: 0 or 1, or 2 (the encoder's down-convs: the
                            // input grid is 2H x 2W, output voxel (y, x) reads input
                            // rows 2y-1..2y+1 and columns 2x-1..2x+1; generic kernel,
                            // one frame, KT = 1, raw input)
};

struct ConvArgs {
  ConvSeg seg[2];
  int nseg;
  int F, H, W;              // output voxel grid (input grid for phase mode)
  int TF, TH, TW;           // tile frames / rows / columns (TW = kTileW except the Winograd GEMM's 8)
  int tiles_x, tiles_y, tiles_f;
  int nphase;               // 4 for EPI_PHASE and EPI_WINO (xi), else 1
  int Cout;
  const float* bias;        // [Cout] fp32 or null
  float scale;
  const h16_t* res;         // fp16 residual on the output grid, or null
  long long res_fstride;
  int ldr;
  void* out;
  long long out_fstride;
  long long out_pstride;    // EPI_WINO: elements per xi plane of the output
  int ldo;
  int epi;
  int out_base;             // EPI_TIME frame base; EPI_VIDEO first frame index
  int video_T;              // EPI_VIDEO total frames of the video
  int nhv_max;              // halo rows per LDS buffer (>= every segment's item rows)
  int bn;                   // Winograd-domain GEMM: output channels per tile, 256 (or 0) or 128
  const h16_t* zero_row;    // zero_len fp16 zeros: source of padding voxels
  int zero_len;             // >= every segment's Cin
};

// Host-validation mode: every launcher checks its arguments and returns
// without enqueuing GPU work (lets the whole schedule run without a GPU).
extern bool g_dry_run;

// nullptr when the launch of `a` satisfies what the kernel assumes, else the
// violated condition.
const char* conv_check(const ConvArgs& a);
// Launches one implicit-GEMM convolution; returns hipSuccess or the error.
hipError_t launch_conv(const ConvArgs& a, hipStream_t stream);
// True when `a` runs on the persistent kernel (one workgroup per CU walking
// tiles) rather than one workgroup per tile.
bool conv_persistent(const ConvArgs& a);
// LDS bytes the launch of `a` needs (host-side check).
size_t conv_lds_bytes(const ConvArgs& a);
// Whether `a` runs on the specialised 3x3x3 kernel.
bool conv_is_333(const ConvArgs& a);
// Whether `a` runs on the dominant instantiation: 8-wave 3x3x3 with the fused
// RMSNorm+SiLU prologue (every ResBlock conv of width >= 256).
bool conv_is_main(const ConvArgs& a);

// out[m][n] = sum_k x[m][k] w[n][k] + bias[n] for the M rows of x (stride
// lda) with fragment-order weights (taps = 1); N a multiple of 256, K of 64.
hipError_t launch_gemm1x1(const h16_t* x, long long M, int lda, int K, const h16_t* w, long long w_bytes, int N,
                          const float* bias, h16_t* out, int ldo, hipStream_t stream);

// Auxiliary kernels (wvd_aux.hip).
hipError_t launch_rms_stats(const h16_t* x, long long x_fstride, int lda, const h16_t* ring,
                            int n_hist, int C, int F, int HW, float* rs, hipStream_t s);
// y = SiLU(x / ||x|| * gamma) per voxel over C channels (gamma carries sqrt(C));
// without act, y = x / ||x|| * gamma.
hipError_t launch_norm_silu(const h16_t* x, long long x_fstride, int lda, int C, int F, int HW, const float* gamma,
                            h16_t* y, long long y_fstride, int ldy, hipStream_t s, bool act = true);
// Attention operands of F frames of qkv [F][L][3C] in fragment order (Np keys,
// a multiple of 256, zero past L): kf [F][Np x C], vf [F][C x Np].
hipError_t launch_attn_frag(const h16_t* qkv, int F, int L, int C, int Np, h16_t* kf, h16_t* vf, hipStream_t s);
// Softmax of the score rows from the score pass's output: row r of
// P[rows][np] (fp16) holds e^(s - m_g) for its columns in group g of 64 and
// st[r][g] = (m_g, sum of those e^(s - m_g)) (float2 as two floats, np / 64
// groups).  With the row's maximum M = max m_g and sum S = sum_g
// st.y e^(m_g - M), every value becomes e^(s - m_g) e^(m_g - M) / S in place.
hipError_t launch_attn_rescale(h16_t* P, const float* st, long long rows, int np, hipStream_t s);

// Batched NT GEMM on fragment-order B (the persistent 256 x 256 kernel of
// the 1x1 shortcut): for frames f < nF, out[f][m][n] = epilogue of
// sum_k x[f][m][k] w[f][n][k], M rows (>= 256) per frame, K a multiple of
// 128, N of 256.
enum GemmEpi {
  G_H16 = 0,   // fp16 out = acc * scale + bias (+ res, which may alias out)
  G_STATS = 1  // per row and group g of 64 columns, of v = acc * scale over the columns < n_valid:
               // m_g = max v and the fp16 out = e^(v - m_g) (0 for columns >= n_valid), and
               // (m_g, sum of e^(v - m_g)) into stats [f][M][N / 64] (float2)
};
struct GemmArgs {
  const h16_t* x;
  long long M;
  int lda, K;
  const h16_t* w;
  long long w_bytes;  // per frame
  int N;
  const float* bias;
  float scale;
  const h16_t* res;
  int ldr;
  h16_t* out;
  int ldo;
  int nF;
  long long a_fs, w_fs, o_fs, r_fs;  // per-frame strides (elements)
  int n_valid;
  float* stats;
};
hipError_t launch_gemm_nt(const GemmArgs& g, int epi, hipStream_t stream);
hipError_t launch_ring_update(h16_t* ring, const h16_t* x, long long x_fstride, int lda, int C,
                              int F, int HW, hipStream_t s);
// Deep variant: 48 -> 48 1x1x1 conv of the 64-wide channels-last latents.
hipError_t launch_pre_conv(const h16_t* zt, long long nvox, const float* A, const float* b, h16_t* zp,
                           hipStream_t s);
hipError_t launch_latent_to_cl(const void* z, int dtype, int T, int t0, int F, int HW, h16_t* zt, hipStream_t s);
hipError_t launch_copy16(void* dst, const void* src, size_t bytes, hipStream_t s);
// Zero-fills bytes (a multiple of 16) with a kernel (no memset node).
hipError_t launch_fill_zero(void* dst, size_t bytes, hipStream_t s);
hipError_t launch_softmax_rows(const float* S, int rows, int L, int Lpad, h16_t* P, hipStream_t s);
hipError_t launch_transpose_v(const h16_t* qkv, int F, int L, int C, int Lpad, h16_t* vt, hipStream_t s);
// Prepare-time kernels.
// Weights arrive as bf16 or fp32 (dtype); conv weights leave as fp16 in MFMA
// fragment order, vectors as fp32.  Fragment order: for output-channel block
// nb (32 channels), input-channel block u (16 channels) and tap t, one block
// of 512 halves at ((nb * U + u) * taps + t) * 512 in which lane l holds, at
// l * 8 .. l * 8 + 7, W[t][nb*32 + l%32][u*16 + (l/32)*8 + 0..7] (zero
// outside cout x cin; output channels are padded to a multiple of 128).
// U = cin_pad / 16; bytes = ceil(cout/128)*128*cin_pad*taps*2.
size_t prep_frag_bytes(int cout, int cin_pad, int taps);
hipError_t launch_prep_frag(const void* w, int dtype, int cout, int cin, int taps, int cin_pad, h16_t* out,
                            hipStream_t s);
// The same for input channels [cin_off, cin_off + cin) of a tensor with
// cin_src input channels (one operand of a conv split into K segments).
hipError_t launch_prep_frag_part(const void* w, int dtype, int cout, int cin_src, int cin_off, int cin, int taps,
                                 int cin_pad, h16_t* out, hipStream_t s);
// Encoder input: video [3][T][2H][2W] (bf16 or fp32; NCTHW without the batch)
// frames t0..t0+F-1 -> channels-last fp16 [F][H][W][kEncInC], channel
// 4k+2dy+dx = pixel (2Y+dy, 2X+dx) of colour k (the inverse of the 2x2 pixel
// shuffle), channels 12..kEncInC-1 zero.
hipError_t launch_patchify(const void* video, int dtype, int T, int t0, int F, int H, int W, h16_t* out,
                           hipStream_t s);
// Up-conv phase weights in the same fragment order with taps = 16
// (phase * 4 + 2x2 tap).
hipError_t launch_prep_phase_frag(const void* w, int dtype, int C, h16_t* out, hipStream_t s);
// Weights of a 3x3 stride-2 conv for its space-to-depth form (C -> C over 4C
// input channels, 2x2 taps at offsets -1, 0; fragment order, tap = 2a + b).
hipError_t launch_prep_s2d_frag(const void* w, int dtype, int C, h16_t* out, hipStream_t s);
// The head's 12 x cin x 27 weights with the x taps in the output columns
// (column 12 dx + co of (dt, dy) tap 3 dt + dy; 64 columns, 36 used) in
// fragment order, prep_frag_bytes(64, cin, 9) bytes; cin a multiple of 32.
hipError_t launch_prep_headx_frag(const void* w, int dtype, int cin, h16_t* out, hipStream_t s);
// x [F][H][W][C] -> y [F][H/2][W/2][4C], block 2 py + px = x[2Y+py][2X+px].
hipError_t launch_space_to_depth(const h16_t* x, long long x_fstride, int C, int F, int H, int W, h16_t* y,
                                 hipStream_t s);
// Winograd F(kWinoM,3) weights of a 3x3x3 conv along x: for each (dt, dy)
// the three x taps g become V = G g (fp32, rounded once to fp16), in
// fragment order with taps = kWinoN * 9 (xi * 9 + dt * 3 + dy).
hipError_t launch_prep_wino_frag(const void* w, int dtype, int cout, int cin, h16_t* out, hipStream_t s);

// Winograd F(m,3) (m = kWinoM) along x of the normalised input: for slots
// s = 0..F+1 (s = 0, 1: the two history frames in `ring`, only the last
// n_hist valid; s >= 2: frame s-2 of x), every column group q and channel,
//   y_k = SiLU(x[mq-1+k] * rs * gamma)  (k = 0..m+1, zero outside 0..W-1)
//   U[xi][s][row][q] = (B^T y)[xi]   (fp16)
// U is [kWinoN][F+2][H][WQ][C] with WQ = ceil(W/m); rs as rms_stats writes it.
hipError_t launch_wino_in(const h16_t* x, long long x_fstride, int lda, const h16_t* ring, int n_hist, int C, int F,
                          int H, int W, const float* gamma, h16_t* U, hipStream_t s, bool history_only = false);
// Output transform of conv1's products fused with conv2's input transform
// (C <= 512): U slots 2..F+1 of conv2, h written for frames >= tail_from.
bool wino_mid_ok(int C);
// Tile shapes (TF frames x TW column groups) of the Winograd-domain GEMM.
bool wino_tile_shape_ok(int TF, int TW);
hipError_t launch_wino_mid(const h16_t* M, const float* bias, int C, int F, int H, int W, const float* gamma,
                           h16_t* U, h16_t* hout, long long h_fstride, int ldh, int tail_from, int h_first,
                           hipStream_t s);
// Output transform: out[f][row][mq + j] = (A^T M)[j] + bias (+ res), with
// M = [kWinoN][F][H][WQ][Cout] fp16; out may alias res.
// With rs != null also writes rs[2+f][row][col] = 1/||out voxel|| exactly as
// launch_rms_stats would for these frames.  With act_gamma != null (and no
// rs) it stores SiLU(v / ||v|| * act_gamma) of each rounded output voxel v
// instead, bit for bit as launch_norm_silu would from the stored v.
hipError_t launch_wino_out(const h16_t* M, int Cout, int F, int H, int W, const float* bias, const h16_t* res,
                           long long res_fstride, int ldr, h16_t* out, long long out_fstride, int ldo, float* rs,
                           const float* act_gamma, hipStream_t s);
hipError_t launch_prep_vec(const void* v, int dtype, int n, float scale, float* out, hipStream_t s);
// out[i] = a[i] + b[i] in fp32 (the two biases of a block with a shortcut).
hipError_t launch_prep_vec_add(const void* a, const void* b, int dtype, int n, float* out, hipStream_t s);

// silu_hw and exp_hw of n fp32 inputs (math self-test).
hipError_t launch_math_probe(const float* x, float* silu_out, float* exp_out, long long n, hipStream_t s);
hipError_t launch_f16_probe(const float* x, uint16_t* h_out, float* rs_out, long long n, hipStream_t s);

// Device addresses of the range flags (see g_range_flags) of the two kernel
// code objects on the current device.
hipError_t conv_range_flags_addr(unsigned int** p);
hipError_t aux_range_flags_addr(unsigned int** p);

}  // namespace wvd
