// Memory-bound helper kernels of the wvd decoder: per-voxel RMS statistics,
// temporal-cache ring updates, latent layout transform, frame copies, the
// attention softmax and V transpose, and the one-time weight transforms.
#include "wvd_internal.h"

namespace wvd {

// No implicit multiply-add fusion in this file: a value that two kernels
// compute (a voxel's norm statistic, the Winograd input transform of a
// history frame and of the same frame inside a pass) must round the same
// way in both, whatever the surrounding code lets the compiler fuse.  The
// fused multiply-adds are written out (fmaf) where they are meant.
#pragma clang fp contract(off)

bool g_dry_run = false;

namespace {

constexpr float kNormEps = 1e-12f;

// rs[slot][pix] = 1 / max(||x_voxel||, eps) over the C channels of a voxel,
// for slots 0,1 = the two history frames held in `ring` (only the last
// n_hist are valid) and slots 2.. = the F frames of the pass.  G lanes share
// a voxel; lane sums run over channel groups of 8 in increasing order, then a
// fixed butterfly combines the G lanes, so the value of a voxel never depends
// on where or when it is computed (fp32 statistics: Wan2.2 VAE decoder page,
// "Limits").
// Each wave takes kStatsU voxel sets per trip and issues all of their loads
// before reducing any, so enough 16-byte loads are in flight to stream HBM.
constexpr int kStatsU = 4;
__global__ __launch_bounds__(256) void rms_stats_kernel(const h16_t* __restrict__ x, long long x_fstride,
                                                        int lda, const h16_t* __restrict__ ring,
                                                        int n_hist, int C, int F, int HW, int G,
                                                        float* __restrict__ rs) {
  const int lane = threadIdx.x & 63;
  const int sub = lane % G;
  const int vox_per_wave = 64 / G;
  const long long gw = ((long long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const long long nw = ((long long)gridDim.x * blockDim.x) >> 6;
  const int first_slot = 2 - n_hist;
  const long long nvox = (long long)(F + n_hist) * HW;
  // G is the largest power of two <= C / 8 (at most 64, and C <= 1024), so a
  // lane holds one or two of the voxel's 8-channel groups: sub and sub + G.
  const bool second = sub + G < (C >> 3);
  const long long step = (long long)vox_per_wave * kStatsU;
  for (long long base = gw * step; base < nvox; base += nw * step) {
    uint4 r[kStatsU][2];
    long long slot[kStatsU], pix[kStatsU];
    bool ok[kStatsU];
#pragma unroll
    for (int u = 0; u < kStatsU; ++u) {
      const long long vv = base + (long long)u * vox_per_wave + lane / G;
      ok[u] = vv < nvox;
      slot[u] = ok[u] ? vv / HW + first_slot : 2;
      pix[u] = ok[u] ? vv % HW : 0;
      const h16_t* p = slot[u] < 2 ? ring + (slot[u] * HW + pix[u]) * C : x + (slot[u] - 2) * x_fstride + pix[u] * lda;
      r[u][1] = make_uint4(0, 0, 0, 0);
      if (ok[u]) {
        r[u][0] = *reinterpret_cast<const uint4*>(p + sub * 8);
        if (second) r[u][1] = *reinterpret_cast<const uint4*>(p + (sub + G) * 8);
      } else {
        r[u][0] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < kStatsU; ++u) {
      float ss = 0.0f;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float f[8];
        unpack8h(r[u][q], f);
        float t = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) t = fmaf(f[k], f[k], t);
        ss += t;
      }
      for (int off = 1; off < G; off <<= 1) ss += __shfl_xor(ss, off, 64);
      if (ok[u] && sub == 0) rs[slot[u] * HW + pix[u]] = 1.0f / fmaxf(sqrtf(ss), kNormEps);
    }
  }
}

// Sum of v over aligned groups of G lanes (G a power of two <= 64), the
// same value, added in the same order, in every lane of a group: DPP steps
// pair lanes within rows of 16 (xor 1, xor 2, then mirrored halves of 8 and
// of 16), cross-lane permutes take the rows of 32 and 64.
__device__ __forceinline__ float dpp_f32(float a, int ctrl) {
  const int x = __builtin_bit_cast(int, a);
  switch (ctrl) {
    case 0: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
    case 1: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
    case 2: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false));
    default: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false));
  }
}

__device__ __forceinline__ float lane_group_sum(float v, int G) {
  if (G >= 2) v += dpp_f32(v, 0);   // quad_perm [1,0,3,2]
  if (G >= 4) v += dpp_f32(v, 1);   // quad_perm [2,3,0,1]
  if (G >= 8) v += dpp_f32(v, 2);   // row_half_mirror
  if (G >= 16) v += dpp_f32(v, 3);  // row_mirror
  if (G >= 32) v += __shfl_xor(v, 16, 64);
  if (G >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// y = SiLU(x * rs * gamma) (ACT) or x * rs * gamma for the F frames of a
// pass, rs from the voxel's channel norm exactly as rms_stats_kernel computes
// it (same lane split; the DPP butterfly adds the same two partials at every
// level as its shuffles, so the sums are identical).  Used where a norm-SiLU
// input feeds a conv with few output channels (the head) and for the
// attention's norm, so every voxel is normalised once instead of once per
// halo that contains it.  The arithmetic per element is the conv prologue's.
template <bool ACT>
__global__ __launch_bounds__(256) void norm_silu_kernel(const h16_t* __restrict__ x, long long x_fstride, int lda,
                                                        int C, int F, int HW, int G,
                                                        const float* __restrict__ gamma, h16_t* __restrict__ y,
                                                        long long y_fstride, int ldy) {
  const int lane = threadIdx.x & 63;
  const int sub = lane % G;
  const int vox_per_wave = 64 / G;
  const int gw = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nw = (gridDim.x * blockDim.x) >> 6;
  const int nvox = F * HW;  // (the launcher checks the range)
  const bool second = sub + G < (C >> 3);
  const int step = vox_per_wave * kStatsU;
  float gm[2][8];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int k = 0; k < 8; ++k) gm[q][k] = q == 0 || second ? gamma[(sub + q * G) * 8 + k] : 0.0f;
  for (int base = gw * step; base < nvox; base += nw * step) {
    uint4 r[kStatsU][2];
    int fr[kStatsU], pix[kStatsU];
    bool ok[kStatsU];
#pragma unroll
    for (int u = 0; u < kStatsU; ++u) {
      const int vv = base + u * vox_per_wave + lane / G;
      ok[u] = vv < nvox;
      fr[u] = ok[u] ? vv / HW : 0;
      pix[u] = ok[u] ? vv % HW : 0;
      const h16_t* p = x + fr[u] * x_fstride + (long long)pix[u] * lda;
      r[u][0] = make_uint4(0, 0, 0, 0);
      r[u][1] = make_uint4(0, 0, 0, 0);
      if (ok[u]) {
        r[u][0] = *reinterpret_cast<const uint4*>(p + sub * 8);
        if (second) r[u][1] = *reinterpret_cast<const uint4*>(p + (sub + G) * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < kStatsU; ++u) {
      float ss = 0.0f;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float f[8];
        unpack8h(r[u][q], f);
        float t = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) t = fmaf(f[k], f[k], t);
        ss += t;
      }
      ss = lane_group_sum(ss, G);
      const float sc = 1.0f / fmaxf(sqrtf(ss), kNormEps);
      if (!ok[u]) continue;
      h16_t* o = y + fr[u] * y_fstride + (long long)pix[u] * ldy;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (q == 1 && !second) break;
        const int g8 = (sub + q * G) * 8;
        float f[8];
        unpack8h(r[u][q], f);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float t = f[k] * sc * gm[q][k];
          f[k] = ACT ? silu_hw(t) : t;
        }
        *reinterpret_cast<uint4*>(o + g8) = pack8h_int(f);
      }
    }
  }
}

// ring <- the last two frames of [ring[0], ring[1], x[0..F-1]] (F >= 1).
__global__ __launch_bounds__(256) void ring_update_kernel(h16_t* __restrict__ ring, const h16_t* __restrict__ x,
                                                          long long x_fstride, int lda, int C, int F, int HW) {
  const int g8 = C >> 3;
  const long long n = (long long)HW * g8;
  const long long fs = (long long)HW * C;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x) {
    const long long pix = e / g8;
    const int g = (int)(e % g8);
    const long long ro = pix * C + g * 8;
    uint4 s1 = *reinterpret_cast<const uint4*>(x + (F - 1) * x_fstride + pix * lda + g * 8);
    uint4 s0 = F >= 2 ? *reinterpret_cast<const uint4*>(x + (F - 2) * x_fstride + pix * lda + g * 8)
                      : *reinterpret_cast<const uint4*>(ring + fs + ro);
    *reinterpret_cast<uint4*>(ring + ro) = s0;
    *reinterpret_cast<uint4*>(ring + fs + ro) = s1;
  }
}

// Deep variant's 1x1x1 conv on the latents: zp[v][o] = b[o] + sum_i A[o][i]
// zt[v][i] for the 48 latent channels (fp32 accumulation in channel order,
// fp16 store); channels 48..63 of the 64-wide layout stay zero.  One thread
// per (voxel, 8 output channels).
__global__ __launch_bounds__(256) void pre_conv_kernel(const h16_t* __restrict__ zt, long long nvox,
                                                       const float* __restrict__ A, const float* __restrict__ b,
                                                       h16_t* __restrict__ zp) {
  const long long n = nvox * 8;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x) {
    const long long v = e >> 3;
    const int og = (int)(e & 7);
    uint4 r = make_uint4(0, 0, 0, 0);
    if (og < 6) {
      float f[48];
#pragma unroll
      for (int q = 0; q < 6; ++q) unpack8h(*reinterpret_cast<const uint4*>(zt + v * 64 + q * 8), f + q * 8);
      float o[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int oc = og * 8 + k;
        float acc = b[oc];
        for (int i = 0; i < 48; ++i) acc += A[oc * 48 + i] * f[i];
        o[k] = acc;
      }
      r = pack8h(o);
    }
    *reinterpret_cast<uint4*>(zp + v * 64 + og * 8) = r;
  }
}

// z [48][T][HW] (bf16 or fp32) frames t0..t0+F-1 -> zt [F][HW][64] fp16
// (channels 48..63 zero).
__global__ __launch_bounds__(256) void latent_to_cl_kernel(const void* __restrict__ z, int dtype, int T, int t0,
                                                           int F, int HW, h16_t* __restrict__ zt) {
  const long long n = (long long)F * HW;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x) {
    const long long f = e / HW, pix = e % HW;
    uint32_t w[32];
#pragma unroll
    for (int c2 = 0; c2 < 32; ++c2) {
      const int c = 2 * c2;
      uint32_t lo = 0, hi = 0;
      if (c < 48) {
        lo = f2h(load_in(z, ((long long)c * T + t0 + f) * HW + pix, dtype));
        hi = f2h(load_in(z, ((long long)(c + 1) * T + t0 + f) * HW + pix, dtype));
      }
      w[c2] = lo | (hi << 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(zt + e * 64);
#pragma unroll
    for (int q = 0; q < 8; ++q) dst[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
  }
}

// Attention operands in MFMA fragment order, per frame f of qkv [F][L][3C]
// (q | k | v thirds): kf = the keys as the "weights" of S = Q K^T (N = Np
// keys, K = C), vf = V^T as the weights of O = P V (N = C, K = Np keys).
// Block (nb, u) of 512 halves: lane l holds at l*8..l*8+7 row nb*32 + l%32
// and columns u*16 + (l/32)*8 + 0..7 of the N x K operand; keys >= L are 0.
__global__ __launch_bounds__(256) void attn_frag_kernel(const h16_t* __restrict__ qkv, int L, int C, int Np,
                                                        h16_t* __restrict__ kf, h16_t* __restrict__ vf) {
  const int f = blockIdx.y;
  const h16_t* q = qkv + (long long)f * L * 3 * C;
  const long long nk = (long long)(Np / 32) * (C / 16) * 64;  // 16-byte pieces of kf per frame
  const long long nv = (long long)(C / 32) * (Np / 16) * 64;
  h16_t* kff = kf + (long long)f * Np * C;
  h16_t* vff = vf + (long long)f * Np * C;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < nk + nv;
       e += (long long)gridDim.x * blockDim.x) {
    if (e < nk) {
      const int l = (int)(e & 63);
      const long long blk = e >> 6;
      const int U = C / 16;
      const int u = (int)(blk % U), nb = (int)(blk / U);
      const int key = nb * 32 + (l & 31), d0 = u * 16 + (l >> 5) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (key < L) v = *reinterpret_cast<const uint4*>(q + (long long)key * 3 * C + C + d0);
      *reinterpret_cast<uint4*>(kff + e * 8) = v;
    } else {
      const long long ev = e - nk;
      const int l = (int)(ev & 63);
      const long long blk = ev >> 6;
      const int U = Np / 16;
      const int u = (int)(blk % U), nb = (int)(blk / U);
      const int d = nb * 32 + (l & 31), key0 = u * 16 + (l >> 5) * 8;
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k0 = key0 + 2 * j, k1 = k0 + 1;
        const uint32_t lo = k0 < L ? q[(long long)k0 * 3 * C + 2 * C + d] : 0u;
        const uint32_t hi = k1 < L ? q[(long long)k1 * 3 * C + 2 * C + d] : 0u;
        w[j] = lo | (hi << 16);
      }
      *reinterpret_cast<uint4*>(vff + ev * 8) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// One wave per score row r: the row's maximum M over the partial maxima
// m_g of its groups of 64 keys, S = sum_g l_g e^(m_g - M) from the groups'
// (m_g, l_g), then each fp16 value e^(s - m_g) of group g is scaled by
// e^(m_g - M) / S in place.  A group whose keys are all padding has l_g = 0
// and scale 0 (its values are zero already).
__global__ __launch_bounds__(256) void attn_rescale_kernel(h16_t* __restrict__ P, const float2* __restrict__ st,
                                                           long long rows, int np) {
  const int lane = threadIdx.x & 63;
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int nst = np / 64;
  const float2* sr = st + r * nst;
  float m = -INFINITY;
  for (int g = lane; g < nst; g += 64) m = fmaxf(m, sr[g].x);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
  float l = 0.0f;
  for (int g = lane; g < nst; g += 64) {
    const float2 p = sr[g];
    if (p.y > 0.0f) l += p.y * exp_hw(p.x - m);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) l += __shfl_xor(l, d, 64);
  const float inv = 1.0f / l;
  uint4* row = reinterpret_cast<uint4*>(P + r * np);
  for (int q = lane; q < np / 8; q += 64) {
    const float2 p = sr[q >> 3];
    const float f = p.y > 0.0f ? exp_hw(p.x - m) * inv : 0.0f;
    float v[8];
    unpack8h(row[q], v);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] *= f;
    row[q] = pack8h(v);
  }
}

// Encoder input: frames t0.. of the video [3][T][2H][2W] -> [F][H][W][16]
// fp16 with channel 4k + 2dy + dx = pixel (2Y+dy, 2X+dx) of colour k (the
// inverse of the decoder's pixel shuffle) and channels 12..15 zero.
__global__ __launch_bounds__(256) void patchify_kernel(const void* __restrict__ v, int dtype, int T, int t0, int F,
                                                       int H, int W, h16_t* __restrict__ out) {
  const long long n = (long long)F * H * W;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x) {
    const int X = (int)(e % W);
    const int Y = (int)((e / W) % H);
    const long long f = e / ((long long)W * H);
    float c[16];
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const long long row = ((long long)k * T + t0 + f) * (2 * H) + 2 * Y + (d >> 1);
        c[4 * k + d] = load_in(v, row * (2 * W) + 2 * X + (d & 1), dtype);
      }
#pragma unroll
    for (int k = 12; k < 16; ++k) c[k] = 0.0f;
    static_assert(kEncInC == 32, "12 patch channels and 20 zeros");
    uint4* dst = reinterpret_cast<uint4*>(out + e * kEncInC);
    dst[0] = pack8h(c);
    dst[1] = pack8h(c + 8);
    dst[2] = make_uint4(0, 0, 0, 0);
    dst[3] = make_uint4(0, 0, 0, 0);
  }
}

__global__ __launch_bounds__(256) void copy16_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src, long long n) {
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x)
    dst[e] = src[e];
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* __restrict__ dst, long long n) {
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x)
    dst[e] = make_uint4(0, 0, 0, 0);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// One wave per row: P = softmax(S) over the L valid columns (max-subtracted,
// fp32), written as fp16 with zeros in columns L..Lpad-1.
__global__ __launch_bounds__(256) void softmax_rows_kernel(const float* __restrict__ S, int rows, int L, int Lpad,
                                                           h16_t* __restrict__ P) {
  const int lane = threadIdx.x & 63;
  const long long row = ((long long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  if (row >= rows) return;
  const float* s = S + row * Lpad;
  float mx = -INFINITY;
  for (int j = lane; j < L; j += 64) mx = fmaxf(mx, s[j]);
  mx = wave_max(mx);
  float sum = 0.0f;
  for (int j = lane; j < L; j += 64) sum += exp_hw(s[j] - mx);
  sum = wave_sum(sum);
  const float inv = 1.0f / sum;
  h16_t* p = P + row * Lpad;
  for (int j = lane; j < Lpad; j += 64) p[j] = j < L ? (h16_t)f2h(exp_hw(s[j] - mx) * inv) : (h16_t)0;
}

// V^T per frame: vt[f][c][l] = qkv[f][l][2C + c], zero for l >= L.
__global__ __launch_bounds__(256) void transpose_v_kernel(const h16_t* __restrict__ qkv, int L, int C, int Lpad,
                                                          h16_t* __restrict__ vt) {
  __shared__ h16_t tile[64][65];
  const int f = blockIdx.z;
  const int l0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const h16_t* src = qkv + (long long)f * L * 3 * C + 2 * C;
  h16_t* dst = vt + (long long)f * C * Lpad;
  for (int k = threadIdx.x; k < 64 * 64; k += 256) {
    const int r = k / 64, cc = k % 64;  // r: token, cc: channel
    const int l = l0 + r, c = c0 + cc;
    tile[r][cc] = (l < L && c < C) ? src[(long long)l * 3 * C + c] : (h16_t)0;
  }
  __syncthreads();
  for (int k = threadIdx.x; k < 64 * 64; k += 256) {
    const int r = k / 64, ll = k % 64;  // r: channel, ll: token
    const int c = c0 + r, l = l0 + ll;
    if (c < C && l < Lpad) dst[(long long)c * Lpad + l] = tile[ll][r];
  }
}

// Fragment-order conv weights (layout in wvd_internal.h) from the PyTorch
// layout w[o][i][tap] (taps flattened).
__global__ void prep_frag_kernel(const void* __restrict__ w, int dtype, int cout, int cin_src, int cin_off, int cin,
                                 int taps, int cin_pad, h16_t* __restrict__ out) {
  const int NB = (cout + 127) / 128 * 4, U = cin_pad / 16;
  const long long n = (long long)NB * U * taps * 512;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x) {
    const int j = (int)(e & 7);
    const int l = (int)((e >> 3) & 63);
    const long long blk = e >> 9;
    const int t = (int)(blk % taps);
    const int u = (int)((blk / taps) % U);
    const int nb = (int)(blk / ((long long)taps * U));
    const int o = nb * 32 + (l & 31);
    const int i = u * 16 + (l >> 5) * 8 + j;
    out[e] = (o < cout && i < cin)
                 ? (h16_t)f2h(load_in(w, ((long long)o * cin_src + cin_off + i) * taps + t, dtype))
                 : (h16_t)0;
  }
}

// The head's 3x3x3 conv (12 output channels) with its three x taps moved
// into the output columns: column n = 12 dx + co (n < 36; the rest zero) of
// the (dt, dy) tap t = 3 dt + dy holds w[co][i][3 t + dx], so a GEMM over the
// nine (t, y) taps gives, per input column x, the partial sums
// P[x][12 dx + co] that the epilogue combines as out[x] = sum over dx of
// P[x + dx - 1][12 dx + co].  Fragment order with taps = 9 and 128 columns.
__global__ void prep_headx_frag_kernel(const void* __restrict__ w, int dtype, int cin, h16_t* __restrict__ out) {
  const int NB = 4, U = cin / 16;
  const long long n = (long long)NB * U * 9 * 512;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x) {
    const int j = (int)(e & 7);
    const int l = (int)((e >> 3) & 63);
    const long long blk = e >> 9;
    const int t = (int)(blk % 9);
    const int u = (int)((blk / 9) % U);
    const int nb = (int)(blk / (9LL * U));
    const int o = nb * 32 + (l & 31);
    const int i = u * 16 + (l >> 5) * 8 + j;
    out[e] = o < 36 ? (h16_t)f2h(load_in(w, ((long long)(o % 12) * cin + i) * 27 + t * 3 + o / 12, dtype))
                    : (h16_t)0;
  }
}

// Phase form of nearest-2x upsampling followed by a 3x3 conv (pad 1): output
// pixel (2i+py, 2j+px) is a 2x2 conv of the low-resolution input at rows
// i+py-1+a, cols j+px-1+b (a, b in {0,1}) whose weights are sums of the 3x3
// weights: rows {0} / {1,2} for py = 0 and {0,1} / {2} for py = 1 (same for
// columns).  Sums in fp32, rounded once to fp16; fragment order with
// tap = phase * 4 + a * 2 + b.
__global__ void prep_phase_frag_kernel(const void* __restrict__ w, int dtype, int C, h16_t* __restrict__ out) {
  const int NB = (C + 127) / 128 * 4, U = C / 16;
  const long long n = (long long)NB * U * 16 * 512;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x) {
    const int j = (int)(e & 7);
    const int l = (int)((e >> 3) & 63);
    const long long blk = e >> 9;
    const int t16 = (int)(blk % 16);
    const int u = (int)((blk / 16) % U);
    const int nb = (int)(blk / (16LL * U));
    const int o = nb * 32 + (l & 31);
    const int i = u * 16 + (l >> 5) * 8 + j;
    float s = 0.0f;
    if (o < C) {
      const int ph = t16 >> 2, tap = t16 & 3;
      const int py = ph >> 1, px = ph & 1, ta = tap >> 1, tb = tap & 1;
      const int ky0 = (py == 0) ? (ta == 0 ? 0 : 1) : (ta == 0 ? 0 : 2);
      const int ky1 = (py == 0) ? (ta == 0 ? 0 : 2) : (ta == 0 ? 1 : 2);
      const int kx0 = (px == 0) ? (tb == 0 ? 0 : 1) : (tb == 0 ? 0 : 2);
      const int kx1 = (px == 0) ? (tb == 0 ? 0 : 2) : (tb == 0 ? 1 : 2);
      const long long wp = ((long long)o * C + i) * 9;
      for (int ky = ky0; ky <= ky1; ++ky)
        for (int kx = kx0; kx <= kx1; ++kx) s += load_in(w, wp + ky * 3 + kx, dtype);
    }
    out[e] = (h16_t)f2h(s);
  }
}

// Weights of a 3x3 stride-2 conv (pad 1) for its space-to-depth form: the
// input's four phase images (py, px) = (row, column parity) side by side in
// channels, block b = 2 py + px holding input channels [b C, (b + 1) C), and
// a 2x2 conv over them at offsets -1, 0.  Along each axis, offset -1 reaches
// only the odd phase (kernel tap 0); offset 0 reaches the even phase (tap 1)
// and the odd one (tap 2).  Seven of the sixteen (tap, block) pairs are zero.
// Fragment order with tap = 2 a + b (a, b: offset + 1 in rows and columns).
__global__ void prep_s2d_frag_kernel(const void* __restrict__ w, int dtype, int C, h16_t* __restrict__ out) {
  const int NB = (C + 127) / 128 * 4, U = 4 * C / 16;
  const long long n = (long long)NB * U * 4 * 512;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x) {
    const int j = (int)(e & 7);
    const int l = (int)((e >> 3) & 63);
    const long long blk = e >> 9;
    const int t4 = (int)(blk % 4);
    const int u = (int)((blk / 4) % U);
    const int nb = (int)(blk / (4LL * U));
    const int o = nb * 32 + (l & 31);
    const int i4 = u * 16 + (l >> 5) * 8 + j;  // channel of the space-to-depth input
    const int b = i4 / C, c = i4 % C;
    const int py = b >> 1, px = b & 1, ta = t4 >> 1, tb = t4 & 1;
    const int ky = ta == 0 ? (py == 1 ? 0 : -1) : (py == 0 ? 1 : 2);
    const int kx = tb == 0 ? (px == 1 ? 0 : -1) : (px == 0 ? 1 : 2);
    float v = 0.0f;
    if (o < C && ky >= 0 && kx >= 0) v = load_in(w, ((long long)o * C + c) * 9 + ky * 3 + kx, dtype);
    out[e] = (h16_t)f2h(v);
  }
}

// Space-to-depth: y[f][Y][X][(2 py + px) C + c] = x[f][2Y + py][2X + px][c]
// (H and W even), 16 bytes per thread.
__global__ __launch_bounds__(256) void space_to_depth_kernel(const h16_t* __restrict__ x, long long x_fstride,
                                                             int C, int F, int H, int W, h16_t* __restrict__ y) {
  const int C8 = C / 8, H2 = H / 2, W2 = W / 2;
  const long long n = (long long)F * H2 * W2 * 4 * C8;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x) {
    const int g = (int)(e % C8);
    long long r = e / C8;
    const int b = (int)(r % 4);
    r /= 4;
    const int X = (int)(r % W2);
    r /= W2;
    const int Y = (int)(r % H2);
    const int f = (int)(r / H2);
    const int py = b >> 1, px = b & 1;
    const uint4 v =
        *reinterpret_cast<const uint4*>(x + f * x_fstride + ((long long)(2 * Y + py) * W + 2 * X + px) * C + g * 8);
    *reinterpret_cast<uint4*>(y + e * 8) = v;
  }
}

// Winograd F(m,3) along x (Lavin and Gray's minimal filtering): m outputs
// x[mq .. mq+m-1] of a 3-tap correlation (pad 1) come from the n = m + 2
// inputs d_k = x[mq-1+k]:
//   U = B^T d (input transform),  V = G g (weight transform),
//   M = sum over channels and (t, y) taps of U * V,  y = A^T M.
// The kernels run m = kWinoM = 6.
template <int WM>
struct Wino;

// F(6,3): interpolation points 0, 1, -1, 1/2, -1/2, 2, -2 and infinity
// (Toom-Cook).  Eight inputs d_k = x[6q-1+k] give six outputs x[6q..6q+5].
// The rows of G are scaled so that V has the magnitude of the taps (fp16
// weights stay out of the subnormal range), the matching factors 2/9, 32/45
// and 2/45 sit in the output transform, and the input transform keeps
// dyadic coefficients (exact in fp32).
template <>
struct Wino<6> {
  static constexpr int N = 8;
  __device__ static void weights(float g0, float g1, float g2, float* v) {
    v[0] = g0;
    v[1] = -(g0 + g1 + g2);
    v[2] = -(g0 - g1 + g2);
    v[3] = g0 + 0.5f * g1 + 0.25f * g2;
    v[4] = g0 - 0.5f * g1 + 0.25f * g2;
    v[5] = 0.25f * g0 + 0.5f * g1 + g2;
    v[6] = 0.25f * g0 - 0.5f * g1 + g2;
    v[7] = g2;
  }
  __device__ static void input(const float* d, float* u) {
    u[0] = fmaf(5.25f, d[4] - d[2], d[0] - d[6]);
    const float t1 = fmaf(-4.25f, d[4], d[2] + d[6]), t2 = fmaf(-4.25f, d[3], d[1] + d[5]);
    u[1] = t1 + t2;
    u[2] = t1 - t2;
    const float t3 = fmaf(-5.0f, d[4], fmaf(4.0f, d[2], d[6]));
    const float t4 = fmaf(0.5f, d[5], fmaf(-2.5f, d[3], 2.0f * d[1]));
    u[3] = t3 + t4;
    u[4] = t3 - t4;
    const float t5 = fmaf(-1.25f, d[4], fmaf(0.25f, d[2], d[6]));
    const float t6 = fmaf(2.0f, d[5], fmaf(-2.5f, d[3], 0.5f * d[1]));
    u[5] = t5 + t6;
    u[6] = t5 - t6;
    u[7] = fmaf(5.25f, d[3] - d[5], d[7] - d[1]);
  }
  __device__ static void output(const float* m, float* o) {
    constexpr float k29 = 2.0f / 9.0f, k45 = 1.0f / 45.0f;
    const float a = k29 * (m[1] + m[2]), b = k29 * (m[1] - m[2]);
    const float c = k45 * (m[3] + m[4]), d = k45 * (m[3] - m[4]);
    const float e = k45 * (m[5] + m[6]), f = k45 * (m[5] - m[6]);
    o[0] = m[0] + a + 32.0f * c + 2.0f * e;
    o[1] = b + 16.0f * d + 4.0f * f;
    o[2] = a + 8.0f * c + 8.0f * e;
    o[3] = b + 4.0f * d + 16.0f * f;
    o[4] = a + 2.0f * c + 32.0f * e;
    o[5] = b + d + 64.0f * f + m[7];
  }
};

// Winograd weights of a 3x3x3 conv: for each (o, i, dt, dy) the x taps
// g0..g2 become V = G g (fp32, rounded once to fp16), in fragment order with
// tap = xi * 9 + dt * 3 + dy.
__global__ void prep_wino_frag_kernel(const void* __restrict__ w, int dtype, int cout, int cin,
                                      h16_t* __restrict__ out) {
  constexpr int NX = Wino<kWinoM>::N;
  const int NB = (cout + 127) / 128 * 4, U = cin / 16;
  const long long n = (long long)NB * U * (NX * 9) * 512;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x) {
    const int j = (int)(e & 7);
    const int l = (int)((e >> 3) & 63);
    const long long blk = e >> 9;
    const int tx = (int)(blk % (NX * 9));
    const int u = (int)((blk / (NX * 9)) % U);
    const int nb = (int)(blk / ((long long)NX * 9 * U));
    const int o = nb * 32 + (l & 31);
    const int i = u * 16 + (l >> 5) * 8 + j;
    float v = 0.0f;
    if (o < cout && i < cin) {
      const int xi = tx / 9, tdy = tx % 9;  // tdy = dt * 3 + dy
      const long long wp = ((long long)o * cin + i) * 27 + tdy * 3;
      float vv[NX];
      Wino<kWinoM>::weights(load_in(w, wp, dtype), load_in(w, wp + 1, dtype), load_in(w, wp + 2, dtype), vv);
#pragma unroll
      for (int k = 0; k < NX; ++k)
        if (k == xi) v = vv[k];
    }
    out[e] = (h16_t)f2h(v);
  }
}

// Zeros that the transforms read in place of columns outside a row (no
// branch around the loads): at least as long as the widest channel count.
__device__ __align__(16) h16_t g_zero_row[1024];

// SiLU(v * rs * gamma) of one column from its fp16 channel values (this
// lane's NG 8-channel groups), with rs = 1 / ||v|| over the column's C
// channels (a sum over the G lanes of the group); zero where !in.  The
// Winograd input transforms take every activation through this function.
template <int NG>
__device__ __forceinline__ void act_column(const uint4 (&v)[NG], bool in, int G, const float (&gm)[NG][8],
                                           float (&y)[NG][8]) {
  float f[NG][8];
#pragma unroll
  for (int h = 0; h < NG; ++h) unpack8h(v[h], f[h]);
  float ss = 0.0f;
#pragma unroll
  for (int h = 0; h < NG; ++h) {
    float t = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) t = fmaf(f[h][k], f[h][k], t);
    ss += t;
  }
  ss = lane_group_sum(ss, G);
  // every activation of a Winograd conv's input comes from this function,
  // so the hardware rsqrt here (not the correctly rounded form of
  // rms_stats_kernel) is the same for every pass
  static_assert(kNormEps == 1e-12f, "norm_scale's floor");
  const float sc = norm_scale(ss);
  // SiLU first, then the select: a conditional expression with the SiLU
  // inside it becomes a branch per element pair
#pragma unroll
  for (int h = 0; h < NG; ++h)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float t = f[h][c] * sc * gm[h][c];
      const float a = silu_hw(t);
      y[h][c] = in ? a : 0.0f;
    }
}

// Input transform with its own norm statistics.  A group of G lanes (G the
// largest power of two <= min(64, C / 8)) takes a run of wino_in_run(NG) column
// groups of one row of one slot; lane sub holds the 8-channel groups sub and
// sub + G (when C / 8 > G).  Each column is loaded once: the lanes sum the
// squares of their channels, a reduction over the G lanes gives the voxel's
// 1/||x|| (the formula of rms_stats_kernel), and SiLU(x * rs *
// gamma) of the column enters a window of Wino<kWinoM>::N columns that
// slides by kWinoM per column group.  History slots (from the ring) and pass frames go through the
// same code, so a voxel's activation does not depend on which pass holds it.
// Column groups per run: two where a lane holds two channel groups (its
// window takes twice the registers, two waves per SIMD: more, shorter runs
// measured 11 % faster), else kWinoInRun.
constexpr int wino_in_run(int NG) { return NG == 2 ? 2 : kWinoInRun; }

template <int NG>  // 8-channel groups per lane: 1 (C <= 512) or 2
__global__ __launch_bounds__(256) void wino_in_kernel(const h16_t* __restrict__ x, long long x_fstride, int lda,
                                                      const h16_t* __restrict__ ring, int first_slot, int slot_end,
                                                      int C, int S, int H, int W, int WQ, int G,
                                                      const float* __restrict__ gamma, h16_t* __restrict__ U) {
  constexpr int WM = kWinoM, NX = Wino<WM>::N, R = wino_in_run(NG);
  const int lane = threadIdx.x & 63;
  const int sub = lane % G;
  const int G8 = C >> 3;
  const bool second = NG == 2 && sub + G < G8;  // this lane's second channel group exists
  const int QB = (WQ + R - 1) / R;   // runs of R column groups per row
  const long long HW = (long long)H * W;
  const long long plane = (long long)S * H * WQ * C;  // elements per xi plane
  const int nrun = (slot_end - first_slot) * H * QB;  // (the launcher checks the range)
  const int runs_per_wave = 64 / G;
  const int gw = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nw = (gridDim.x * blockDim.x) >> 6;
  float gm[NG][8];
#pragma unroll
  for (int h = 0; h < NG; ++h) {
    const int g = sub + h * G;
#pragma unroll
    for (int c = 0; c < 8; ++c) gm[h][c] = 0.0f;
    if (h == 0 || second) {
      const float4 g0 = *reinterpret_cast<const float4*>(gamma + g * 8);
      const float4 g1 = *reinterpret_cast<const float4*>(gamma + g * 8 + 4);
      gm[h][0] = g0.x; gm[h][1] = g0.y; gm[h][2] = g0.z; gm[h][3] = g0.w;
      gm[h][4] = g1.x; gm[h][5] = g1.y; gm[h][6] = g1.z; gm[h][7] = g1.w;
    }
  }
  for (int base = gw * runs_per_wave; base < nrun; base += nw * runs_per_wave) {
    const int e = base + lane / G;
    const bool ok = e < nrun;  // whole lane groups agree
    const int ee = ok ? e : 0;
    const int qb = ee % QB;
    const int r = ee / QB;
    const int row = r % H;
    const int slot = r / H + first_slot;
    const h16_t* src_row = slot < 2 ? ring + ((long long)slot * HW + (long long)row * W) * C
                                    : x + (slot - 2) * x_fstride + (long long)row * W * lda;
    const long long ld = slot < 2 ? C : lda;
    // SiLU(x * rs * gamma) of column `col` for this lane's channels (zero
    // outside the row); every lane of the group runs it (butterfly)
    // raw channels of column `col` (zero outside the row)
    auto load_col = [&](int col, uint4 (&v)[NG]) {
      const h16_t* p = ok && col >= 0 && col < W ? src_row + (long long)col * ld : g_zero_row;
      v[0] = *reinterpret_cast<const uint4*>(p + sub * 8);
      if (NG == 2) v[NG - 1] = *reinterpret_cast<const uint4*>(second ? p + (sub + G) * 8 : g_zero_row);
    };
    auto in_row = [&](int col) { return ok && col >= 0 && col < W; };
    float y[NX][NG][8];
    const int q0 = qb * R;
    {
      uint4 v[NX - WM][NG];
#pragma unroll
      for (int k = 0; k < NX - WM; ++k) load_col(WM * q0 - 1 + k, v[k]);
#pragma unroll
      for (int k = 0; k < NX - WM; ++k) act_column<NG>(v[k], in_row(WM * q0 - 1 + k), G, gm, y[k]);
    }
    // the columns a group adds to the window, loaded one group ahead so
    // the loads are in flight while the previous group is transformed
    uint4 raw[WM][NG];
#pragma unroll
    for (int k = 0; k < WM; ++k) load_col(WM * q0 + (NX - WM) - 1 + k, raw[k]);
    h16_t* dst = U + ((long long)slot * H * WQ + (long long)row * WQ + q0) * C;
#pragma unroll
    for (int qq = 0; qq < R; ++qq) {
      const int q = q0 + qq;
      if (q >= WQ) break;  // uniform over the lane group
#pragma unroll
      for (int k = 0; k < WM; ++k)
        act_column<NG>(raw[k], in_row(WM * q + (NX - WM) - 1 + k), G, gm, y[NX - WM + k]);
      if (qq + 1 < R) {
#pragma unroll
        for (int k = 0; k < WM; ++k) load_col(WM * (q + 1) + (NX - WM) - 1 + k, raw[k]);
      }
#pragma unroll
      for (int h = 0; h < NG; ++h) {
        if (h == 1 && !second) break;
        float u[NX][8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float d[NX], uu[NX];
#pragma unroll
          for (int k = 0; k < NX; ++k) d[k] = y[k][h][c];
          Wino<WM>::input(d, uu);
#pragma unroll
          for (int k = 0; k < NX; ++k) u[k][c] = uu[k];
        }
        if (ok) {
#pragma unroll
          for (int k = 0; k < NX; ++k)
            *reinterpret_cast<uint4*>(dst + qq * C + (sub + h * G) * 8 + k * plane) = pack8h(u[k]);
        }
      }
      // the last two columns of this window open the next one
#pragma unroll
      for (int k = 0; k < NX - WM; ++k)
#pragma unroll
        for (int h = 0; h < NG; ++h)
#pragma unroll
          for (int c = 0; c < 8; ++c) y[k][h][c] = y[WM + k][h][c];
    }
  }
}

// Output transform of one conv fused with the input transform of the next
// (conv1 -> conv2 of a ResBlock): from the planes of conv1's products,
// a run of kWinoInRun column groups gets h = A^T M + bias rounded to fp16
// (exactly the values the unfused path would store), each column is
// activated once through act_column, and the column window of conv2's
// input transform slides over them.  The window's outer columns come from
// the neighbouring groups (the last column of group q0 - 1, the first of
// q0 + R), so a run reads R + 2 groups of products.  h itself is written only
// for frames >= tail_from (the frames the next pass reads as history), frame
// f at hout + (f - h_first) * h_fstride.
template <int NG>
__global__ __launch_bounds__(256) void wino_mid_kernel(const h16_t* __restrict__ M, const float* __restrict__ bias,
                                                       int C, int F, int H, int W, int WQ, int G,
                                                       const float* __restrict__ gamma, h16_t* __restrict__ U,
                                                       h16_t* __restrict__ hout, long long h_fstride, int ldh,
                                                       int tail_from, int h_first) {
  constexpr int WM = kWinoM, NX = Wino<WM>::N, R = kWinoInRun;
  const int lane = threadIdx.x & 63;
  const int sub = lane % G;
  const int G8 = C >> 3;
  const bool second = NG == 2 && sub + G < G8;
  const int QB = (WQ + R - 1) / R;
  const long long mplane = (long long)F * H * WQ * C;        // conv1 product planes
  const long long uplane = (long long)(F + 2) * H * WQ * C;  // conv2 input planes (two history slots first)
  const int nrun = F * H * QB;  // (the launcher checks the range)
  const int runs_per_wave = 64 / G;
  const int gw = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nw = (gridDim.x * blockDim.x) >> 6;
  float gm[NG][8], bv[NG][8];
#pragma unroll
  for (int h = 0; h < NG; ++h) {
    const int g = sub + h * G;
#pragma unroll
    for (int c = 0; c < 8; ++c) gm[h][c] = bv[h][c] = 0.0f;
    if (h == 0 || second) {
      const float4 g0 = *reinterpret_cast<const float4*>(gamma + g * 8);
      const float4 g1 = *reinterpret_cast<const float4*>(gamma + g * 8 + 4);
      gm[h][0] = g0.x; gm[h][1] = g0.y; gm[h][2] = g0.z; gm[h][3] = g0.w;
      gm[h][4] = g1.x; gm[h][5] = g1.y; gm[h][6] = g1.z; gm[h][7] = g1.w;
      if (bias) {
        const float4 b0 = *reinterpret_cast<const float4*>(bias + g * 8);
        const float4 b1 = *reinterpret_cast<const float4*>(bias + g * 8 + 4);
        bv[h][0] = b0.x; bv[h][1] = b0.y; bv[h][2] = b0.z; bv[h][3] = b0.w;
        bv[h][4] = b1.x; bv[h][5] = b1.y; bv[h][6] = b1.z; bv[h][7] = b1.w;
      }
    }
  }
  for (int base = gw * runs_per_wave; base < nrun; base += nw * runs_per_wave) {
    const int e = base + lane / G;
    const bool ok = e < nrun;
    const int ee = ok ? e : 0;
    const int qb = ee % QB;
    const int r = ee / QB;
    const int row = r % H;
    const int f = r / H;
    // raw products of group q (zero outside: the zero row, plane stride 0)
    auto load_group = [&](int q, uint4 (&mr)[NX][NG]) {
      const bool valid = ok && q >= 0 && q < WQ;
      const h16_t* p = valid ? M + (long long)((f * H + row) * WQ + q) * C : g_zero_row;
      const long long ps = valid ? mplane : 0;
#pragma unroll
      for (int k = 0; k < NX; ++k)
#pragma unroll
        for (int h = 0; h < NG; ++h)
          mr[k][h] = *reinterpret_cast<const uint4*>(h == 0 || second ? p + k * ps + (sub + h * G) * 8 : g_zero_row);
    };
    // h (fp16, as stored) of the kWinoM columns of group q; zero outside
    auto finish_group = [&](int q, const uint4 (&mr)[NX][NG], uint4 (&hv)[WM][NG]) {
      const bool valid = ok && q >= 0 && q < WQ;
#pragma unroll
      for (int h = 0; h < NG; ++h) {
        float m[NX][8];
#pragma unroll
        for (int k = 0; k < NX; ++k) unpack8h(mr[k][h], m[k]);
        float o[WM][8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float mm[NX], oo[WM];
#pragma unroll
          for (int k = 0; k < NX; ++k) mm[k] = m[k][c];
          Wino<WM>::output(mm, oo);
#pragma unroll
          for (int e2 = 0; e2 < WM; ++e2) o[e2][c] = oo[e2];
        }
#pragma unroll
        for (int e2 = 0; e2 < WM; ++e2) {
          float v[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) v[c] = o[e2][c] + bv[h][c];
          hv[e2][h] = (valid && WM * q + e2 < W) ? pack8h(v) : make_uint4(0, 0, 0, 0);
        }
      }
    };
    const int q0 = qb * R;
    float y[NX][NG][8];
    float yn[NG][8];  // activation of the next group's first column
    uint4 nxt[WM][NG];
    uint4 mr[NX][NG];  // products of the group after next, loaded one group ahead
    {
      uint4 prev[WM][NG];
      load_group(q0 - 1, mr);
      finish_group(q0 - 1, mr, prev);
      act_column<NG>(prev[WM - 1], ok && q0 > 0, G, gm, y[0]);
    }
    load_group(q0, mr);
    finish_group(q0, mr, nxt);
    load_group(q0 + 1, mr);
    act_column<NG>(nxt[0], ok, G, gm, yn);
#pragma unroll
    for (int qq = 0; qq < R; ++qq) {
      const int q = q0 + qq;
      if (q >= WQ) break;  // uniform over the lane group
      uint4 cur[WM][NG];
#pragma unroll
      for (int e2 = 0; e2 < WM; ++e2)
#pragma unroll
        for (int h = 0; h < NG; ++h) cur[e2][h] = nxt[e2][h];
      if (ok && f >= tail_from) {
#pragma unroll
        for (int e2 = 0; e2 < WM; ++e2)
#pragma unroll
          for (int h = 0; h < NG; ++h)
            if (WM * q + e2 < W && (h == 0 || second))
              *reinterpret_cast<uint4*>(hout + (f - h_first) * h_fstride + ((long long)row * W + WM * q + e2) * ldh +
                                        (sub + h * G) * 8) = cur[e2][h];
      }
#pragma unroll
      for (int h = 0; h < NG; ++h)
#pragma unroll
        for (int c = 0; c < 8; ++c) y[1][h][c] = yn[h][c];
#pragma unroll
      for (int e2 = 1; e2 < WM; ++e2) act_column<NG>(cur[e2], ok && WM * q + e2 < W, G, gm, y[1 + e2]);
      finish_group(q + 1, mr, nxt);
      if (qq + 1 < R) load_group(q + 2, mr);
      act_column<NG>(nxt[0], ok && q + 1 < WQ, G, gm, yn);
#pragma unroll
      for (int h = 0; h < NG; ++h)
#pragma unroll
        for (int c = 0; c < 8; ++c) y[NX - 1][h][c] = yn[h][c];
      h16_t* dst = U + ((long long)(f + 2) * H * WQ + (long long)row * WQ + q) * C;
#pragma unroll
      for (int h = 0; h < NG; ++h) {
        if (h == 1 && !second) break;
        float u[NX][8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float d[NX], uu[NX];
#pragma unroll
          for (int k = 0; k < NX; ++k) d[k] = y[k][h][c];
          Wino<WM>::input(d, uu);
#pragma unroll
          for (int k = 0; k < NX; ++k) u[k][c] = uu[k];
        }
        if (ok) {
#pragma unroll
          for (int k = 0; k < NX; ++k)
            *reinterpret_cast<uint4*>(dst + (sub + h * G) * 8 + k * uplane) = pack8h(u[k]);
        }
      }
      // this group's last column opens the next window
#pragma unroll
      for (int h = 0; h < NG; ++h)
#pragma unroll
        for (int c = 0; c < 8; ++c) y[0][h][c] = y[WM][h][c];
    }
  }
}

// Output transform.  G lanes share a column group (G as in rms_stats_kernel);
// lane `sub` takes channel groups sub and sub + G.  With rs != null the
// kernel also writes the norm statistics of the group's output voxels,
// summed over the rounded fp16 outputs in exactly rms_stats_kernel's order
// (lane sums in group order, then the same butterfly), so a voxel's
// statistic does not depend on which kernel computed it.  ACT: the stored
// value is instead SiLU(v / ||v|| * gamma) of the rounded fp16 output v, with
// norm_silu_kernel's arithmetic (same sums, scale and products), for a
// consumer that reads only the activated tensor (the head).  NG: channel
// groups per lane (2 only where Cout / 8 > G, i.e. Cout = 1024), a
// compile-time bound so the narrower launches hold one group's registers.
template <bool ACT, int NG>
__global__ __launch_bounds__(256) void wino_out_kernel(const h16_t* __restrict__ M, int Cout, int F, int H, int W,
                                                       int WQ, int G, const float* __restrict__ bias,
                                                       const h16_t* res, long long res_fstride, int ldr, h16_t* out,
                                                       long long out_fstride, int ldo, float* __restrict__ rs,
                                                       const float* __restrict__ gamma) {
  constexpr int WM = kWinoM, NX = Wino<WM>::N;
  const int lane = threadIdx.x & 63;
  const int sub = lane % G;
  const int G8 = Cout >> 3;
  const long long plane = (long long)F * H * WQ * Cout;
  const long long ngrp = (long long)F * H * WQ;
  const int grp_per_wave = 64 / G;
  const long long gw = ((long long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const long long nw = ((long long)gridDim.x * blockDim.x) >> 6;
  float gm[NG][8];
#pragma unroll
  for (int q2 = 0; q2 < NG; ++q2)
#pragma unroll
    for (int k = 0; k < 8; ++k) gm[q2][k] = ACT && sub + q2 * G < G8 ? gamma[(sub + q2 * G) * 8 + k] : 0.0f;
  for (long long base = gw * grp_per_wave; base < ngrp; base += nw * grp_per_wave) {
    const long long pr = base + lane / G;
    const bool ok = pr < ngrp;
    const int q = ok ? (int)(pr % WQ) : 0;
    const long long r = ok ? pr / WQ : 0;
    const int row = (int)(r % H);
    const int f = (int)(r / H);
    const int nout = min(WM, W - WM * q);  // output columns of this group
    const long long pix0 = (long long)row * W + WM * q;
    float ss[WM];
#pragma unroll
    for (int e2 = 0; e2 < WM; ++e2) ss[e2] = 0.0f;
    uint4 hv[NG][WM];  // ACT: the rounded outputs, activated once their norms are known
#pragma unroll
    for (int q2 = 0; q2 < NG; ++q2) {
      const int g = sub + q2 * G;
      if (!ok || g >= G8) continue;
      const h16_t* src = M + (((long long)f * H + row) * WQ + q) * Cout + g * 8;
      uint4 mr[NX];
#pragma unroll
      for (int k = 0; k < NX; ++k) mr[k] = *reinterpret_cast<const uint4*>(src + k * plane);
      uint4 rr[WM];
#pragma unroll
      for (int e2 = 0; e2 < WM; ++e2) {
        rr[e2] = make_uint4(0, 0, 0, 0);
        if (res && e2 < nout) rr[e2] = *reinterpret_cast<const uint4*>(res + f * res_fstride + (pix0 + e2) * ldr + g * 8);
      }
      float b[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (bias) {
        const float4 b0 = *reinterpret_cast<const float4*>(bias + g * 8);
        const float4 b1 = *reinterpret_cast<const float4*>(bias + g * 8 + 4);
        b[0] = b0.x; b[1] = b0.y; b[2] = b0.z; b[3] = b0.w;
        b[4] = b1.x; b[5] = b1.y; b[6] = b1.z; b[7] = b1.w;
      }
      float m[NX][8];
#pragma unroll
      for (int k = 0; k < NX; ++k) unpack8h(mr[k], m[k]);
      float o[WM][8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float mm[NX], oo[WM];
#pragma unroll
        for (int k = 0; k < NX; ++k) mm[k] = m[k][c];
        Wino<WM>::output(mm, oo);
#pragma unroll
        for (int e2 = 0; e2 < WM; ++e2) o[e2][c] = oo[e2];
      }
#pragma unroll
      for (int e2 = 0; e2 < WM; ++e2) {
        if (e2 >= nout) break;
        float v[8], r8[8];
        unpack8h(rr[e2], r8);
#pragma unroll
        for (int c = 0; c < 8; ++c) v[c] = o[e2][c] + b[c] + r8[c];
        const uint4 packed = pack8h_int(v);
        h16_t* const dst = out + f * out_fstride + (pix0 + e2) * ldo + g * 8;
        if constexpr (ACT && NG == 2)
          hv[q2][e2] = packed;
        else if constexpr (!ACT)
          *reinterpret_cast<uint4*>(dst) = packed;
        float h[8];
        unpack8h(packed, h);
        float t = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) t = fmaf(h[k], h[k], t);
        ss[e2] += t;
        if constexpr (ACT && NG == 1) {
          // one channel group per lane: the column's sum is complete here
          // (the group's G lanes share q, so they all reach this point)
          const float sc = 1.0f / fmaxf(sqrtf(lane_group_sum(ss[e2], G)), kNormEps);
#pragma unroll
          for (int k = 0; k < 8; ++k) h[k] = silu_hw(h[k] * sc * gm[0][k]);
          *reinterpret_cast<uint4*>(dst) = pack8h_int(h);
        }
      }
    }
    if (ACT ? NG == 2 : rs != nullptr) {
#pragma unroll
      for (int e2 = 0; e2 < WM; ++e2) {
        float v = ss[e2];
        for (int off = 1; off < G; off <<= 1) v += __shfl_xor(v, off, 64);
        const float sc = 1.0f / fmaxf(sqrtf(v), kNormEps);
        if (rs && ok && sub == 0 && e2 < nout) rs[(long long)(f + 2) * H * W + pix0 + e2] = sc;
        if constexpr (ACT) {
#pragma unroll
          for (int q2 = 0; q2 < NG; ++q2) {
            const int g = sub + q2 * G;
            if (!ok || g >= G8 || e2 >= nout) continue;
            float a[8];
            unpack8h(hv[q2][e2], a);
#pragma unroll
            for (int k = 0; k < 8; ++k) a[k] = silu_hw(a[k] * sc * gm[q2][k]);
            *reinterpret_cast<uint4*>(out + f * out_fstride + (pix0 + e2) * ldo + g * 8) = pack8h_int(a);
          }
        }
      }
    }
  }
}

__global__ void prep_vec_kernel(const void* __restrict__ v, int dtype, int n, float scale, float* __restrict__ out) {
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < n; e += gridDim.x * blockDim.x)
    out[e] = load_in(v, e, dtype) * scale;
}

__global__ void prep_vec_add_kernel(const void* __restrict__ a, const void* __restrict__ b, int dtype, int n,
                                    float* __restrict__ out) {
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < n; e += gridDim.x * blockDim.x)
    out[e] = load_in(a, e, dtype) + load_in(b, e, dtype);
}

unsigned grid_for(long long n, int per_block = 256, long long cap = 65536) {
  long long g = (n + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_rms_stats(const h16_t* x, long long x_fstride, int lda, const h16_t* ring, int n_hist,
                            int C, int F, int HW, float* rs, hipStream_t s) {
  if (g_dry_run) return hipSuccess;
  int G = 1;
  while (G < 64 && G * 2 <= C / 8) G *= 2;
  if (C % 8 || C / 8 > 2 * G || C > 1024) return hipErrorInvalidValue;  // at most two groups per lane
  const long long nvox = (long long)(F + n_hist) * HW;
  const long long waves = (nvox + (64 / G) * kStatsU - 1) / ((64 / G) * kStatsU);
  hipLaunchKernelGGL(rms_stats_kernel, dim3(grid_for(waves * 64, 256, 16384)), dim3(256), 0, s, x, x_fstride, lda,
                     ring, n_hist, C, F, HW, G, rs);
  return hipGetLastError();
}

hipError_t launch_norm_silu(const h16_t* x, long long x_fstride, int lda, int C, int F, int HW, const float* gamma,
                            h16_t* y, long long y_fstride, int ldy, hipStream_t s, bool act) {
  if (g_dry_run) return hipSuccess;
  int G = 1;
  while (G < 64 && G * 2 <= C / 8) G *= 2;
  if (C % 8 || C / 8 > 2 * G || C > 1024) return hipErrorInvalidValue;
  const long long nvox = (long long)F * HW;
  if (nvox >= (1LL << 30)) return hipErrorInvalidValue;  // the kernel counts voxels in 32 bits
  const long long waves = (nvox + (64 / G) * kStatsU - 1) / ((64 / G) * kStatsU);
  if (act)
    hipLaunchKernelGGL(norm_silu_kernel<true>, dim3(grid_for(waves * 64, 256, 16384)), dim3(256), 0, s, x, x_fstride,
                       lda, C, F, HW, G, gamma, y, y_fstride, ldy);
  else
    hipLaunchKernelGGL(norm_silu_kernel<false>, dim3(grid_for(waves * 64, 256, 16384)), dim3(256), 0, s, x, x_fstride,
                       lda, C, F, HW, G, gamma, y, y_fstride, ldy);
  return hipGetLastError();
}

hipError_t launch_ring_update(h16_t* ring, const h16_t* x, long long x_fstride, int lda, int C, int F, int HW,
                              hipStream_t s) {
  if (g_dry_run) return hipSuccess;
  const long long n = (long long)HW * (C / 8);
  hipLaunchKernelGGL(ring_update_kernel, dim3(grid_for(n, 256, 16384)), dim3(256), 0, s, ring, x, x_fstride, lda, C,
                     F, HW);
  return hipGetLastError();
}

hipError_t launch_pre_conv(const h16_t* zt, long long nvox, const float* A, const float* b, h16_t* zp,
                           hipStream_t s) {
  if (g_dry_run) return hipSuccess;
  if (!zt || !A || !b || !zp || nvox < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pre_conv_kernel, dim3(grid_for(nvox * 8)), dim3(256), 0, s, zt, nvox, A, b, zp);
  return hipGetLastError();
}

hipError_t launch_latent_to_cl(const void* z, int dtype, int T, int t0, int F, int HW, h16_t* zt, hipStream_t s) {
  if (g_dry_run) return hipSuccess;
  hipLaunchKernelGGL(latent_to_cl_kernel, dim3(grid_for((long long)F * HW)), dim3(256), 0, s, z, dtype, T, t0, F, HW,
                     zt);
  return hipGetLastError();
}

hipError_t launch_attn_frag(const h16_t* qkv, int F, int L, int C, int Np, h16_t* kf, h16_t* vf, hipStream_t s) {
  if (g_dry_run) return hipSuccess;
  if (F < 1 || L < 1 || C % 32 || Np % 256 || Np < L || F > 65535) return hipErrorInvalidValue;
  const long long n = (long long)(Np / 32) * (C / 16) * 64 + (long long)(C / 32) * (Np / 16) * 64;
  hipLaunchKernelGGL(attn_frag_kernel, dim3(grid_for(n, 256, 4096), F), dim3(256), 0, s, qkv, L, C, Np, kf, vf);
  return hipGetLastError();
}

hipError_t launch_attn_rescale(h16_t* P, const float* st, long long rows, int np, hipStream_t s) {
  if (rows < 1 || np < 64 || np % 64) return hipErrorInvalidValue;
  if (g_dry_run) return hipSuccess;
  hipLaunchKernelGGL(attn_rescale_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, P,
                     reinterpret_cast<const float2*>(st), rows, np);
  return hipGetLastError();
}

hipError_t launch_patchify(const void* video, int dtype, int T, int t0, int F, int H, int W, h16_t* out,
                           hipStream_t s) {
  if (g_dry_run) return hipSuccess;
  const long long n = (long long)F * H * W;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(patchify_kernel, dim3(grid_for(n)), dim3(256), 0, s, video, dtype, T, t0, F, H, W, out);
  return hipGetLastError();
}

hipError_t launch_copy16(void* dst, const void* src, size_t bytes, hipStream_t s) {
  if (g_dry_run) return hipSuccess;
  const long long n = (long long)(bytes / 16);
  hipLaunchKernelGGL(copy16_kernel, dim3(grid_for(n, 256, 16384)), dim3(256), 0, s, static_cast<uint4*>(dst),
                     static_cast<const uint4*>(src), n);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* dst, size_t bytes, hipStream_t s) {
  if (g_dry_run) return hipSuccess;
  const long long n = (long long)(bytes / 16);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n, 256, 16384)), dim3(256), 0, s, static_cast<uint4*>(dst), n);
  return hipGetLastError();
}

hipError_t launch_softmax_rows(const float* S, int rows, int L, int Lpad, h16_t* P, hipStream_t s) {
  if (g_dry_run) return hipSuccess;
  hipLaunchKernelGGL(softmax_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, S, rows, L, Lpad, P);
  return hipGetLastError();
}

hipError_t launch_transpose_v(const h16_t* qkv, int F, int L, int C, int Lpad, h16_t* vt, hipStream_t s) {
  if (g_dry_run) return hipSuccess;
  dim3 grid((unsigned)((Lpad + 63) / 64), (unsigned)((C + 63) / 64), (unsigned)F);
  hipLaunchKernelGGL(transpose_v_kernel, grid, dim3(256), 0, s, qkv, L, C, Lpad, vt);
  return hipGetLastError();
}

size_t prep_frag_bytes(int cout, int cin_pad, int taps) {
  return (size_t)((cout + 127) / 128) * 128 * cin_pad * taps * 2;
}

hipError_t launch_prep_frag(const void* w, int dtype, int cout, int cin, int taps, int cin_pad, h16_t* out,
                            hipStream_t s) {
  if (g_dry_run) return hipSuccess;
  const long long n = (long long)prep_frag_bytes(cout, cin_pad, taps) / 2;
  hipLaunchKernelGGL(prep_frag_kernel, dim3(grid_for(n)), dim3(256), 0, s, w, dtype, cout, cin, 0, cin, taps,
                     cin_pad, out);
  return hipGetLastError();
}

hipError_t launch_prep_frag_part(const void* w, int dtype, int cout, int cin_src, int cin_off, int cin, int taps,
                                 int cin_pad, h16_t* out, hipStream_t s) {
  if (g_dry_run) return hipSuccess;
  if (cin_off < 0 || cin_off + cin > cin_src || cin > cin_pad) return hipErrorInvalidValue;
  const long long n = (long long)prep_frag_bytes(cout, cin_pad, taps) / 2;
  hipLaunchKernelGGL(prep_frag_kernel, dim3(grid_for(n)), dim3(256), 0, s, w, dtype, cout, cin_src, cin_off, cin,
                     taps, cin_pad, out);
  return hipGetLastError();
}

hipError_t launch_prep_headx_frag(const void* w, int dtype, int cin, h16_t* out, hipStream_t s) {
  if (g_dry_run) return hipSuccess;
  if (cin < 32 || cin % 32) return hipErrorInvalidValue;
  const long long n = (long long)prep_frag_bytes(64, cin, 9) / 2;
  hipLaunchKernelGGL(prep_headx_frag_kernel, dim3(grid_for(n)), dim3(256), 0, s, w, dtype, cin, out);
  return hipGetLastError();
}

hipError_t launch_prep_s2d_frag(const void* w, int dtype, int C, h16_t* out, hipStream_t s) {
  if (g_dry_run) return hipSuccess;
  if (C % 8) return hipErrorInvalidValue;
  const long long n = (long long)prep_frag_bytes(C, 4 * C, 4) / 2;
  hipLaunchKernelGGL(prep_s2d_frag_kernel, dim3(grid_for(n)), dim3(256), 0, s, w, dtype, C, out);
  return hipGetLastError();
}

hipError_t launch_space_to_depth(const h16_t* x, long long x_fstride, int C, int F, int H, int W, h16_t* y,
                                 hipStream_t s) {
  if (g_dry_run) return hipSuccess;
  if (!x || !y || C % 8 || H % 2 || W % 2 || F < 1 || x_fstride < (long long)H * W * C) return hipErrorInvalidValue;
  const long long n = (long long)F * (H / 2) * (W / 2) * 4 * (C / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(space_to_depth_kernel, dim3(grid_for(n, 256, 65536)), dim3(256), 0, s, x, x_fstride, C, F, H, W,
                     y);
  return hipGetLastError();
}

hipError_t launch_prep_phase_frag(const void* w, int dtype, int C, h16_t* out, hipStream_t s) {
  if (g_dry_run) return hipSuccess;
  const long long n = (long long)prep_frag_bytes(C, C, 16) / 2;
  hipLaunchKernelGGL(prep_phase_frag_kernel, dim3(grid_for(n)), dim3(256), 0, s, w, dtype, C, out);
  return hipGetLastError();
}

hipError_t launch_prep_wino_frag(const void* w, int dtype, int cout, int cin, h16_t* out, hipStream_t s) {
  if (g_dry_run) return hipSuccess;
  if (cin % 16) return hipErrorInvalidValue;
  const long long n = (long long)prep_frag_bytes(cout, cin, kWinoN * 9) / 2;
  hipLaunchKernelGGL(prep_wino_frag_kernel, dim3(grid_for(n)), dim3(256), 0, s, w, dtype, cout, cin, out);
  return hipGetLastError();
}

hipError_t launch_wino_in(const h16_t* x, long long x_fstride, int lda, const h16_t* ring, int n_hist, int C, int F,
                          int H, int W, const float* gamma, h16_t* U, hipStream_t s, bool history_only) {
  if (g_dry_run) return hipSuccess;
  if (C % 8 || C > 1024 || n_hist < 0 || n_hist > 2 || (n_hist > 0 && !ring) || F < 1) return hipErrorInvalidValue;
  const int WQ = (W + kWinoM - 1) / kWinoM;
  int G = 1;
  while (G * 2 <= (C >> 3) && G * 2 <= 64) G *= 2;
  const int first = 2 - n_hist, end = history_only ? 2 : F + 2;
  if (end <= first) return hipSuccess;
  const int R = wino_in_run(C / 8 > G ? 2 : 1);
  const long long runs = (long long)(end - first) * H * ((WQ + R - 1) / R);
  if (runs >= (1LL << 30)) return hipErrorInvalidValue;  // the kernel counts runs in 32 bits
  const long long threads = (runs + 64 / G - 1) / (64 / G) * 64;
  if (C / 8 > G)
    hipLaunchKernelGGL(wino_in_kernel<2>, dim3(grid_for(threads, 256, 65536)), dim3(256), 0, s, x, x_fstride, lda,
                       ring, first, end, C, F + 2, H, W, WQ, G, gamma, U);
  else
    hipLaunchKernelGGL(wino_in_kernel<1>, dim3(grid_for(threads, 256, 65536)), dim3(256), 0, s, x, x_fstride, lda,
                       ring, first, end, C, F + 2, H, W, WQ, G, gamma, U);
  return hipGetLastError();
}

bool wino_mid_ok(int C) { return C % 8 == 0 && C <= 512; }

hipError_t launch_wino_mid(const h16_t* M, const float* bias, int C, int F, int H, int W, const float* gamma,
                           h16_t* U, h16_t* hout, long long h_fstride, int ldh, int tail_from, int h_first,
                           hipStream_t s) {
  if (g_dry_run) return hipSuccess;
  if (!wino_mid_ok(C) || F < 1 || ldh % 8 || ldh < C) return hipErrorInvalidValue;
  const int WQ = (W + kWinoM - 1) / kWinoM;
  int G = 1;
  while (G * 2 <= (C >> 3) && G * 2 <= 64) G *= 2;
  const long long runs = (long long)F * H * ((WQ + kWinoInRun - 1) / kWinoInRun);
  // the kernel counts runs and column groups in 32 bits
  if ((long long)F * H * WQ >= (1LL << 30)) return hipErrorInvalidValue;
  const long long threads = (runs + 64 / G - 1) / (64 / G) * 64;
  hipLaunchKernelGGL(wino_mid_kernel<1>, dim3(grid_for(threads, 256, 65536)), dim3(256), 0, s, M, bias, C, F, H, W,
                     WQ, G, gamma, U, hout, h_fstride, ldh, tail_from, h_first);
  return hipGetLastError();
}

hipError_t launch_wino_out(const h16_t* M, int Cout, int F, int H, int W, const float* bias, const h16_t* res,
                           long long res_fstride, int ldr, h16_t* out, long long out_fstride, int ldo, float* rs,
                           const float* act_gamma, hipStream_t s) {
  if (Cout % 8 || ldo % 8 || (res && ldr % 8) || Cout > 1024 || (act_gamma && rs)) return hipErrorInvalidValue;
  if (g_dry_run) return hipSuccess;
  int G = 1;
  while (G < 64 && G * 2 <= Cout / 8) G *= 2;
  const int WQ = (W + kWinoM - 1) / kWinoM;
  const long long ngrp = (long long)F * H * WQ;
  const long long waves = (ngrp + (64 / G) - 1) / (64 / G);
  const dim3 grid(grid_for(waves * 64, 256, 65536));
  if (Cout / 8 > G) {  // two channel groups per lane
    if (act_gamma)
      hipLaunchKernelGGL((wino_out_kernel<true, 2>), grid, dim3(256), 0, s, M, Cout, F, H, W, WQ, G, bias, res,
                         res_fstride, ldr, out, out_fstride, ldo, rs, act_gamma);
    else
      hipLaunchKernelGGL((wino_out_kernel<false, 2>), grid, dim3(256), 0, s, M, Cout, F, H, W, WQ, G, bias, res,
                         res_fstride, ldr, out, out_fstride, ldo, rs, nullptr);
  } else {
    if (act_gamma)
      hipLaunchKernelGGL((wino_out_kernel<true, 1>), grid, dim3(256), 0, s, M, Cout, F, H, W, WQ, G, bias, res,
                         res_fstride, ldr, out, out_fstride, ldo, rs, act_gamma);
    else
      hipLaunchKernelGGL((wino_out_kernel<false, 1>), grid, dim3(256), 0, s, M, Cout, F, H, W, WQ, G, bias, res,
                         res_fstride, ldr, out, out_fstride, ldo, rs, nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_prep_vec(const void* v, int dtype, int n, float scale, float* out, hipStream_t s) {
  if (g_dry_run) return hipSuccess;
  hipLaunchKernelGGL(prep_vec_kernel, dim3(grid_for(n)), dim3(256), 0, s, v, dtype, n, scale, out);
  return hipGetLastError();
}

hipError_t launch_prep_vec_add(const void* a, const void* b, int dtype, int n, float* out, hipStream_t s) {
  if (g_dry_run) return hipSuccess;
  hipLaunchKernelGGL(prep_vec_add_kernel, dim3(grid_for(n)), dim3(256), 0, s, a, b, dtype, n, out);
  return hipGetLastError();
}

// The device SiLU and exp of the kernels, evaluated elementwise (the math
// self-test bounds their error against an exact reference).
__global__ void math_probe_kernel(const float* __restrict__ x, float* __restrict__ silu_out,
                                  float* __restrict__ exp_out, long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float t = x[i];
  silu_out[i] = silu_hw(t);
  exp_out[i] = exp_hw(t);
}

hipError_t launch_math_probe(const float* x, float* silu_out, float* exp_out, long long n, hipStream_t s) {
  if (g_dry_run || n == 0) return hipSuccess;
  hipLaunchKernelGGL(math_probe_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, silu_out, exp_out, n);
  return hipGetLastError();
}

// The kernels' fp16 packing (eight values at a time) and the input
// transforms' norm scale, elementwise (the conversion self-test).
__global__ void f16_probe_kernel(const float* __restrict__ x, uint16_t* __restrict__ h_out,
                                 float* __restrict__ rs_out, long long n8) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const float4 a = *reinterpret_cast<const float4*>(x + 8 * i);
  const float4 b = *reinterpret_cast<const float4*>(x + 8 * i + 4);
  const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  *reinterpret_cast<uint4*>(h_out + 8 * i) = pack8h(f);
  float r[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) r[k] = norm_scale(f[k]);
  *reinterpret_cast<float4*>(rs_out + 8 * i) = make_float4(r[0], r[1], r[2], r[3]);
  *reinterpret_cast<float4*>(rs_out + 8 * i + 4) = make_float4(r[4], r[5], r[6], r[7]);
}

hipError_t launch_f16_probe(const float* x, uint16_t* h_out, float* rs_out, long long n, hipStream_t s) {
  if (g_dry_run || n == 0) return hipSuccess;
  const long long n8 = n / 8;
  hipLaunchKernelGGL(f16_probe_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, x, h_out, rs_out, n8);
  return hipGetLastError();
}

// Device address of this code object's range flags on the current device.
hipError_t aux_range_flags_addr(unsigned int** p) {
  return hipGetSymbolAddress(reinterpret_cast<void**>(p), HIP_SYMBOL(g_range_flags));
}

}  // namespace wvd
