// Implicit-GEMM causal convolution on fp16 MFMA (gfx950), with the channel
// RMSNorm (+ SiLU) applied while the input tile is staged into LDS and the
// bias / residual / frame-interleave / phase-scatter / pixel-shuffle work
// done in the epilogue.
//
// GEMM view: M = output voxels (tile TF x TH x 16), N = output channels
// (tile BN), K = taps x input channels.  The K loop runs segment by segment
// (the main conv, then optionally a 1x1x1 shortcut over the raw block input),
// input-channel chunk by chunk (BK channels), tap by tap.
//
//  * A (activations): for each chunk the input halo of the tile -- e.g.
//    4 x 10 x 18 voxels for a 3x3x3 conv over a 2 x 8 x 16 tile -- is staged
//    into LDS once (normalised on the way in), and every tap reads a shifted
//    window of it.  Rows are padded to BK*2+16 bytes, which makes the 16-byte
//    fragment reads of 16 consecutive voxels bank-conflict free and turns
//    every tap offset into an instruction immediate.  The next chunk's halo
//    is loaded while the current one is multiplied (double buffer), so the
//    only barrier is one per chunk.
//  * B (weights): wvd_prepare stores each conv in MFMA fragment order -- one
//    1 KiB block per (32 output channels, 16 input channels, tap) holding
//    exactly what the 64 lanes of a wave feed the matrix core -- so each wave
//    streams its own B fragments from L2 into registers with fully coalesced
//    loads, several taps ahead of use.  Activation operands of the attention
//    GEMMs are read the same way from their row-major layout.
//
// The accumulation order (segment, chunk, tap, k16 step) does not depend on
// where a tile lies, which keeps every output bit-identical for any
// frames_per_pass.
//
// The conv definition (cross-correlation, causal in time with two history
// frames, zero spatial padding) follows the decoder the Wan2.2 VAE decoder
// page describes; normalisation is channel RMSNorm with affine scale and SiLU
// as the TensorRT-LLM norm-SiLU issue describes for the decoder's residual
// norms and norm_out, statistics in fp32 (Wan2.2 page, "Limits").
#include <cstring>
#include <type_traits>

#include "wvd_internal.h"

namespace wvd {

namespace {

// Geometry of the specialised 3x3x3 tile: 2 frames x 8 rows x 16 columns.
constexpr int kTF333 = 2;
constexpr int kTH333 = 8;
constexpr int kHX = kTileW + 2;
constexpr int kHY333 = kTH333 + 2;
constexpr int kHF333 = kTF333 + 2;
constexpr int kNHV333 = kHF333 * kHY333 * kHX;  // 720 halo voxels
constexpr int kBRing = 6;       // k16 steps of B fragments in flight
constexpr int kPhaseBRing = 4;  // the same for the up-conv phase loop
constexpr int kWinoLag = 3;     // Winograd GEMM: taps between a halo item's load and its LDS store
// Tile of the Winograd-domain GEMM: 2 frames x 8 rows x 16 column groups
// (halo 4 x 10 x 16 rows; a 4 x 4 x 16 tile has fewer halo rows but measured slower).
constexpr int kTFWino = kWinoTF;
}  // namespace
// Tile shapes (frames x column groups) the Winograd-domain GEMM is built for;
// rows = 256 / (TF * TW).  Deeper tiles in t and y cut the halo per output.
bool wino_tile_shape_ok(int TF, int TW) {
  return (TF == 2 && (TW == 16 || TW == 8)) || (TF == 4 && (TW == 8 || TW == 4)) || (TF == 8 && TW == 4);
}
namespace {

__device__ __forceinline__ f16x8_t ld_frag(const h16_t* p) { return *reinterpret_cast<const f16x8_t*>(p); }

// 16-byte load through the global address space.  Halo pointers come from an
// LDS table, so the compiler cannot infer their address space; a generic
// (flat) load would also count against the LDS wait counter and serialise the
// fragment reads behind HBM latency.
__device__ __forceinline__ uint4 ld_global16(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u v = *(const __attribute__((address_space(1))) v4u*)(reinterpret_cast<uintptr_t>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *static_cast<const uint4*>(p);
#endif
}

// Per-segment state shared by the tap loops.
template <int BK, int MI, int NJ, int NT_>
struct SegCtx {
  static constexpr int NT = NT_;        // threads per workgroup
  static constexpr int NP = BK / 8;
  static constexpr int ROWB = BK * 2 + 16;
  static constexpr int KS = BK / 16;
  unsigned char* halo0;  // halo buffer b at halo0 + b * halo_bytes
  int halo_bytes;
  const h16_t* const* vptr;
  const float* rs;
  const float* gamma;
  int abase[MI];         // LDS byte address of each A row at tap (0,0,0), k16 step 0
  int bvoff[NJ];         // buffer offset of this lane's B fragments (fragment order)
  __amdgpu_buffer_rsrc_t wrsrc;
  int wtaps, tap0;       // taps per (n32, k16) block and this phase's first tap
  int tid;
};

// One halo item (row idx / NP, 16-byte part idx % NP) of chunk `chunk`.
template <class G>
__device__ __forceinline__ uint4 halo_load(const G& g, int idx, int chunk) {
  constexpr int NP = G::NP;
  return ld_global16(g.vptr[idx / NP] + chunk * (NP * 8) + (idx % NP) * 8);
}

// The same item split in two: its row's address (an LDS table read that can
// be issued a step early) and the load of chunk `chunk` of the item from it.
template <class G>
__device__ __forceinline__ const h16_t* halo_row(const G& g, int idx) {
  return g.vptr[idx / G::NP];
}

template <class G>
__device__ __forceinline__ uint4 halo_load_at(const h16_t* row, int idx, int chunk) {
  constexpr int NP = G::NP;
  return ld_global16(row + chunk * (NP * 8) + (idx % NP) * 8);
}

template <bool NORM, bool ACT, class G>
__device__ __forceinline__ void halo_store(const G& g, int idx, int chunk, uint4 r, unsigned char* hbuf) {
  constexpr int NP = G::NP;
  constexpr int BK = NP * 8;
  constexpr int ROWB = G::ROWB;
  const int v = idx / NP;
  const int p = idx % NP;
  if constexpr (NORM) {
    float f[8];
    unpack8h(r, f);
    const float sc = g.rs[v];
    const float* gm = g.gamma + chunk * BK + p * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float t = f[k] * sc * gm[k];
      f[k] = ACT ? silu_hw(t) : t;
    }
    r = pack8h(f);
  }
  *reinterpret_cast<uint4*>(hbuf + v * ROWB + 16 * p) = r;
}

// B fragments of (chunk, tap) from fragment-order weights.
template <int BK, int NJ, class G>
__device__ __forceinline__ void load_b_frag(const G& g, f16x8_t (&b)[NJ][BK / 16], int chunk, int tap) {
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int soff = ((chunk * (BK / 16) + ks) * g.wtaps + g.tap0 + tap) * 1024;
      b[j][ks] = __builtin_bit_cast(f16x8_t, __builtin_amdgcn_raw_buffer_load_b128(g.wrsrc, g.bvoff[j], soff, 0));
    }
}

template <int BK, int MI, int NJ, class G>
__device__ __forceinline__ void mma_tap(const G& g, f32x16_t (&acc)[MI][NJ],
                                        const unsigned char* hsrc, int toff_bytes,
                                        const f16x8_t (&b)[NJ][BK / 16]) {
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    f16x8_t av[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
      av[i] = *reinterpret_cast<const f16x8_t*>(hsrc + g.abase[i] + toff_bytes + ks * 32);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], b[j][ks], acc[i][j], 0, 0, 0);
  }
}

// 3x3x3 segment over a 2 x 8 x 16 tile: 9 (dt, dy) groups of 3 dx taps per
// chunk, each tap two k16 steps.  B fragments of k16 step u (= 2 * tap + ks)
// live in slot u % 3 and are refilled with step u + 3 right after use (1.5
// taps of lookahead in 3 x NJ fragment registers); halo item t of the next
// chunk is loaded at tap t and normalised into LDS at tap t + 3.  Everything
// that selects code is a compile-time constant here.
template <int BK, int MI, int NJ, bool NORM, bool ACT, int DEPTH, class G>
__device__ __forceinline__ void run_333(const G& g, f32x16_t (&acc)[MI][NJ], int nchunks) {
  static_assert(BK == 32, "the 3x3x3 path runs two k16 steps per tap");
  static_assert(DEPTH == 3 || DEPTH == 6, "the B ring must divide the 6 k16 steps of a dx group");
  constexpr int NP = BK / 8;
  constexpr int ROWB = BK * 2 + 16;
  constexpr int NT = G::NT;
  constexpr int IPT = (kNHV333 * NP + NT - 1) / NT;  // halo items per thread per chunk
  static_assert(IPT + 3 <= 27, "halo items must land inside a chunk");
  f16x8_t bq[DEPTH][NJ];
  auto load_step = [&](f16x8_t (&b)[NJ], int chunk, int tap, int ks) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int soff = ((chunk * 2 + ks) * g.wtaps + g.tap0 + tap) * 1024;
      b[j] = __builtin_bit_cast(f16x8_t, __builtin_amdgcn_raw_buffer_load_b128(g.wrsrc, g.bvoff[j], soff, 0));
    }
  };
  // Issue order matters: the wait at the top of the chunk loop must hold for
  // both the first entry and the back edge, so the preloads go out in the
  // same order as the in-loop refills.
#pragma unroll
  for (int u = 0; u < DEPTH; ++u) {
    load_step(bq[u], 0, u >> 1, u & 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int c = 0; c < nchunks; ++c) {
    const unsigned char* hsrc = g.halo0 + (c & 1) * g.halo_bytes;
    unsigned char* hdst = g.halo0 + ((c + 1) & 1) * g.halo_bytes;
    // The last chunk streams its own halo and weights once more into the
    // spare buffer and ring slots instead of branching around the prefetch:
    // with no branch the wait counters stay exact and keep the full ring in
    // flight up to the chunk's end.
    const int cn = c + 1 < nchunks ? c + 1 : c;
    uint4 hr[3];
    for (int gi = 0; gi < 9; ++gi) {
      const int goff = ((gi / 3) * kHY333 + (gi % 3)) * kHX * ROWB;
#pragma unroll
      for (int s6 = 0; s6 < 6; ++s6) {
        const int dx = s6 >> 1, ks = s6 & 1;
        const int t = 3 * gi + dx;
        if (ks == 0) {
          if (t >= 3 && t - 3 < IPT) halo_store<NORM, ACT>(g, g.tid + NT * (t - 3), cn, hr[dx], hdst);
          if (t < IPT) hr[dx] = halo_load(g, g.tid + NT * t, cn);
        }
        {
          f16x8_t av[MI];
#pragma unroll
          for (int i = 0; i < MI; ++i)
            av[i] = *reinterpret_cast<const f16x8_t*>(hsrc + g.abase[i] + goff + dx * ROWB + ks * 32);
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bq[s6 % DEPTH][j], acc[i][j], 0, 0, 0);
        }
        // refill with k16 step u + DEPTH
        const int t3 = 3 * gi + (s6 + DEPTH) / 2;
        const int ks3 = (s6 + DEPTH) & 1;
        if (t3 < 27) {
          load_step(bq[s6 % DEPTH], c, t3, ks3);
        } else {
          load_step(bq[s6 % DEPTH], cn, t3 - 27, ks3);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();  // next chunk's halo complete; this chunk's reads done
  }
}

// 3x3x3 segment for 8-wave workgroups (two waves per SIMD, 256 registers
// each): a runtime loop over the 27 taps with the two k16 steps unrolled.  B
// fragments of step ks of the next tap are refilled into slot ks as soon as
// the current tap's step ks is issued (one tap of lookahead; the other wave
// on the SIMD covers the rest), and halo item t of the next chunk is loaded
// and normalised within tap t.
template <int BK, int MI, int NJ, bool NORM, bool ACT, class G>
__device__ __forceinline__ void run_333_lean(const G& g, f32x16_t (&acc)[MI][NJ], int nchunks) {
  static_assert(BK == 32, "the 3x3x3 path runs two k16 steps per tap");
  constexpr int NP = BK / 8;
  constexpr int ROWB = BK * 2 + 16;
  constexpr int NT = G::NT;
  constexpr int IPT = (kNHV333 * NP + NT - 1) / NT;  // halo items per thread per chunk
  static_assert(IPT <= 27, "halo items must land inside a chunk");
  f16x8_t bq[2][NJ];
  auto load_step = [&](f16x8_t (&b)[NJ], int chunk, int tap, int ks) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int soff = ((chunk * 2 + ks) * g.wtaps + g.tap0 + tap) * 1024;
      b[j] = __builtin_bit_cast(f16x8_t, __builtin_amdgcn_raw_buffer_load_b128(g.wrsrc, g.bvoff[j], soff, 0));
    }
  };
  load_step(bq[0], 0, 0, 0);
  load_step(bq[1], 0, 0, 1);
  for (int c = 0; c < nchunks; ++c) {
    const unsigned char* hsrc = g.halo0 + (c & 1) * g.halo_bytes;
    unsigned char* hdst = g.halo0 + ((c + 1) & 1) * g.halo_bytes;
    const bool hnext = c + 1 < nchunks;
    int dt = 0, dy = 0, dx = 0;
    for (int t = 0; t < 27; ++t) {
      const int toff = ((dt * kHY333 + dy) * kHX + dx) * ROWB;
      const bool item = hnext && t < IPT;
      uint4 hr;
      if (item) hr = halo_load(g, g.tid + NT * t, c + 1);
      const int tn = t + 1 < 27 ? t + 1 : 0;
      const int cn = t + 1 < 27 ? c : c + 1;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        f16x8_t av[MI];
#pragma unroll
        for (int i = 0; i < MI; ++i)
          av[i] = *reinterpret_cast<const f16x8_t*>(hsrc + g.abase[i] + toff + ks * 32);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bq[ks][j], acc[i][j], 0, 0, 0);
        if (cn < nchunks) load_step(bq[ks], cn, tn, ks);
      }
      if (item) halo_store<NORM, ACT>(g, g.tid + NT * t, c + 1, hr, hdst);
      if (++dx == 3) {
        dx = 0;
        if (++dy == 3) {
          dy = 0;
          ++dt;
        }
      }
    }
    __syncthreads();  // next chunk's halo complete; this chunk's reads done
  }
}

// Up-conv phase segment (nearest-2x + 3x3 conv in phase form) over a
// 1 x 16 x 16 low-resolution tile: per chunk the phase's 2x2 taps x two k16
// steps run unrolled; B fragments of step u live in slot u % 4 and are
// refilled with step u + 4 (two taps ahead, across chunks); halo item k of
// the next chunk is loaded at step k and normalised into LDS LAG steps later.
template <int BK, int MI, int NJ, class G>
__device__ __forceinline__ void run_phase(const G& g, f32x16_t (&acc)[MI][NJ], int nchunks, int py, int px,
                                          int nitems) {
  static_assert(BK == 32, "two k16 steps per tap");
  constexpr int ROWB = BK * 2 + 16;
  constexpr int NT = G::NT;
  constexpr int HX = kTileW + 2;
  constexpr int IPT = ((1 * 18 * 18) * (BK / 8) + NT - 1) / NT;  // halo items per thread per chunk
  constexpr int LAG = 8 - IPT;
  static_assert(IPT >= 1 && IPT <= 7, "phase halo items per chunk");
  (void)nitems;
  int toff[4];
#pragma unroll
  for (int tap = 0; tap < 4; ++tap) toff[tap] = ((py + (tap >> 1)) * HX + (px + (tap & 1))) * ROWB;
  f16x8_t bq[4][NJ];
  auto load_step = [&](f16x8_t (&b)[NJ], int chunk, int tap, int ks) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int soff = ((chunk * 2 + ks) * g.wtaps + g.tap0 + tap) * 1024;
      b[j] = __builtin_bit_cast(f16x8_t, __builtin_amdgcn_raw_buffer_load_b128(g.wrsrc, g.bvoff[j], soff, 0));
    }
  };
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    load_step(bq[u], 0, u >> 1, u & 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int c = 0; c < nchunks; ++c) {
    const unsigned char* hsrc = g.halo0 + (c & 1) * g.halo_bytes;
    unsigned char* hdst = g.halo0 + ((c + 1) & 1) * g.halo_bytes;
    // the last chunk re-streams its own halo and weights (no branch: exact
    // wait counters across the chunk boundary)
    const int cn = c + 1 < nchunks ? c + 1 : c;
    uint4 hr[IPT];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int tap = u >> 1, ks = u & 1;
      if (u >= LAG && u - LAG < IPT) halo_store<false, false>(g, g.tid + NT * (u - LAG), cn, hr[u - LAG], hdst);
      if (u < IPT) hr[u] = halo_load(g, g.tid + NT * u, cn);
      f16x8_t av[MI];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        av[i] = *reinterpret_cast<const f16x8_t*>(hsrc + g.abase[i] + toff[tap] + ks * 32);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bq[u & 3][j], acc[i][j], 0, 0, 0);
      if (u + 4 < 8) {
        load_step(bq[u & 3], c, (u + 4) >> 1, ks);
      } else {
        load_step(bq[u & 3], cn, (u + 4 - 8) >> 1, ks);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  }
}

// 1x1x1 segment over raw input (the shortcut of a block whose width
// changes) for 8-wave workgroups: per chunk two k16 steps, B one chunk
// ahead, the next chunk's halo loaded and stored within the chunk.
template <int BK, int MI, int NJ, class G>
__device__ __forceinline__ void run_111_lean(const G& g, f32x16_t (&acc)[MI][NJ], int nchunks, int nitems) {
  static_assert(BK == 32, "two k16 steps per chunk");
  constexpr int NT = G::NT;
  const int ipt = (nitems + NT - 1) / NT;
  f16x8_t bq[2][NJ];
  auto load_step = [&](f16x8_t (&b)[NJ], int chunk, int ks) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int soff = ((chunk * 2 + ks) * g.wtaps + g.tap0) * 1024;
      b[j] = __builtin_bit_cast(f16x8_t, __builtin_amdgcn_raw_buffer_load_b128(g.wrsrc, g.bvoff[j], soff, 0));
    }
  };
  load_step(bq[0], 0, 0);
  load_step(bq[1], 0, 1);
  for (int c = 0; c < nchunks; ++c) {
    const unsigned char* hsrc = g.halo0 + (c & 1) * g.halo_bytes;
    unsigned char* hdst = g.halo0 + ((c + 1) & 1) * g.halo_bytes;
    const bool hnext = c + 1 < nchunks;
    for (int k = 0; k < ipt && hnext; ++k) {
      const int idx = g.tid + NT * k;
      halo_store<false, false>(g, idx, c + 1, halo_load(g, idx, c + 1), hdst);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      f16x8_t av[MI];
#pragma unroll
      for (int i = 0; i < MI; ++i) av[i] = *reinterpret_cast<const f16x8_t*>(hsrc + g.abase[i] + ks * 32);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bq[ks][j], acc[i][j], 0, 0, 0);
      if (hnext) load_step(bq[ks], c + 1, ks);
    }
    __syncthreads();
  }
}

// Any tap set (KT x K2 x K2, phases), B one tap ahead, halo items spread over
// the taps.  B comes from fragment-order weights (WFRAG) or from a row-major
// operand read with plain loads.
template <int BK, int MI, int NJ, bool NORM, bool ACT, bool WFRAG, class G>
__device__ __forceinline__ void run_generic(const G& g, f32x16_t (&acc)[MI][NJ], int nchunks,
                                            int ntaps, int KT, int K2, int KSm, int HY, int HX, int py, int px,
                                            int nitems, const h16_t* const (&bsrc)[NJ], const bool (&bok)[NJ]) {
  constexpr int ROWB = BK * 2 + 16;
  constexpr int KS = BK / 16;
  constexpr int NT = G::NT;
  const int ipt = (nitems + NT - 1) / NT;
  const int per_tap = (ipt + ntaps - 1) / ntaps;
  auto load_b = [&](f16x8_t (&b)[NJ][KS], int chunk, int tap) {
    if constexpr (WFRAG) {
      load_b_frag<BK, NJ>(g, b, chunk, tap);
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) b[j][ks] = bok[j] ? ld_frag(bsrc[j] + chunk * BK + ks * 16) : f16x8_t{};
    }
  };
  f16x8_t bc[NJ][KS], bn[NJ][KS];
  load_b(bc, 0, 0);
  for (int c = 0; c < nchunks; ++c) {
    const unsigned char* hsrc = g.halo0 + (c & 1) * g.halo_bytes;
    unsigned char* hdst = g.halo0 + ((c + 1) & 1) * g.halo_bytes;
    const bool hnext = c + 1 < nchunks;
    for (int t = 0; t < ntaps; ++t) {
      int cn = c, tn = t + 1;
      if (tn == ntaps) { tn = 0; cn = c + 1; }
      if (cn < nchunks) load_b(bn, cn, tn);
      uint4 hr[kMaxHaloItemsPerTap];
      const int j0 = t * per_tap;
      if (hnext) {
#pragma unroll
        for (int k = 0; k < kMaxHaloItemsPerTap; ++k)
          if (k < per_tap && j0 + k < ipt) hr[k] = halo_load(g, g.tid + NT * (j0 + k), c + 1);
      }
      const int dt = t / (K2 * K2);
      const int a2 = (t / K2) % K2;
      const int b2 = t % K2;
      const int dy = KSm == 2 ? py + a2 : a2;
      const int dx = KSm == 2 ? px + b2 : b2;
      mma_tap<BK, MI, NJ>(g, acc, hsrc, ((dt * HY + dy) * HX + dx) * ROWB, bc);
      if (hnext) {
#pragma unroll
        for (int k = 0; k < kMaxHaloItemsPerTap; ++k)
          if (k < per_tap && j0 + k < ipt)
            halo_store<NORM, ACT>(g, g.tid + NT * (j0 + k), c + 1, hr[k], hdst);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bc[j][ks] = bn[j][ks];
    }
    __syncthreads();
  }
}

// MODE: 0 any tap set, 1 specialised 3x3x3 (2 x 8 x 16 tiles), 2 specialised
// up-conv phase (1 x 16 x 16 tiles).  PRO0: prologue of segment 0 fixed at
// compile time (PRO_RAW, PRO_NORM, PRO_NORM_SILU) or -1 to take it from the
// arguments.
template <int BK, int BN, int WAVES_N, int NW, int MODE, int PRO0>
__global__ __launch_bounds__(NW * 64) void conv_igemm(ConvArgs a) {
  constexpr int NT = NW * 64;           // threads per workgroup
  constexpr int NP = BK / 8;            // 16-byte parts per voxel row
  constexpr int ROWB = BK * 2 + 16;     // padded LDS row (bytes)
  constexpr int WAVES_M = NW / WAVES_N;
  constexpr int WM = kTileM / WAVES_M;
  constexpr int WN = BN / WAVES_N;
  constexpr int MI = WM / 32;
  constexpr int NJ = WN / 32;

  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_m = wave / WAVES_N;
  const int wave_n = wave % WAVES_N;

  // ---- LDS carve-up: two halo buffers, then the per-voxel tables ----
  const int halo_bytes = a.nhv_max * ROWB;
  const h16_t** vptr_s = reinterpret_cast<const h16_t**>(smem + 2 * halo_bytes);
  float* rs_s = reinterpret_cast<float*>(vptr_s + a.nhv_max);
  float* gamma_s = rs_s + a.nhv_max;

  // ---- tile coordinates; consecutive logical tiles share an XCD ----
  const int nM = a.tiles_x * a.tiles_y * a.tiles_f;
  const int nN = (a.Cout + BN - 1) / BN;
  const int total = nM * nN * a.nphase;
  int logical;
  {
    const int id = blockIdx.x;
    const int q = total >> 3, r = total & 7, xcd = id & 7, slot = id >> 3;
    logical = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + slot;
  }
  const int nt = logical % nN;
  const int ph = (logical / nN) % a.nphase;
  const int mt = logical / (nN * a.nphase);
  const int py = ph >> 1, px = ph & 1;
  constexpr bool K333 = MODE == 1;
  const int TF = K333 ? kTF333 : (MODE == 2 ? 1 : a.TF);
  const int TH = K333 ? kTH333 : (MODE == 2 ? 16 : a.TH);
  const int txi = mt % a.tiles_x;
  const int tyi = (mt / a.tiles_x) % a.tiles_y;
  const int tfi = mt / (a.tiles_x * a.tiles_y);
  const int f0 = tfi * TF, y0 = tyi * TH, x0 = txi * kTileW;
  const int n0 = nt * BN;
  const int HW = a.H * a.W;
  const int kpart = lane >> 5;  // which 8-wide K group of a k16 step this lane feeds
  const int lrow = lane & 31;
  const int ncol0 = n0 + wave_n * WN;  // first output channel of this wave

  f32x16_t acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Segments run as straight-line code (segment 0, then the optional second
  // one), so the register allocator sees each tap loop on its own.
  auto do_segment = [&](const int s) {
    const ConvSeg& S = a.seg[s];
    const bool spec = K333 && s == 0;  // the specialised 3x3x3 segment
    const int KT = spec ? 3 : S.KT;
    const int hs = spec ? 1 : (S.KS == 1 ? 0 : 1);
    const int K2 = spec ? 3 : (S.KS == 3 ? 3 : (S.KS == 2 ? 2 : 1));
    const int st = S.stride == 2 ? 2 : 1;   // input rows/columns per output row/column
    const int HX = st * kTileW + 2 * hs - (st - 1);
    const int HY = st * TH + 2 * hs - (st - 1);
    const int IH = st * a.H, IW = st * a.W;  // input grid
    const int HF = TF + KT - 1;
    const int nhv = HF * HY * HX;
    const int ntaps = KT * K2 * K2;
    const int nchunks = S.Cin / BK;
    const int pro = (PRO0 >= 0 && s == 0) ? PRO0 : S.prologue;
    const bool norm = pro != PRO_RAW;

    __syncthreads();  // the previous segment (or tile setup) is done with LDS
    // Per-halo-row source pointer and norm scale.  Padding voxels and the
    // spare rows past the halo read the zero row with scale 0, so the item
    // loops need no per-lane branches.
    for (int v = tid; v < a.nhv_max; v += NT) {
      const h16_t* p = a.zero_row;
      float rsv = 0.0f;
      if (v < nhv) {
        const int hx = v % HX;
        const int t2 = v / HX;
        const int hy = t2 % HY;
        const int hf = t2 / HY;
        const int fo = f0 + hf - (KT - 1);
        const int y = st * y0 + hy - hs;
        const int x = st * x0 + hx - hs;
        if (y >= 0 && y < IH && x >= 0 && x < IW && fo < a.F) {
          const long long pix = (long long)y * IW + x;
          const h16_t* q = nullptr;
          if (fo >= 0) {
            q = S.x + fo * S.x_fstride + pix * S.lda;
          } else if (fo + 2 >= 2 - S.n_hist) {
            q = S.ring + (long long)(fo + 2) * HW * S.Cin + pix * S.Cin;
          }
          if (q) {
            p = q;
            if (norm) rsv = S.rs[(long long)(fo + 2) * HW + pix];
          }
        }
      }
      vptr_s[v] = p;
      rs_s[v] = rsv;
    }
    if (norm)
      for (int c = tid; c < S.Cin; c += NT) gamma_s[c] = S.gamma[c];
    __syncthreads();

    SegCtx<BK, MI, NJ, NT> g;
    g.halo0 = smem;
    g.halo_bytes = halo_bytes;
    g.vptr = vptr_s;
    g.rs = rs_s;
    g.gamma = gamma_s;
    g.tid = tid;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int m = wave_m * WM + 32 * i + lrow;
      const int tx = m & (kTileW - 1);
      const int t2 = m / kTileW;
      g.abase[i] = (((t2 / TH) * HY + st * (t2 % TH)) * HX + st * tx) * ROWB + kpart * 16;
    }
    const int U = S.Cin / 16;
    g.wtaps = a.nphase * ntaps;
    g.tap0 = ph * ntaps;
    g.wrsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<h16_t*>(S.w), 0, (int)S.w_bytes, 0x00020000);
    const h16_t* bsrc[NJ];
    bool bok[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int nb = ncol0 / 32 + j;
      g.bvoff[j] = (nb * U * g.wtaps) * 1024 + lane * 16;
      const int n = ncol0 + 32 * j + lrow;
      bok[j] = n < a.Cout;
      bsrc[j] = S.w + (long long)f0 * S.w_frame_stride + (long long)n * S.ldw + kpart * 8;
    }

    // Chunk 0 halo, synchronously (all rows, spare ones included).
    const int rows_items = a.nhv_max * NP;
    if (pro == PRO_NORM_SILU) {
      for (int idx = tid; idx < rows_items; idx += NT)
        halo_store<true, true>(g, idx, 0, halo_load(g, idx, 0), g.halo0);
    } else if (pro == PRO_NORM) {
      for (int idx = tid; idx < rows_items; idx += NT)
        halo_store<true, false>(g, idx, 0, halo_load(g, idx, 0), g.halo0);
    } else {
      for (int idx = tid; idx < rows_items; idx += NT)
        halo_store<false, false>(g, idx, 0, halo_load(g, idx, 0), g.halo0);
    }
    __syncthreads();

    if constexpr (K333) {
      if (s == 0) {
        constexpr bool kNorm = PRO0 == PRO_NORM || PRO0 == PRO_NORM_SILU;
        constexpr bool kAct = PRO0 == PRO_NORM_SILU;
        run_333<BK, MI, NJ, kNorm, kAct, kBRing>(g, acc, nchunks);
        return;
      }
    }
    const int nitems = nhv * NP;
    if constexpr (MODE == 2) {
      run_phase<BK, MI, NJ>(g, acc, nchunks, py, px, nitems);
      return;
    }
    if constexpr (NW == 8) {
      // the 8-wave kernel's only other segment: a raw 1x1x1 shortcut
      run_111_lean<BK, MI, NJ>(g, acc, nchunks, nitems);
      return;
    }
    if (S.wfrag) {
      if (pro == PRO_NORM_SILU)
        run_generic<BK, MI, NJ, true, true, true>(g, acc, nchunks, ntaps, KT, K2, S.KS, HY, HX, py, px, nitems,
                                                   bsrc, bok);
      else if (pro == PRO_NORM)
        run_generic<BK, MI, NJ, true, false, true>(g, acc, nchunks, ntaps, KT, K2, S.KS, HY, HX, py, px, nitems,
                                                    bsrc, bok);
      else
        run_generic<BK, MI, NJ, false, false, true>(g, acc, nchunks, ntaps, KT, K2, S.KS, HY, HX, py, px, nitems,
                                                     bsrc, bok);
    } else {
      run_generic<BK, MI, NJ, false, false, false>(g, acc, nchunks, ntaps, KT, K2, S.KS, HY, HX, py, px, nitems,
                                                    bsrc, bok);
    }
  };
  do_segment(0);
  if (a.nseg > 1) do_segment(1);

  // ---- epilogue ----
  // Each wave moves one 32-row block of its accumulators at a time through
  // its own LDS region (compile-time register indices only), then every lane
  // takes one output voxel and a contiguous run of CPL channels, so stores go
  // out as 16-byte vectors along the channel axis.
  constexpr int CPL = WN / 2;          // channels per lane in the store phase
  constexpr int EROW = WN + 4;         // padded LDS row (floats)
  __syncthreads();                     // all waves are done with the halo tiles
  float* ep = reinterpret_cast<float*>(smem) + wave * 32 * EROW;
  const int er = lane >> 1;            // row of the block this lane stores
  const int ec0 = (lane & 1) * CPL;    // first column of the block this lane stores
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        ep[(8 * (e >> 2) + 4 * kpart + (e & 3)) * EROW + 32 * j + lrow] = acc[i][j][e];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the block is in LDS
    __builtin_amdgcn_wave_barrier();
    const int m = wave_m * WM + 32 * i + er;
    const int tx = m & (kTileW - 1);
    const int t2 = m / kTileW;
    const int f = f0 + t2 / TH, y = y0 + t2 % TH, x = x0 + tx;
    const int nb = ncol0 + ec0;  // first output channel of this lane
    if (f < a.F && y < a.H && x < a.W && nb < a.Cout) {
      const long long pix = (long long)y * a.W + x;
      const float* row = ep + er * EROW + ec0;
      if (a.epi == EPI_VIDEO) {
        for (int c = 0; c < CPL && nb + c < a.Cout; ++c) {
          const int n = nb + c;
          float v = row[c] * a.scale + (a.bias ? a.bias[n] : 0.0f);
          v = clamp_unit(v);
          const int k = n >> 2, ddy = (n >> 1) & 1, ddx = n & 1;
          const long long r2 = ((long long)k * a.video_T + a.out_base + f) * (2 * a.H) + 2 * y + ddy;
          static_cast<bf16_t*>(a.out)[r2 * (2 * a.W) + 2 * x + ddx] = (bf16_t)f2bf(v);
        }
      } else if (a.epi == EPI_F32) {
        float* o = static_cast<float*>(a.out) + f * a.out_fstride + pix * a.ldo;
        for (int c = 0; c < CPL && nb + c < a.Cout; ++c)
          o[nb + c] = row[c] * a.scale + (a.bias ? a.bias[nb + c] : 0.0f);
      } else if (a.epi == EPI_LATENT) {
        float* o = static_cast<float*>(a.out);
        for (int c = 0; c < CPL && nb + c < a.Cout; ++c) {
          const int n = nb + c;
          o[((long long)n * a.video_T + a.out_base + f) * HW + pix] = row[c] * a.scale + (a.bias ? a.bias[n] : 0.0f);
        }
      } else {
        // fp16 channels-last destinations: plain, time-interleaved or phase.
        h16_t* o;
        int nc = nb;
        if (a.epi == EPI_TIME) {
          const int Chalf = a.Cout >> 1;
          const int half = nb >= Chalf ? 1 : 0;
          nc = nb - half * Chalf;
          o = static_cast<h16_t*>(a.out) + (long long)(a.out_base + 2 * f + half) * a.out_fstride + pix * a.ldo;
        } else if (a.epi == EPI_PHASE) {
          const long long op = (long long)(2 * y + py) * (2 * a.W) + (2 * x + px);
          o = static_cast<h16_t*>(a.out) + f * a.out_fstride + op * a.ldo;
        } else {
          o = static_cast<h16_t*>(a.out) + f * a.out_fstride + pix * a.ldo;
        }
        const h16_t* rp = a.res ? a.res + f * a.res_fstride + pix * a.ldr + nb : nullptr;
        const bool full = nb + CPL <= a.Cout;
        for (int c8 = 0; c8 < CPL; c8 += 8) {
          float v[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) v[k] = row[c8 + k] * a.scale;
          if (full) {
            if (a.bias) {
#pragma unroll
              for (int k = 0; k < 8; ++k) v[k] += a.bias[nb + c8 + k];
            }
            if (rp) {
              float r[8];
              unpack8h(*reinterpret_cast<const uint4*>(rp + c8), r);
#pragma unroll
              for (int k = 0; k < 8; ++k) v[k] += r[k];
            }
            *reinterpret_cast<uint4*>(o + nc + c8) = pack8h(v);
          } else {
            for (int k = 0; k < 8 && nb + c8 + k < a.Cout; ++k) {
              float t = v[k] + (a.bias ? a.bias[nb + c8 + k] : 0.0f);
              if (rp) t += h2f(rp[c8 + k]);
              o[nc + c8 + k] = (h16_t)f2h(t);
            }
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ---------------------------------------------------------------------------
// Persistent 8-wave kernel for the specialised one-segment convs (3x3x3 and
// up-conv phase).  One workgroup per CU walks its XCD's share of the tiles;
// while a tile's last chunk is multiplied, the next tile's first halo chunk
// and B fragments stream in, and the halo tables of the tile after next are
// built during the epilogue.  A tile switch then costs only the epilogue,
// not a workgroup launch, two table/halo round trips and a B refill.

// Work split: the 8 XCDs take contiguous ranges of logical tiles in
// proportion to their workgroup count; workgroup `slot` of an XCD takes
// tiles start + slot, start + slot + n, ... so the tiles running at one time
// on an XCD are neighbours (shared weights and halos in its L2).
struct TileSeq {
  int start, end, slot, n;
  __device__ int at(int k) const {
    const int t = start + slot + k * n;
    return t < end ? t : -1;
  }
};

__device__ __forceinline__ TileSeq tile_seq(int total) {
  const int G = gridDim.x, b = blockIdx.x, xcd = b & 7;
  int before = 0;
  for (int x = 0; x < xcd; ++x) before += (G - x + 7) >> 3;
  const int n = (G - xcd + 7) >> 3;
  TileSeq s;
  s.start = (int)((long long)total * before / G);
  s.end = (int)((long long)total * (before + n) / G);
  s.slot = b >> 3;
  s.n = n;
  return s;
}

// Output tile of a logical tile index.
struct TileGeo {
  int f0, y0, x0, n0, ph;
};

template <int BN, int MODE, int TW = kTileW, int TF4 = kTFWino>
__device__ __forceinline__ TileGeo tile_geo(const ConvArgs& a, int logical) {
  constexpr bool TYX = MODE == 4 || MODE == 5;  // (t, y) taps over whole columns
  constexpr int TF = MODE == 2 ? 1 : (TYX ? TF4 : kTF333);
  constexpr int TH = MODE == 2 ? 16 : (TYX ? kTileM / TW / TF4 : kTH333);
  // the head's tiles overlap: columns x0 .. x0 + TW - 1 make outputs x0 + 1 ..
  // x0 + TW - 2, so tile tx starts at column (TW - 2) tx - 1
  constexpr int XSTEP = MODE == 5 ? TW - 2 : TW, XOFF = MODE == 5 ? -1 : 0;
  // Output positions vary fastest: the tiles running together on an XCD
  // share one (phase, channel block) of weights in its L2 and neighbouring
  // halos (interleaving the phases made them stream one weight set per phase).
  const int nN = (a.Cout + BN - 1) / BN;
  const int nMt = a.tiles_x * a.tiles_y * a.tiles_f;
  const int mt = logical % nMt;
  const int nt = (logical / nMt) % nN;
  const int ph = logical / (nMt * nN);
  TileGeo t;
  if (MODE == 2) {  // no temporal halo: rows of x-neighbours (shared x halo)
    t.x0 = (mt % a.tiles_x) * TW;
    t.y0 = ((mt / a.tiles_x) % a.tiles_y) * TH;
    t.f0 = (mt / (a.tiles_x * a.tiles_y)) * TF;
  } else {  // temporal taps: frames fastest, so the tiles that share their
            // history frames run together and read them from one L2
    t.f0 = (mt % a.tiles_f) * TF;
    t.x0 = ((mt / a.tiles_f) % a.tiles_x) * XSTEP + XOFF;
    t.y0 = (mt / (a.tiles_f * a.tiles_x)) * TH;
  }
  t.n0 = nt * BN;
  t.ph = ph;
  return t;
}

template <int BN, int WAVES_N, int MODE, int PRO0, int NW = 8, int TWW = kTileW, int TFW = kTFWino>
__global__ __launch_bounds__(NW * 64) void conv_persist(ConvArgs a) {
  constexpr int BK = 32, NT = NW * 64, NP = 4;
  // With 4 waves (one per SIMD, 512 registers: accumulators in AGPRs) each
  // wave owns a 128 x 128 sub-tile and reads its A fragments one k16 step
  // ahead; with 8 waves the second wave on the SIMD hides that latency.
  constexpr bool APF = NW == 4;
  constexpr int ROWB = BK * 2 + 16;
  constexpr int WAVES_M = NW / WAVES_N;
  constexpr int WM = kTileM / WAVES_M;
  constexpr int WN = BN / WAVES_N;
  constexpr int MI = WM / 32;
  constexpr int NJ = WN / 32;
  constexpr bool K333 = MODE == 1;
  constexpr bool NORM = PRO0 == PRO_NORM || PRO0 == PRO_NORM_SILU;
  constexpr bool ACT = PRO0 == PRO_NORM_SILU;
  constexpr bool KT3 = MODE == 3;   // 3x1x1 temporal conv (time_conv)
  // Winograd-domain 3x3x1 (t, y) GEMM, one xi per phase; the same loop runs
  // the head (MODE 5: input columns, the x taps in the output columns)
  constexpr bool HEADX = MODE == 5;
  constexpr bool WINO = MODE == 4 || HEADX;
  // the Winograd and phase loops pass B as the MFMA's first operand: rows of
  // the product are output channels, columns output positions
  constexpr bool SWAPPED = WINO || MODE == 2;
  constexpr int TW = WINO ? TWW : kTileW;  // tile columns (Winograd: column groups)
  static_assert(WINO || (TWW == kTileW && TFW == kTFWino), "tile shape choice is the Winograd GEMM's");
  constexpr int TF = MODE == 2 ? 1 : (WINO ? TFW : kTF333);
  constexpr int TH = MODE == 2 ? 16 : (WINO ? kTileM / TW / TFW : kTH333);
  constexpr int KT = MODE == 2 ? 1 : 3;
  constexpr int HSX = KT3 || WINO ? 0 : 1;  // spatial halo along x
  constexpr int HSY = KT3 ? 0 : 1;          // and along y
  constexpr int HX = TW + 2 * HSX, HY = TH + 2 * HSY, HF = TF + KT - 1;
  constexpr int NHV = HF * HY * HX;
  constexpr int NTAPS = K333 ? 27 : (KT3 ? 3 : (WINO ? 9 : 4));
  static_assert(MODE >= 1 && MODE <= 5, "specialised tap sets only");
  static_assert(WN % 32 == 0 && MI >= 1, "wave tile");

  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_m = wave / WAVES_N;
  const int wave_n = wave % WAVES_N;
  const int kpart = lane >> 5;
  const int lrow = lane & 31;
  const ConvSeg& S = a.seg[0];

  // LDS: halo[2] | vptr[2][nhv_max] | rs[2][nhv_max] | gamma[Cin]
  const int nhv_max = a.nhv_max;
  const int halo_bytes = nhv_max * ROWB;
  const h16_t** vptr_s = reinterpret_cast<const h16_t**>(smem + 2 * halo_bytes);
  float* rs_s = reinterpret_cast<float*>(vptr_s + 2 * nhv_max);
  float* gamma_s = rs_s + 2 * nhv_max;
  const int HW = a.H * a.W;
  const int nchunks = S.Cin / BK;
  const int nN = (a.Cout + BN - 1) / BN;
  const int total = a.tiles_x * a.tiles_y * a.tiles_f * nN * a.nphase;
  const TileSeq seq = tile_seq(total);
  if (seq.at(0) < 0) return;  // uniform: no tile for this workgroup

  // Halo table of tile `logical` into table set `tb`: per halo row the
  // source pointer and (norm) scale; padding voxels read the zero row.
  auto build_tables = [&](int tb, int logical) {
    const TileGeo t = tile_geo<BN, MODE, TW, TF>(a, logical);
    for (int v = tid; v < nhv_max; v += NT) {
      const h16_t* p = a.zero_row;
      float rsv = 0.0f;
      if (v < NHV) {
        const int hx = v % HX;
        const int t2 = v / HX;
        const int hy = t2 % HY;
        const int hf = t2 / HY;
        const int fo = t.f0 + hf - (KT - 1);
        const int y = t.y0 + hy - HSY;
        const int x = t.x0 + hx - HSX;
        if (y >= 0 && y < a.H && x >= 0 && x < a.W && fo < a.F) {
          const long long pix = (long long)y * a.W + x;
          const h16_t* q = nullptr;
          if (fo >= 0) {
            q = S.x + t.ph * S.x_pstride + fo * S.x_fstride + pix * S.lda;
          } else if (fo + 2 >= 2 - S.n_hist) {
            q = S.ring + t.ph * S.x_pstride + (long long)(fo + 2) * HW * S.Cin + pix * S.Cin;
          }
          if (q) {
            p = q;
            if (NORM) rsv = S.rs[(long long)(fo + 2) * HW + pix];
          }
        }
      }
      vptr_s[tb * nhv_max + v] = p;
      rs_s[tb * nhv_max + v] = rsv;
    }
  };

  // Per-tile fragment addressing (A rows are the same for every tile).
  SegCtx<BK, MI, NJ, NT> g0;
  g0.halo0 = smem;
  g0.halo_bytes = halo_bytes;
  g0.gamma = gamma_s;
  g0.tid = tid;
  g0.wtaps = a.nphase * NTAPS;
  g0.wrsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<h16_t*>(S.w), 0, (int)S.w_bytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int m = wave_m * WM + 32 * i + lrow;
    const int tx = m & (TW - 1);
    const int t2 = m / TW;
    g0.abase[i] = (((t2 / TH) * HY + (t2 % TH)) * HX + tx) * ROWB + kpart * 16;
  }
  const int U = S.Cin / 16;
  auto ctx_for = [&](int logical, int tb) {
    SegCtx<BK, MI, NJ, NT> g = g0;
    const TileGeo t = tile_geo<BN, MODE, TW, TF>(a, logical);
    g.vptr = vptr_s + tb * nhv_max;
    g.rs = rs_s + tb * nhv_max;
    g.tap0 = t.ph * NTAPS;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int nb = (t.n0 + wave_n * WN) / 32 + j;
      g.bvoff[j] = (nb * U * g.wtaps) * 1024 + lane * 16;
    }
    return g;
  };

  f16x8_t bq[kBRing][NJ];
  auto load_step = [&](const SegCtx<BK, MI, NJ, NT>& g, f16x8_t (&b)[NJ], int chunk, int tap, int ks) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int soff = ((chunk * 2 + ks) * g.wtaps + g.tap0 + tap) * 1024;
      b[j] = __builtin_bit_cast(f16x8_t, __builtin_amdgcn_raw_buffer_load_b128(g.wrsrc, g.bvoff[j], soff, 0));
    }
  };

  // ---- first tile: tables of tiles 0 and 1, synchronous first halo chunk ----
  if (NORM)
    for (int c = tid; c < S.Cin; c += NT) gamma_s[c] = S.gamma[c];
  build_tables(0, seq.at(0));
  if (seq.at(1) >= 0) build_tables(1, seq.at(1));
  __syncthreads();
  {
    const SegCtx<BK, MI, NJ, NT> g = ctx_for(seq.at(0), 0);
    for (int idx = tid; idx < nhv_max * NP; idx += NT)
      halo_store<NORM, ACT>(g, idx, 0, halo_load(g, idx, 0), smem);
    constexpr int PRE = K333 || WINO ? kBRing : (KT3 ? 3 : kPhaseBRing);
#pragma unroll
    for (int u = 0; u < PRE; ++u) {
      load_step(g, bq[u], 0, u >> 1, u & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();

  f32x16_t acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  int gc = 0;  // chunks done by this workgroup (halo buffer parity)
  for (int k = 0;; ++k) {
    const int cur = seq.at(k);
    if (cur < 0) break;
    const int nxt = seq.at(k + 1);
    const SegCtx<BK, MI, NJ, NT> g = ctx_for(cur, k & 1);
    // The last chunk prefetches the next tile's first chunk, or (no next
    // tile) streams its own halo and weights once more into the spare
    // buffer and ring slots: no branch, exact wait counters.
    const SegCtx<BK, MI, NJ, NT> gl = nxt >= 0 ? ctx_for(nxt, (k + 1) & 1) : g;
    const TileGeo geo = tile_geo<BN, MODE, TW, TF>(a, cur);

    for (int c = 0; c < nchunks; ++c, ++gc) {
      const bool last = c + 1 == nchunks;
      const SegCtx<BK, MI, NJ, NT>& gn = last ? gl : g;
      const int cn = last ? (nxt >= 0 ? 0 : c) : c + 1;
      const unsigned char* hsrc = smem + (gc & 1) * halo_bytes;
      unsigned char* hdst = smem + ((gc + 1) & 1) * halo_bytes;
      if constexpr (K333) {
        constexpr int IPT = (kNHV333 * NP + NT - 1) / NT;
        static_assert(IPT + 3 <= 27, "halo items must land inside a chunk");
        static_assert(6 % kBRing == 0, "slot s6 % kBRing must continue across tap groups");
        uint4 hr[3];
        f16x8_t ap[2][MI];  // A fragments one step ahead (APF)
        if constexpr (APF) {
#pragma unroll
          for (int i = 0; i < MI; ++i) ap[0][i] = *reinterpret_cast<const f16x8_t*>(hsrc + g.abase[i]);
        }
#pragma unroll
        for (int gi = 0; gi < 9; ++gi) {
          const int goff = ((gi / 3) * kHY333 + (gi % 3)) * kHX * ROWB;
#pragma unroll
          for (int s6 = 0; s6 < 6; ++s6) {
            const int dx = s6 >> 1, ks = s6 & 1;
            const int t = 3 * gi + dx;
            f16x8_t av[MI];
            if constexpr (APF) {
              const int u1 = 6 * gi + s6 + 1;  // next k16 step of this chunk
              if (u1 < 54) {
                const int g1 = u1 / 6, s1 = u1 % 6;
                const int off = ((g1 / 3) * kHY333 + (g1 % 3)) * kHX * ROWB + (s1 >> 1) * ROWB + (s1 & 1) * 32;
#pragma unroll
                for (int i = 0; i < MI; ++i)
                  ap[(s6 + 1) & 1][i] = *reinterpret_cast<const f16x8_t*>(hsrc + g.abase[i] + off);
              }
              __builtin_amdgcn_sched_barrier(0);
#pragma unroll
              for (int i = 0; i < MI; ++i) av[i] = ap[s6 & 1][i];
            } else {
#pragma unroll
              for (int i = 0; i < MI; ++i)
                av[i] = *reinterpret_cast<const f16x8_t*>(hsrc + g.abase[i] + goff + dx * ROWB + ks * 32);
            }
            // the halo item's normalisation shares the step with the MFMAs so
            // the scheduler can interleave its VALU work between them
            const bool hstore = ks == 0 && t >= 3 && t - 3 < IPT;
            if (hstore) halo_store<NORM, ACT>(gn, tid + NT * (t - 3), cn, hr[dx], hdst);
            if (ks == 0 && t < IPT) hr[dx] = halo_load(gn, tid + NT * t, cn);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
              for (int j = 0; j < NJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bq[s6 % kBRing][j], acc[i][j], 0, 0, 0);
            if (hstore) {
#pragma unroll
              for (int q = 0; q < MI * NJ; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, NORM ? 80 / (MI * NJ) : 1, 0);  // then VALU
              }
            }
            // refill with k16 step u + kBRing
            const int t3 = 3 * gi + (s6 + kBRing) / 2;
            const int ks3 = (s6 + kBRing) & 1;
            if (t3 < 27)
              load_step(g, bq[s6 % kBRing], c, t3, ks3);
            else
              load_step(gn, bq[s6 % kBRing], cn, t3 - 27, ks3);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      } else if constexpr (WINO) {
        // 9 (dt, dy) taps x two k16 steps over one xi plane; B fragments of
        // step u in slot u % 6, refilled with step u + 6 (three taps ahead);
        // IPK halo items loaded at each of taps 0..4 and stored three taps
        // later.  With APF (4 waves) A fragments run one step ahead.
        constexpr int IPT = (NHV * NP + NT - 1) / NT;
        constexpr int IPK = (IPT + 4) / 5;
        static_assert(IPK <= 2, "halo items per tap");
        static_assert(18 % kBRing == 0, "slot u % kBRing must continue across chunks");
        constexpr int LAGT = kWinoLag;
        static_assert(LAGT >= 1 && LAGT + 4 <= 8, "halo items stored inside the chunk");
        uint4 hr[LAGT][IPK];
        f16x8_t ap[2][MI];
        // Row addresses of a tap's halo items come from the LDS table one
        // step before their loads (tap 0's ahead of the chunk's first A
        // reads), so waiting for them never waits for A reads issued later.
        const h16_t* hp[2][IPK];
#pragma unroll
        for (int j = 0; j < IPK; ++j)
          if (j < IPT) hp[0][j] = halo_row(gn, tid + NT * j);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (APF) {
#pragma unroll
          for (int i = 0; i < MI; ++i) ap[0][i] = *reinterpret_cast<const f16x8_t*>(hsrc + g.abase[i]);
        }
#pragma unroll
        for (int u = 0; u < 18; ++u) {
          const int tap = u >> 1, ks = u & 1;
          const int dt = tap / 3, dy = tap % 3;
          f16x8_t av[MI];
          if constexpr (APF) {
            if (u + 1 < 18) {
              const int t1 = (u + 1) >> 1, k1 = (u + 1) & 1;
              const int off = ((t1 / 3) * HY + t1 % 3) * HX * ROWB + k1 * 32;
#pragma unroll
              for (int i = 0; i < MI; ++i)
                ap[(u + 1) & 1][i] = *reinterpret_cast<const f16x8_t*>(hsrc + g.abase[i] + off);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < MI; ++i) av[i] = ap[u & 1][i];
          } else {
            const int toff = (dt * HY + dy) * HX * ROWB;
#pragma unroll
            for (int i = 0; i < MI; ++i)
              av[i] = *reinterpret_cast<const f16x8_t*>(hsrc + g.abase[i] + toff + ks * 32);
          }
          if (ks == 0) {
#pragma unroll
            for (int j = 0; j < IPK; ++j) {
              const int is = (tap - LAGT) * IPK + j, il = tap * IPK + j;
              if (tap >= LAGT && is < IPT) halo_store<false, false>(gn, tid + NT * is, cn, hr[tap % LAGT][j], hdst);
              if (tap < 5 && il < IPT) hr[tap % LAGT][j] = halo_load_at<SegCtx<BK, MI, NJ, NT>>(hp[tap & 1][j], tid + NT * il, cn);
            }
          } else {
#pragma unroll
            for (int j = 0; j < IPK; ++j) {
              const int il = (tap + 1) * IPK + j;
              if (tap + 1 < 5 && il < IPT) hp[(tap + 1) & 1][j] = halo_row(gn, tid + NT * il);
            }
          }
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
              // operands swapped: rows of the product are output channels and
              // columns positions, so a lane's accumulators are runs of four
              // consecutive channels of one position
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bq[u % kBRing][j], av[i], acc[i][j], 0, 0, 0);
          if (u + kBRing < 18)
            load_step(g, bq[u % kBRing], c, (u + kBRing) >> 1, (u + kBRing) & 1);
          else
            load_step(gn, bq[u % kBRing], cn, (u + kBRing - 18) >> 1, (u + kBRing) & 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else if constexpr (KT3) {
        // three temporal taps x two k16 steps; B fragments of step u live in
        // slot u % 3 and are refilled with step u + 3 (half a chunk ahead)
        // halo items: two loads at each of steps 0 and 1, stored four steps
        // later (HBM latency covered by four steps of MFMAs)
        constexpr int IPT = (NHV * NP + NT - 1) / NT;
        static_assert(IPT >= 1 && IPT <= 4, "time_conv halo items per chunk");
        uint4 hr[4];
#pragma unroll
        for (int u = 0; u < 6; ++u) {
          const int tap = u >> 1, ks = u & 1;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int is = 2 * (u - 4) + q, il = 2 * u + q;
            if (u >= 4 && is < IPT) halo_store<false, false>(gn, tid + NT * is, cn, hr[is], hdst);
            if (u < 2 && il < IPT) hr[il] = halo_load(gn, tid + NT * il, cn);
          }
          const int toff = tap * (HY * HX) * ROWB;
          f16x8_t av[MI];
#pragma unroll
          for (int i = 0; i < MI; ++i)
            av[i] = *reinterpret_cast<const f16x8_t*>(hsrc + g.abase[i] + toff + ks * 32);
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bq[u % 3][j], acc[i][j], 0, 0, 0);
          if (u + 3 < 6)
            load_step(g, bq[u % 3], c, (u + 3) >> 1, (u + 3) & 1);
          else
            load_step(gn, bq[u % 3], cn, (u - 3) >> 1, (u - 3) & 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        // four 2x2 taps x two k16 steps on 8 waves; halo items are loaded
        // one per step over the first NLS steps and stored LAG steps later
        static_assert(!APF, "the phase loop runs on 8 waves");
        constexpr int IPT = ((1 * 18 * 18) * NP + NT - 1) / NT;
        constexpr int PD = kPhaseBRing;  // B fragments of step u in slot u % PD, refilled with step u + PD
        static_assert(8 % PD == 0, "slot u % PD must continue across chunks");
        constexpr int NLS = IPT;
        constexpr int LAG = 8 - NLS;
        static_assert(NLS >= 1 && LAG >= 3, "phase halo items land inside a chunk");
        // the phase's (py, px) offset goes into the row bases once per chunk,
        // so each step's tap offset is an instruction immediate
        const int phoff = ((geo.ph >> 1) * HX + (geo.ph & 1)) * ROWB;
        const unsigned char* hph = hsrc + phoff;
        uint4 hr[IPT];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          f16x8_t av[MI];
          {
            const int tap = u >> 1;
            const int o = ((tap >> 1) * HX + (tap & 1)) * ROWB + (u & 1) * 32;
#pragma unroll
            for (int i = 0; i < MI; ++i) av[i] = *reinterpret_cast<const f16x8_t*>(hph + g.abase[i] + o);
          }
          {
            const int is = u - LAG, il = u;
            if (u >= LAG && is < IPT) halo_store<false, false>(gn, tid + NT * is, cn, hr[is], hdst);
            if (u < NLS && il < IPT) hr[il] = halo_load(gn, tid + NT * il, cn);
          }
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bq[u % PD][j], av[i], acc[i][j], 0, 0, 0);  // swapped, as below
          if (u + PD < 8)
            load_step(g, bq[u % PD], c, (u + PD) >> 1, (u + PD) & 1);
          else
            load_step(gn, bq[u % PD], cn, (u + PD - 8) >> 1, (u + PD) & 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __syncthreads();  // next chunk's halo complete; this chunk's reads done
    }

    // Tables of the tile after next go into this tile's (now unused) set.
    const int nn = seq.at(k + 2);
    if (nn >= 0) build_tables(k & 1, nn);

    if constexpr (HEADX) {
      // ---- epilogue of the head: the partial sums P[m][12 dx + co] of the
      // tile's TW columns (one extra on each side of its TW - 2 outputs) go to
      // LDS (fp32, 40 of the 64 columns: 36 used); output column x of a row is
      // P[x - 1][co] + P[x][12 + co] + P[x + 1][24 + co] + bias, clamped and
      // stored as a bf16 pair of one video row (co = 4k + 2 dy + (0, 1):
      // colour k, row 2y + dy, pixels 2x and 2x + 1).  A row of TW positions
      // lies inside one wave's 32-row block, so each wave combines its own.
      static_assert(BN == 64 && NJ == 2 && WN == 64 && WM == 64 && MI == 2 && TW == 16, "head tile");
      constexpr int PROW = 44;                        // staged row: 40 floats + pad (conflict-free)
      constexpr int NROW = WM / TW;                   // rows of TW positions per wave
      constexpr int NITEM = NROW * 6 * (TW - 2);      // (row, colour and video row, output column)
      static_assert(NW * WM * PROW * 4 <= kHeadXEpiBytes, "staged rows fit in one halo buffer");
      float* ep = reinterpret_cast<float*>(smem + ((gc - 1) & 1) * halo_bytes) + wave * WM * PROW;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            if (j == 1 && g4 > 0) continue;  // columns 40..63: zero weights
            const f32x16_t& c = acc[i][j];
            f32x4_t v = {c[4 * g4], c[4 * g4 + 1], c[4 * g4 + 2], c[4 * g4 + 3]};
            *reinterpret_cast<f32x4_t*>(ep + (32 * i + lrow) * PROW + 32 * j + 8 * g4 + 4 * kpart) = v;
          }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the rows are in LDS
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int rnd = 0; rnd < (NITEM + 63) / 64; ++rnd) {
        const int q = rnd * 64 + lane;
        const int ox = q % (TW - 2), t6 = q / (TW - 2);
        const int pr = t6 % 6, row = t6 / 6;  // pr = 2k + dy
        const int t2 = wave_m * NROW + row;   // (frame, row) of the tile
        const int f = geo.f0 + t2 / TH, y = geo.y0 + t2 % TH, x = geo.x0 + 1 + ox;
        if (q < NITEM && f < a.F && y < a.H && x < a.W) {
          const float* pp = ep + (row * TW + ox) * PROW + 2 * pr;
          const float2 p0 = *reinterpret_cast<const float2*>(pp);
          const float2 p1 = *reinterpret_cast<const float2*>(pp + PROW + 12);
          const float2 p2 = *reinterpret_cast<const float2*>(pp + 2 * PROW + 24);
          const int n = 2 * pr;
          const float v0 = clamp_unit((p0.x + p1.x + p2.x) * a.scale + (a.bias ? a.bias[n] : 0.0f));
          const float v1 = clamp_unit((p0.y + p1.y + p2.y) * a.scale + (a.bias ? a.bias[n + 1] : 0.0f));
          const long long r2 = ((long long)(pr >> 1) * a.video_T + a.out_base + f) * (2 * a.H) + 2 * y + (pr & 1);
          *reinterpret_cast<uint32_t*>(static_cast<bf16_t*>(a.out) + r2 * (2 * a.W) + 2 * x) =
              f2bf(v0) | (f2bf(v1) << 16);
        }
      }
      // the next tile's halo stores reuse this buffer after the tile barrier
      __builtin_amdgcn_s_waitcnt(0xc07f);
    } else if constexpr (WINO && NW == 4 && BN == 256) {
      // ---- epilogue of the Winograd-domain GEMM (plain fp16 products): lane
      // (kpart, lrow) of block (i, j) holds position 32i + lrow of the wave's
      // rows and channels 32j + 8g + 4*kpart + r (accumulator 4g + r).  Per
      // 32-row block the wave packs its accumulators to fp16 and writes them
      // as 8-byte runs into its own LDS rows (128 channels + 16 bytes of pad;
      // rows 16..31 swap the two halves of every 16-byte piece, so the 32
      // lanes of a write pass cover all 64 banks once), waits once, reads
      // 8 rows x 16 pieces (four rows per read, one 16-byte piece per lane),
      // waits once and stores the 16-byte pieces along the output rows.  The
      // stores go through a buffer resource at the tile's first output
      // element; positions outside the grid get an offset past its range, so
      // the hardware drops them and no lane branches.
      constexpr int EROWB = 128 * 2 + 16;
      static_assert(WN == 128 && NJ == 4 && NW * 32 * EROWB <= kSwapEpiBytes, "staged rows fit in one halo buffer");
      unsigned char* st = smem + ((gc - 1) & 1) * halo_bytes + wave * 32 * EROWB;
      const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
          static_cast<h16_t*>(a.out) + geo.ph * a.out_pstride + geo.f0 * a.out_fstride +
              ((long long)geo.y0 * a.W + geo.x0) * a.ldo + geo.n0 + wave_n * WN,
          0, 0x7fffffff, 0x00020000);
      const int lf = a.F - geo.f0, ly = a.H - geo.y0, lx = a.W - geo.x0;
      const unsigned ofs = (unsigned)a.out_fstride, ors_row = (unsigned)a.W * (unsigned)a.ldo;
      const int rsel = lrow >> 4;  // this lane's write rows: halves swapped
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int gp = 0; gp < 2; ++gp) {
            const f32x16_t& c = acc[i][j];
            float v8[8];
            // read each accumulator where it is used (the compiler would
            // otherwise copy all of them out of the AGPRs at the loop exit)
#pragma unroll
            for (int e = 0; e < 8; ++e) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v8[e]) : "a"(c[8 * gp + e]));
            const uint4 pk = pack8h(v8);  // channels 32j + 16gp + 4kpart + (0..3, 8..11)
            unsigned char* rowp = st + lrow * EROWB + (4 * j + 2 * gp) * 16;
            *reinterpret_cast<uint2*>(rowp + 8 * (kpart ^ rsel)) = make_uint2(pk.x, pk.y);
            *reinterpret_cast<uint2*>(rowp + 16 + 8 * (kpart ^ rsel)) = make_uint2(pk.z, pk.w);
          }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the block is in LDS
        __builtin_amdgcn_wave_barrier();
        uint4 pv[8];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          const uint4 q = *reinterpret_cast<const uint4*>(st + (rr * 4 + lane / 16) * EROWB + (lane % 16) * 16);
          pv[rr] = rr < 4 ? q : make_uint4(q.z, q.w, q.x, q.y);  // rows 16..31: halves back in order
        }
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          const int m = wave_m * WM + 32 * i + rr * 4 + lane / 16;
          const int tx = m & (TW - 1), t2 = m / TW;
          const int dy = t2 % TH, df = t2 / TH;
          const unsigned off = (unsigned)df * ofs + (unsigned)dy * ors_row + (unsigned)tx * (unsigned)a.ldo +
                               (unsigned)(lane % 16) * 8u;
          const bool ok = df < lf && dy < ly && tx < lx;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, pv[rr]), ors, ok ? off * 2u : 0x80000000u,
                                                 0, 0);
        }
        // the next block's writes reuse these rows: this block's reads first
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (SWAPPED) {
      // ---- epilogue of the swapped-operand loops (Winograd-domain GEMM on
      // 128-channel tiles, up-conv phases): lane (kpart, lrow) of block (i, j) holds position
      // 32i + lrow of the wave's rows and channels 32j + 8g + 4*kpart + r
      // (accumulator 4g + r).  Per 32 positions and SCH channels the wave
      // writes the runs of four straight from the accumulators into its own
      // fp32 LDS rows (16-byte writes), then reads eight channels per lane,
      // adds the bias, packs them to fp16 and stores 16 bytes per lane along
      // the output row.
      constexpr int JH = NW == 4 ? 2 : 1;   // channel blocks per staging round
      constexpr int SCH = 32 * JH;          // staged channels per row
      constexpr int SROW = SCH * 4 + 16;    // staged row bytes: fp32 + pad
      constexpr int LPR = SCH / 8;          // lanes per staged row (8 channels each)
      constexpr int RPI = 64 / LPR;         // rows per read
      static_assert(NJ % JH == 0 && 64 % LPR == 0, "staging split");
      static_assert(NW * 32 * SROW <= kSwapEpiBytes, "staged rows fit in one halo buffer (nhv_max)");
      unsigned char* st = smem + ((gc - 1) & 1) * halo_bytes + wave * 32 * SROW;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int jh = 0; jh < NJ / JH; ++jh) {
#pragma unroll
          for (int jj = 0; jj < JH; ++jj)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const f32x16_t& c = acc[i][jh * JH + jj];
              f32x4_t v = {c[4 * g4], c[4 * g4 + 1], c[4 * g4 + 2], c[4 * g4 + 3]};
              *reinterpret_cast<f32x4_t*>(st + lrow * SROW + (32 * jj + 8 * g4 + 4 * kpart) * 4) = v;
            }
          __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the block is in LDS
          __builtin_amdgcn_wave_barrier();
          const int ncol = geo.n0 + wave_n * WN + jh * SCH + (lane % LPR) * 8;
          float bv[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) bv[k] = 0.0f;
          if (!WINO && a.bias) {
            const f32x4_t b0 = *reinterpret_cast<const f32x4_t*>(a.bias + ncol);
            const f32x4_t b1 = *reinterpret_cast<const f32x4_t*>(a.bias + ncol + 4);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              bv[k] = b0[k];
              bv[4 + k] = b1[k];
            }
          }
#pragma unroll
          for (int rr = 0; rr < 32 / RPI; ++rr) {
            const int r = rr * RPI + lane / LPR;
            const float* row = reinterpret_cast<const float*>(st + r * SROW) + (lane % LPR) * 8;
            const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(row);
            const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(row + 4);
            const int m = wave_m * WM + 32 * i + r;
            const int tx = m & (TW - 1);
            const int t2 = m / TW;
            const int f = geo.f0 + t2 / TH, y = geo.y0 + t2 % TH, x = geo.x0 + tx;
            if (f < a.F && y < a.H && x < a.W) {
              float v8[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
              h16_t* o;
              if constexpr (WINO) {
                const long long pix = (long long)y * a.W + x;
                o = static_cast<h16_t*>(a.out) + geo.ph * a.out_pstride + f * a.out_fstride + pix * a.ldo;
              } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) v8[k] = v8[k] * a.scale + bv[k];
                // phase (py, px) of the 2x output, or (one phase) the plain grid
                const long long op = a.epi == EPI_PHASE
                                         ? (long long)(2 * y + (geo.ph >> 1)) * (2 * a.W) + (2 * x + (geo.ph & 1))
                                         : (long long)y * a.W + x;
                o = static_cast<h16_t*>(a.out) + f * a.out_fstride + op * a.ldo;
              }
              *reinterpret_cast<uint4*>(o + ncol) = pack8h(v8);
            }
          }
          // the next round's writes reuse these rows: this round's reads first
          __builtin_amdgcn_s_waitcnt(0xc07f);
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
      // ---- epilogue: 8-row quarters of each 32-row block through the last
      // chunk's halo buffer (free now), then 16-byte stores along channels ----
      constexpr int EROW = WN + 8;          // padded LDS row (floats)
      constexpr int LPR = 64 / 8;           // lanes per staged row
      constexpr int CPL = WN / LPR;         // channels per lane
      float* ep = reinterpret_cast<float*>(smem + ((gc - 1) & 1) * halo_bytes) + wave * 8 * EROW;
      const int er = lane / LPR;
      const int ec0 = (lane % LPR) * CPL;
      const int ncol0 = geo.n0 + wave_n * WN;
  #pragma unroll
      for (int i = 0; i < MI; ++i) {
  #pragma unroll
        for (int q = 0; q < 4; ++q) {
  #pragma unroll
          for (int j = 0; j < NJ; ++j)
  #pragma unroll
            for (int e = 4 * q; e < 4 * q + 4; ++e) ep[(4 * kpart + (e & 3)) * EROW + 32 * j + lrow] = acc[i][j][e];
          __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the rows are in LDS
          __builtin_amdgcn_wave_barrier();
          const int m = wave_m * WM + 32 * i + 8 * q + er;
          const int tx = m & (TW - 1);
          const int t2 = m / TW;
          const int f = geo.f0 + t2 / TH, y = geo.y0 + t2 % TH, x = geo.x0 + tx;
          const int nb = ncol0 + ec0;
          if (a.epi == EPI_VIDEO) {
            // head (12 channels): lane slot sl < 6 of the row's eight writes
            // colour sl / 2, video row 2y + sl % 2: channels 4k + 2dy + 0, 1
            // as one bf16 pair, so the eight rows of a quarter (consecutive
            // x) fill 32 contiguous bytes of each video row
            const int sl = lane % LPR;
            if (f < a.F && y < a.H && x < a.W && sl < 6) {
              const int kk = sl >> 1, ddy = sl & 1, n = 4 * kk + 2 * ddy;
              const float* rowv = ep + er * EROW + n - ncol0;
              const float v0 = clamp_unit(rowv[0] * a.scale + (a.bias ? a.bias[n] : 0.0f));
              const float v1 = clamp_unit(rowv[1] * a.scale + (a.bias ? a.bias[n + 1] : 0.0f));
              const long long r2 = ((long long)kk * a.video_T + a.out_base + f) * (2 * a.H) + 2 * y + ddy;
              *reinterpret_cast<uint32_t*>(static_cast<bf16_t*>(a.out) + r2 * (2 * a.W) + 2 * x) =
                  f2bf(v0) | (f2bf(v1) << 16);
            }
          } else if (f < a.F && y < a.H && x < a.W && nb < a.Cout) {
            const long long pix = (long long)y * a.W + x;
            const float* row = ep + er * EROW + ec0;
            if constexpr (CPL % 8 == 0) {
              h16_t* o;
              int ob = nb;  // output channel of this lane's first column
              if (a.epi == EPI_PHASE) {
                const long long op = (long long)(2 * y + (geo.ph >> 1)) * (2 * a.W) + (2 * x + (geo.ph & 1));
                o = static_cast<h16_t*>(a.out) + f * a.out_fstride + op * a.ldo;
              } else if (a.epi == EPI_WINO) {
                o = static_cast<h16_t*>(a.out) + geo.ph * a.out_pstride + f * a.out_fstride + pix * a.ldo;
              } else if (a.epi == EPI_TIME) {
                // channel half h of frame f -> output frame out_base + 2f + h
                const int Chalf = a.Cout >> 1;
                const int half = nb >= Chalf ? 1 : 0;
                ob = nb - half * Chalf;
                o = static_cast<h16_t*>(a.out) + (long long)(a.out_base + 2 * f + half) * a.out_fstride + pix * a.ldo;
              } else {
                o = static_cast<h16_t*>(a.out) + f * a.out_fstride + pix * a.ldo;
              }
              const h16_t* rp = a.res ? a.res + f * a.res_fstride + pix * a.ldr + nb : nullptr;
              const bool full = nb + CPL <= a.Cout;
  #pragma unroll
              for (int c8 = 0; c8 < CPL; c8 += 8) {
                float v[8];
  #pragma unroll
                for (int kk = 0; kk < 8; ++kk) v[kk] = row[c8 + kk] * a.scale;
                if (full) {
                  if (a.bias) {
  #pragma unroll
                    for (int kk = 0; kk < 8; ++kk) v[kk] += a.bias[nb + c8 + kk];
                  }
                  if (rp) {
                    float r[8];
                    unpack8h(*reinterpret_cast<const uint4*>(rp + c8), r);
  #pragma unroll
                    for (int kk = 0; kk < 8; ++kk) v[kk] += r[kk];
                  }
                  *reinterpret_cast<uint4*>(o + ob + c8) = pack8h(v);
                } else {
                  for (int kk = 0; kk < 8 && nb + c8 + kk < a.Cout; ++kk) {
                    float t = v[kk] + (a.bias ? a.bias[nb + c8 + kk] : 0.0f);
                    if (rp) t += h2f(rp[c8 + kk]);
                    o[ob + c8 + kk] = (h16_t)f2h(t);
                  }
                }
              }
            }
          }
          __builtin_amdgcn_wave_barrier();
        }
      }
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    // staging buffer and the new tables are complete before the next tile
    // stores halo rows into that buffer and reads those tables
    __syncthreads();
  }
}

template <int BN, int WAVES_N, int MODE, int PRO0, int NW = 8, int TW = kTileW, int TF = kTFWino>
hipError_t launch_persist_impl(const ConvArgs& a, hipStream_t stream) {
  if (g_dry_run) return hipSuccess;
  const size_t lds = conv_lds_bytes(a);
  auto kern = conv_persist<BN, WAVES_N, MODE, PRO0, NW, TW, TF>;
  static size_t attr_bytes = 0;
  if (lds > attr_bytes) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_bytes = lds;
  }
  const int nM = a.tiles_x * a.tiles_y * a.tiles_f;
  const int nN = (a.Cout + BN - 1) / BN;
  const long long total = (long long)nM * nN * a.nphase;
  if (total <= 0) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static int ncu[64] = {0};
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!ncu[dev]) {
    e = hipDeviceGetAttribute(&ncu[dev], hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
  }
  const long long grid = total < ncu[dev] ? total : ncu[dev];
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NW * 64), lds, stream, a);
  return hipGetLastError();
}

template <int BK, int BN, int WAVES_N, int NW, int MODE, int PRO0>
hipError_t launch_impl(const ConvArgs& a, hipStream_t stream) {
  if (g_dry_run) return hipSuccess;
  const size_t lds = conv_lds_bytes(a);
  auto kern = conv_igemm<BK, BN, WAVES_N, NW, MODE, PRO0>;
  static size_t attr_bytes = 0;
  if (lds > attr_bytes) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_bytes = lds;
  }
  const int nM = a.tiles_x * a.tiles_y * a.tiles_f;
  const int nN = (a.Cout + BN - 1) / BN;
  const long long total = (long long)nM * nN * a.nphase;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)total), dim3(NW * 64), lds, stream, a);
  return hipGetLastError();
}

int conv_bk(const ConvArgs& a) {
  for (int s = 0; s < a.nseg; ++s)
    if (a.seg[s].Cin % 32 || a.seg[s].stride == 2) return 16;  // strided halos are 4x larger: 16-channel chunks
  return 32;
}

// Kernel variant a launch runs on.
struct Variant {
  int bk, bn, nw;
  int mode;  // 0 generic, 1 3x3x3, 2 up-conv phase
};

Variant conv_variant(const ConvArgs& a) {
  const ConvSeg& g = a.seg[0];
  Variant v;
  v.bk = conv_bk(a);
  const bool k333 = g.KT == 3 && g.KS == 3 && a.TF == kTF333 && a.TH == kTH333 && v.bk == 32 && a.nphase == 1 &&
                    g.wfrag && (a.Cout > 32 ? (g.prologue == PRO_NORM_SILU || g.prologue == PRO_RAW)
                                            : (g.prologue == PRO_RAW && a.nseg == 1));
  // phase taps: the up-conv's four output phases, or one phase with a plain
  // store (a stride-2 conv in space-to-depth form)
  const bool kph = g.KT == 1 && g.KS == 2 && (a.nphase == 4 || (a.nphase == 1 && a.epi == EPI_H16)) &&
                   a.TF == 1 && a.TH == 16 && a.Cout > 32 &&
                   v.bk == 32 && a.nseg == 1 && g.wfrag && g.prologue == PRO_RAW;
  const bool kt3 = g.KT == 3 && g.KS == 1 && a.nphase == 1 && a.TF == kTF333 && a.TH == kTH333 && v.bk == 32 &&
                   a.nseg == 1 && g.wfrag && g.prologue == PRO_RAW && a.Cout % 256 == 0 && a.epi == EPI_TIME;
  const bool kwino = g.KT == 3 && g.KS == KS_3x1 && a.nphase == kWinoN && wino_tile_shape_ok(a.TF, a.TW) &&
                     a.TF * a.TH * a.TW == kTileM &&
                     v.bk == 32 && a.nseg == 1 && g.wfrag && g.prologue == PRO_RAW && a.Cout % 256 == 0 &&
                     a.epi == EPI_WINO;
  // the head with its x taps in the output columns: (t, y) taps over 16
  // input columns per tile row, 64 output columns (36 used)
  const bool khead = g.KT == 3 && g.KS == KS_3x1 && a.nphase == 1 && a.TF == 4 && a.TW == 16 && a.TH == 4 &&
                     a.Cout == 64 && v.bk == 32 && a.nseg == 1 && g.wfrag && g.prologue == PRO_RAW &&
                     a.epi == EPI_VIDEO;
  const bool shortcut_ok = a.nseg == 1 || (a.seg[1].KT == 1 && a.seg[1].KS == 1 && a.seg[1].prologue == PRO_RAW &&
                                            a.seg[1].wfrag && a.seg[1].Cin % 32 == 0);
  v.mode = k333 ? 1 : (kph ? 2 : (kt3 ? 3 : (kwino ? 4 : (khead ? 5 : 0))));
  if (v.mode == 5) {
    v.bn = 64;
    v.nw = 8;
  } else if (v.mode != 0 && a.Cout % 256 == 0 && shortcut_ok) {
    v.bn = 256;
    v.nw = 8;
  } else if (v.mode == 1 && a.Cout <= 32) {
    // narrow raw 3x3x3 (the head): one n32 block (the generic kernel runs it
    // as eight waves of 32 x 32, the persistent one as four of 64 x 32)
    v.bn = 32;
    v.nw = 8;
  } else {
    v.bn = a.Cout <= 32 ? 32 : 128;
    v.nw = 4;
  }
  return v;
}

// ---------------------------------------------------------------------------
// 1x1 convolution as a plain GEMM, out[m][n] = sum_k x[m][k] w[n][k] + bias[n]
// (the shortcut of a width-changing block).  It streams its activations from
// HBM once, so it is organised for that: one persistent workgroup per CU walks
// 256 x 256 tiles in K chunks of kS1K channels, a chunk stream that runs on
// from one tile into the next.  Two LDS buffers hold chunks g and g + 1 and two
// register sets stage the loads (8 coalesced 16-byte pieces of A rows and 8
// fragment-order weight blocks per thread): chunk g + 2 is issued at the start
// of chunk g and chunk g + 1 committed to LDS at its end, so every load has two
// chunks of MFMAs to arrive in and every CU keeps two chunks of loads in
// flight.  Four waves of 128 x 128 (accumulators in AGPRs, weights as the
// MFMA's first operand) read their fragments from LDS one k16 step ahead.
// A call is about 0.9 TFLOP over 5.4 GB at the c=256 shapes, so the MFMA and
// HBM floors (about 0.7 and 0.9 ms) are both close to its time (1.3 ms); the
// rolling pipeline measured 3 % faster than one 128-channel chunk per wait.
constexpr int kS1K = 64;                 // K channels per chunk
constexpr int kS1ARow = kS1K * 2 + 16;   // staged A row bytes (36 dwords: conflict-free fragment reads)
constexpr int kS1Buf = 256 * kS1ARow + 256 * kS1K * 2;
constexpr int kS1Lds = 2 * kS1Buf;

__global__ __launch_bounds__(256) void gemm1x1_kernel(const h16_t* __restrict__ x, long long M, int lda, int K,
                                                      const h16_t* __restrict__ w, int w_bytes, int N,
                                                      const float* __restrict__ bias, h16_t* __restrict__ out,
                                                      int ldo) {
  constexpr int MI = 4, NJ = 4, CS = kS1K / 16, PPR = kS1K * 2 / 16, IPT = 8;
  static_assert(PPR == 8 && CS == 4 && 256 * PPR == 256 * IPT, "8 A pieces (32 rows apart) and 8 B blocks per thread");
  extern __shared__ __align__(16) unsigned char g1s[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int kpart = lane >> 5, lrow = lane & 31;
  const int nN = N / 256;
  const long long nMt = (M + 255) / 256;
  const TileSeq seq = tile_seq((int)(nMt * nN));
  if (seq.at(0) < 0) return;
  const int nch = K / kS1K;  // even (the launcher checks)
  const int U = K / 16;
  const __amdgpu_buffer_rsrc_t brsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<h16_t*>(w), 0, w_bytes, 0x00020000);

  // this thread's pieces: A row (tid / PPR) + 32 r, part tid % PPR; B block
  // (n32 block r of the tile, k16 step `wave` of the chunk), lane (tid % 64)
  uint4 sa[2][IPT], sb[2][IPT];
  const int avoff = ((tid / PPR) * lda + (tid % PPR) * 8) * 2;
  const int bvoff = lane * 16;
  // The last row tile is shifted back to end at row M (M >= 256), so every
  // A read is in range; its rows that the previous tile also covers are
  // recomputed with the same values.
  auto tile_m0 = [&](int tile) {
    const long long m0 = (long long)(tile / nN) * 256;
    return m0 + 256 <= M ? m0 : M - 256;
  };
  auto issue = [&](uint4 (&ra)[IPT], uint4 (&rb)[IPT], int tile, int ch) {
    const long long m0 = tile_m0(tile);
    const int bn = tile % nN;
    const __amdgpu_buffer_rsrc_t arsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<h16_t*>(x + m0 * lda), 0, 256 * lda * 2, 0x00020000);
#pragma unroll
    for (int r = 0; r < IPT; ++r)
      ra[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            arsrc, avoff, (32 * r * lda + ch * kS1K) * 2, 0));
#pragma unroll
    for (int r = 0; r < IPT; ++r) {
      const int nb = bn * 8 + r, u = ch * CS + wave;
      rb[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(brsrc, bvoff, (nb * U + u) * 1024, 0));
    }
  };
  // LDS buffer b: A rows at b * kS1Buf, B blocks (n32 block nb, k16 step s at
  // (nb * CS + s) * 1024) after them
  const int aloff = (tid / PPR) * kS1ARow + (tid % PPR) * 16;
  const int bloff = 256 * kS1ARow + wave * 1024 + lane * 16;
  auto commit = [&](const uint4 (&ra)[IPT], const uint4 (&rb)[IPT], int buf) {
    unsigned char* base = g1s + buf * kS1Buf;
#pragma unroll
    for (int r = 0; r < IPT; ++r) {
      *reinterpret_cast<uint4*>(base + aloff + 32 * r * kS1ARow) = ra[r];
      *reinterpret_cast<uint4*>(base + bloff + r * CS * 1024) = rb[r];
    }
  };
  int abase[MI], bbase[NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i) abase[i] = (wm * 128 + 32 * i + lrow) * kS1ARow + kpart * 16;
#pragma unroll
  for (int j = 0; j < NJ; ++j) bbase[j] = 256 * kS1ARow + (wn * 4 + j) * CS * 1024 + lane * 16;

  f32x16_t acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Chunk g + 1 and g + 2 of the stream after chunk ch of tile cur (next
  // tile nxt; tile < 0: past the end).  nch is even, so every tile's chunks
  // alternate parity 0, 1, ... and the last one has parity 1.
  auto ahead = [&](int cur, int nxt, int ch, int d, int& tile, int& c) {
    tile = ch + d < nch ? cur : nxt;
    c = ch + d < nch ? ch + d : ch + d - nch;
  };
  {
    int t1, c1;
    ahead(seq.at(0), seq.at(1), 0, 1, t1, c1);
    issue(sa[0], sb[0], seq.at(0), 0);
    issue(sa[1], sb[1], t1 >= 0 ? t1 : seq.at(0), t1 >= 0 ? c1 : 0);
    commit(sa[0], sb[0], 0);
  }
  __syncthreads();

  // Chunk ch of tile cur with register set / LDS buffer parity P (a
  // compile-time value, so the staging sets stay in registers).
  auto chunk = [&](auto parity, int cur, int nxt, int ch) {
    constexpr int P = decltype(parity)::value;
    int t1, c1, t2, c2;
    ahead(cur, nxt, ch, 1, t1, c1);
    ahead(cur, nxt, ch, 2, t2, c2);
    // unconditional (past the end of the stream it reloads this chunk,
    // unused), so the set's previous values need not live on
    issue(sa[P], sb[P], t2 >= 0 ? t2 : cur, t2 >= 0 ? c2 : ch);
    __builtin_amdgcn_sched_barrier(0);
    const unsigned char* buf = g1s + P * kS1Buf;
    f16x8_t ap[2][MI], bp[2][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i) ap[0][i] = *reinterpret_cast<const f16x8_t*>(buf + abase[i]);
#pragma unroll
    for (int j = 0; j < NJ; ++j) bp[0][j] = *reinterpret_cast<const f16x8_t*>(buf + bbase[j]);
#pragma unroll
    for (int s = 0; s < CS; ++s) {
      if (s + 1 < CS) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
          ap[(s + 1) & 1][i] = *reinterpret_cast<const f16x8_t*>(buf + abase[i] + (s + 1) * 32);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          bp[(s + 1) & 1][j] = *reinterpret_cast<const f16x8_t*>(buf + bbase[j] + (s + 1) * 1024);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bp[s & 1][j], ap[s & 1][i], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // chunk g + 1 (issued two chunks ago) into the other buffer, whose last
    // reader (chunk g - 1) finished before the previous barrier; the barrier
    // makes it visible and ends every wave's reads of this buffer
    if (t1 >= 0) commit(sa[P ^ 1], sb[P ^ 1], P ^ 1);
    __syncthreads();
  };

  for (int k = 0;; ++k) {
    const int cur = seq.at(k);
    if (cur < 0) break;
    const int nxt = seq.at(k + 1);
    for (int ch = 0; ch < nch; ch += 2) {
      chunk(std::integral_constant<int, 0>{}, cur, nxt, ch);
      chunk(std::integral_constant<int, 1>{}, cur, nxt, ch + 1);
    }
    // epilogue through the A rows of buffer 1 (the tile's last chunk): lane
    // (kpart, lrow) of block (i, j) holds row 32i + lrow of the wave's rows
    // and channels 32j + 8g + 4*kpart + r (accumulator 4g + r); per 32 rows
    // and 64 channels the runs go straight from the accumulators into fp32
    // LDS rows, then eight channels per lane get the bias, fp16 and a
    // 16-byte store.
    constexpr int SROW = 64 * 4 + 16, LPR = 8, RPI = 8;
    static_assert(4 * 32 * SROW <= 256 * kS1ARow, "staging fits in a buffer's A rows");
    unsigned char* st = g1s + kS1Buf + wave * 32 * SROW;
    const long long m0 = tile_m0(cur);
    const int n0 = (cur % nN) * 256 + wn * 128;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int jh = 0; jh < NJ / 2; ++jh) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x16_t& c = acc[i][jh * 2 + jj];
            f32x4_t v = {c[4 * g4], c[4 * g4 + 1], c[4 * g4 + 2], c[4 * g4 + 3]};
            *reinterpret_cast<f32x4_t*>(st + lrow * SROW + (32 * jj + 8 * g4 + 4 * kpart) * 4) = v;
          }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the block is in LDS
        __builtin_amdgcn_wave_barrier();
        const int ncol = n0 + jh * 64 + (lane % LPR) * 8;
        float bv[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) bv[q] = 0.0f;
        if (bias) {
          const f32x4_t b0 = *reinterpret_cast<const f32x4_t*>(bias + ncol);
          const f32x4_t b1 = *reinterpret_cast<const f32x4_t*>(bias + ncol + 4);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            bv[q] = b0[q];
            bv[4 + q] = b1[q];
          }
        }
#pragma unroll
        for (int rr = 0; rr < 32 / RPI; ++rr) {
          const int r = rr * RPI + lane / LPR;
          const float* row = reinterpret_cast<const float*>(st + r * SROW) + (lane % LPR) * 8;
          const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(row);
          const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(row + 4);
          const long long m = m0 + wm * 128 + 32 * i + r;
          const float v8[8] = {lo[0] + bv[0], lo[1] + bv[1], lo[2] + bv[2], lo[3] + bv[3],
                               hi[0] + bv[4], hi[1] + bv[5], hi[2] + bv[6], hi[3] + bv[7]};
          *reinterpret_cast<uint4*>(out + m * ldo + ncol) = pack8h(v8);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // this round's reads before the next round's writes
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    __syncthreads();  // the staging rows are read before the next tile's chunk 1 lands here
  }
}

template <int EPI>
__global__ __launch_bounds__(256) void gemm_nt_kernel(GemmArgs ga) {
  constexpr int MI = 4, NJ = 4, CS = kS1K / 16, PPR = kS1K * 2 / 16, IPT = 8;
  static_assert(PPR == 8 && CS == 4, "8 A pieces (32 rows apart) and 8 B blocks per thread");
  extern __shared__ __align__(16) unsigned char g1s[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int kpart = lane >> 5, lrow = lane & 31;
  const long long M = ga.M;
  const int lda = ga.lda, K = ga.K, N = ga.N;
  const int nN = N / 256;
  const long long nMt = (M + 255) / 256;
  const int tpf = (int)(nMt * nN);  // tiles per frame
  const TileSeq seq = tile_seq(tpf * ga.nF);
  if (seq.at(0) < 0) return;
  const int nch = K / kS1K;  // even (the check requires K % 128 == 0)
  const int U = K / 16;

  // The shortcut GEMM's pipeline (gemm1x1_kernel) with frames as a batch
  // dimension: this thread's pieces are A row (tid / PPR) + 32 r, part
  // tid % PPR, and B block (n32 block r of the tile, k16 step `wave`).
  uint4 sa[2][IPT], sb[2][IPT];
  const int avoff = ((tid / PPR) * lda + (tid % PPR) * 8) * 2;
  const int bvoff = lane * 16;
  // The last row tile is shifted back to end at row M (M >= 256), so every
  // A read is in range; its rows that the previous tile also covers are
  // recomputed but stored by the previous tile only.
  auto tile_m0 = [&](int tile) {
    const long long m0 = (long long)((tile % tpf) / nN) * 256;
    return m0 + 256 <= M ? m0 : M - 256;
  };
  auto issue = [&](uint4 (&ra)[IPT], uint4 (&rb)[IPT], int tile, int ch) {
    const int f = tile / tpf;
    const long long m0 = tile_m0(tile);
    const int bn = (tile % tpf) % nN;
    const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<h16_t*>(ga.x + f * ga.a_fs + m0 * lda), 0, 256 * lda * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t brsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<h16_t*>(ga.w + f * ga.w_fs), 0, (int)ga.w_bytes, 0x00020000);
#pragma unroll
    for (int r = 0; r < IPT; ++r)
      ra[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            arsrc, avoff, (32 * r * lda + ch * kS1K) * 2, 0));
#pragma unroll
    for (int r = 0; r < IPT; ++r) {
      const int nb = bn * 8 + r, u = ch * CS + wave;
      rb[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(brsrc, bvoff, (nb * U + u) * 1024, 0));
    }
  };
  const int aloff = (tid / PPR) * kS1ARow + (tid % PPR) * 16;
  const int bloff = 256 * kS1ARow + wave * 1024 + lane * 16;
  auto commit = [&](const uint4 (&ra)[IPT], const uint4 (&rb)[IPT], int buf) {
    unsigned char* base = g1s + buf * kS1Buf;
#pragma unroll
    for (int r = 0; r < IPT; ++r) {
      *reinterpret_cast<uint4*>(base + aloff + 32 * r * kS1ARow) = ra[r];
      *reinterpret_cast<uint4*>(base + bloff + r * CS * 1024) = rb[r];
    }
  };
  int abase[MI], bbase[NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i) abase[i] = (wm * 128 + 32 * i + lrow) * kS1ARow + kpart * 16;
#pragma unroll
  for (int j = 0; j < NJ; ++j) bbase[j] = 256 * kS1ARow + (wn * 4 + j) * CS * 1024 + lane * 16;

  f32x16_t acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // chunk g + d (d <= 2 < nch) after chunk ch of tile cur (next tile nxt;
  // tile < 0: past the end)
  auto ahead = [&](int cur, int nxt, int ch, int d, int& tile, int& c) {
    tile = ch + d < nch ? cur : nxt;
    c = ch + d < nch ? ch + d : ch + d - nch;
  };
  {
    int t1, c1;
    ahead(seq.at(0), seq.at(1), 0, 1, t1, c1);
    issue(sa[0], sb[0], seq.at(0), 0);
    issue(sa[1], sb[1], t1 >= 0 ? t1 : seq.at(0), t1 >= 0 ? c1 : 0);
    commit(sa[0], sb[0], 0);
  }
  __syncthreads();

  auto chunk = [&](auto parity, int cur, int nxt, int ch) {
    constexpr int P = decltype(parity)::value;
    int t1, c1, t2, c2;
    ahead(cur, nxt, ch, 1, t1, c1);
    ahead(cur, nxt, ch, 2, t2, c2);
    // unconditional (past the end it reloads this chunk, unused)
    issue(sa[P], sb[P], t2 >= 0 ? t2 : cur, t2 >= 0 ? c2 : ch);
    __builtin_amdgcn_sched_barrier(0);
    const unsigned char* buf = g1s + P * kS1Buf;
    f16x8_t ap[2][MI], bp[2][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i) ap[0][i] = *reinterpret_cast<const f16x8_t*>(buf + abase[i]);
#pragma unroll
    for (int j = 0; j < NJ; ++j) bp[0][j] = *reinterpret_cast<const f16x8_t*>(buf + bbase[j]);
#pragma unroll
    for (int s = 0; s < CS; ++s) {
      if (s + 1 < CS) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
          ap[(s + 1) & 1][i] = *reinterpret_cast<const f16x8_t*>(buf + abase[i] + (s + 1) * 32);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          bp[(s + 1) & 1][j] = *reinterpret_cast<const f16x8_t*>(buf + bbase[j] + (s + 1) * 1024);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bp[s & 1][j], ap[s & 1][i], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // chunk g + 1 (issued two chunks ago) into the other buffer; the barrier
    // makes it visible and ends every wave's reads of this buffer
    if (t1 >= 0) commit(sa[P ^ 1], sb[P ^ 1], P ^ 1);
    __syncthreads();
  };

  for (int k = 0;; ++k) {
    const int cur = seq.at(k);
    if (cur < 0) break;
    const int nxt = seq.at(k + 1);
    for (int ch = 0; ch < nch; ch += 2) {
      chunk(std::integral_constant<int, 0>{}, cur, nxt, ch);
      chunk(std::integral_constant<int, 1>{}, cur, nxt, ch + 1);
    }
    {
    // lane (kpart, lrow) of block (i, j) holds row 32i + lrow of the
    // wave's rows and columns 32j + 8g + 4*kpart + r (accumulator 4g + r)
    const int f = cur / tpf;
    const long long m0 = tile_m0(cur);
    // rows below mown belong to the previous row tile (the last tile is
    // shifted back): only their owner stores them, so an in-place
    // residual is read and written once per row
    const long long mown = (long long)((cur % tpf) / nN) * 256;
    const int ct = (cur % tpf) % nN;  // column tile
    const int n0 = ct * 256 + wn * 128;
    // Every epilogue goes through buffer 1's A rows (the tile's last chunk): per 32 rows and 64
    // columns the accumulator runs go straight into fp32 LDS rows; then
    // each lane takes eight columns of one row (eight lanes per row):
    //   G_H16: bias (and residual), fp16, a 16-byte store;
    //   G_STATS: the row's max m over those 64 columns (a reduction over
    //     the eight lanes), e^(v - m) as fp16 with a 16-byte store, and
    //     (m, sum of e^(v - m)) as one float2.
    constexpr int SROW = 64 * 4 + 16, LPR = 8, RPI = 8;
    static_assert(4 * 32 * SROW <= 256 * kS1ARow, "staging fits in a buffer's A rows");
    unsigned char* st = g1s + kS1Buf + wave * 32 * SROW;
    const float scale = ga.scale;
    // per-tile row bases (uniform): row m of the tile's frame is row
    // m - m0 + (tile base), so the loops below need 32-bit offsets only
    h16_t* const outb = ga.out + f * ga.o_fs + m0 * ga.ldo;
    const h16_t* const resb = EPI == G_H16 && ga.res ? ga.res + f * ga.r_fs + m0 * ga.ldr : nullptr;
    float* const stb = EPI == G_STATS ? ga.stats + (f * M + m0) * (N / 64) * 2 : nullptr;
    const int mskip = (int)(mown - m0);  // tile rows below this belong to the previous tile
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int jh = 0; jh < NJ / 2; ++jh) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x16_t& c = acc[i][jh * 2 + jj];
            f32x4_t v = {c[4 * g4], c[4 * g4 + 1], c[4 * g4 + 2], c[4 * g4 + 3]};
            *reinterpret_cast<f32x4_t*>(st + lrow * SROW + (32 * jj + 8 * g4 + 4 * kpart) * 4) = v;
          }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the block is in LDS
        __builtin_amdgcn_wave_barrier();
        const int ncol = n0 + jh * 64 + (lane % LPR) * 8;
        float bv[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) bv[q] = 0.0f;
        if (EPI == G_H16 && ga.bias) {
          const f32x4_t b0 = *reinterpret_cast<const f32x4_t*>(ga.bias + ncol);
          const f32x4_t b1 = *reinterpret_cast<const f32x4_t*>(ga.bias + ncol + 4);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            bv[q] = b0[q];
            bv[4 + q] = b1[q];
          }
        }
#pragma unroll 1
        for (int rr = 0; rr < 32 / RPI; ++rr) {
          const int r = rr * RPI + lane / LPR;
          const float* row = reinterpret_cast<const float*>(st + r * SROW) + (lane % LPR) * 8;
          const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(row);
          const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(row + 4);
          const int mt = wm * 128 + 32 * i + r;  // row within the tile
          float v8[8] = {lo[0] * scale + bv[0], lo[1] * scale + bv[1], lo[2] * scale + bv[2],
                         lo[3] * scale + bv[3], hi[0] * scale + bv[4], hi[1] * scale + bv[5],
                         hi[2] * scale + bv[6], hi[3] * scale + bv[7]};
          if constexpr (EPI == G_STATS) {
            float mx = -INFINITY;
#pragma unroll
            for (int q = 0; q < 8; ++q)
              if (ncol + q < ga.n_valid) mx = fmaxf(mx, v8[q]);
            mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 4, 64));
            float sm = 0.0f;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              v8[q] = ncol + q < ga.n_valid ? exp_hw(v8[q] - mx) : 0.0f;
              sm += v8[q];
            }
            sm += __shfl_xor(sm, 1, 64);
            sm += __shfl_xor(sm, 2, 64);
            sm += __shfl_xor(sm, 4, 64);
            if (mt < mskip) continue;
            if (lane % LPR == 0)
              *reinterpret_cast<float2*>(stb + (mt * (N / 64) + ct * 4 + wn * 2 + jh) * 2) = make_float2(mx, sm);
            *reinterpret_cast<uint4*>(outb + mt * ga.ldo + ncol) = pack8h(v8);
          } else {
            if (mt < mskip) continue;
            if (resb) {
              float rv[8];
              unpack8h(*reinterpret_cast<const uint4*>(resb + mt * ga.ldr + ncol), rv);
#pragma unroll
              for (int q = 0; q < 8; ++q) v8[q] += rv[q];
            }
            *reinterpret_cast<uint4*>(outb + mt * ga.ldo + ncol) = pack8h(v8);
          }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // this round's reads before the next round's writes
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    __syncthreads();  // the staging rows are read before the next tile's chunk 1 lands here
  }
}

}  // namespace

const char* gemm_nt_check(const GemmArgs& g, int epi) {
  if (epi != G_H16 && epi != G_STATS) return "epilogue";
  if (!g.x || !g.w || g.M < 256 || g.N % 256 || g.K % (2 * kS1K) || g.K > 4096 || g.lda % 8 || g.lda < g.K)
    return "A / B shapes";
  if (g.w_bytes <= 0 || g.w_bytes > 0x7fffffffLL || (long long)256 * g.lda * 2 > 0x7fffffffLL) return "B bytes";
  if (g.nF < 1 || (g.nF > 1 && (g.a_fs < 0 || g.w_fs < 0 || g.o_fs < 0 || g.r_fs < 0))) return "frames";
  if ((long long)(g.M + 255) / 256 * (g.N / 256) * g.nF > 0x7fffffffLL) return "tile count";
  if (!g.out || g.ldo % 8 || g.ldo < g.N) return "output";
  if (g.res && (g.ldr % 8 || g.ldr < g.N || epi != G_H16)) return "residual";
  if (epi == G_STATS && (!g.stats || g.n_valid < 1 || g.n_valid > g.N || g.bias)) return "statistics operands";
  return nullptr;
}

hipError_t launch_gemm_nt(const GemmArgs& g, int epi, hipStream_t stream) {
  if (g_dry_run) return gemm_nt_check(g, epi) ? hipErrorInvalidValue : hipSuccess;
  if (gemm_nt_check(g, epi)) return hipErrorInvalidValue;
  const void* kern = epi == G_STATS ? reinterpret_cast<const void*>(gemm_nt_kernel<G_STATS>)
                                    : reinterpret_cast<const void*>(gemm_nt_kernel<G_H16>);
  static bool attr[2] = {false, false};
  if (!attr[epi]) {
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, kS1Lds);
    if (e != hipSuccess) return e;
    attr[epi] = true;
  }
  const long long tiles = (g.M + 255) / 256 * (g.N / 256) * g.nF;
  int dev = 0, ncu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const long long grid = tiles < ncu ? tiles : ncu;
  if (epi == G_STATS)
    hipLaunchKernelGGL(gemm_nt_kernel<G_STATS>, dim3((unsigned)grid), dim3(256), kS1Lds, stream, g);
  else
    hipLaunchKernelGGL(gemm_nt_kernel<G_H16>, dim3((unsigned)grid), dim3(256), kS1Lds, stream, g);
  return hipGetLastError();
}

hipError_t launch_gemm1x1(const h16_t* x, long long M, int lda, int K, const h16_t* w, long long w_bytes, int N,
                          const float* bias, h16_t* out, int ldo, hipStream_t stream) {
  if (g_dry_run) return hipSuccess;
  if (!x || !w || !out || M < 256 || N % 256 || K % (2 * kS1K) || K > 4096 || lda % 8 || lda < K ||
      ldo % 8 || ldo < N ||
      w_bytes <= 0 || w_bytes > 0x7fffffffLL || (long long)256 * lda * 2 > 0x7fffffffLL)
    return hipErrorInvalidValue;
  const long long tiles = (M + 255) / 256 * (N / 256);
  if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm1x1_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kS1Lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  int dev = 0, ncu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const long long grid = tiles < ncu ? tiles : ncu;
  hipLaunchKernelGGL(gemm1x1_kernel, dim3((unsigned)grid), dim3(256), kS1Lds, stream, x, M, lda, K, w, (int)w_bytes,
                     N, bias, out, ldo);
  return hipGetLastError();
}

// Launches that run on the persistent kernel: the specialised one-segment
// tap sets on 8-wave tiles, with the epilogues that kernel implements.
bool conv_persistent(const ConvArgs& a) {
  const Variant v = conv_variant(a);
  if (v.mode == 0 || v.nw != 8 || a.nseg != 1) return false;
  if (v.bn == 32) return v.mode == 1 && a.epi == EPI_VIDEO && a.seg[0].prologue == PRO_RAW;
  if (v.mode == 3) return a.epi == EPI_TIME;
  if (v.mode == 4) return a.epi == EPI_WINO;
  if (v.mode == 5) return true;
  if (v.mode == 2) return a.epi == EPI_PHASE || (a.nphase == 1 && a.epi == EPI_H16);
  return a.epi == EPI_H16 || (v.mode == 1 && a.epi == EPI_VIDEO);
}

bool conv_is_333(const ConvArgs& a) { return conv_variant(a).mode == 1; }

bool conv_is_main(const ConvArgs& a) {
  const Variant v = conv_variant(a);
  return conv_persistent(a) &&
         (v.mode == 4 || (v.mode == 1 && v.bn == 256 && a.seg[0].prologue == PRO_NORM_SILU));
}

size_t conv_lds_bytes(const ConvArgs& a) {
  const Variant v = conv_variant(a);
  int cin_max = 0;
  for (int s = 0; s < a.nseg; ++s)
    if (a.seg[s].prologue != PRO_RAW && a.seg[s].Cin > cin_max) cin_max = a.seg[s].Cin;
  if (conv_persistent(a))  // two halo buffers, two table sets, gamma; the epilogue stages inside a halo buffer
    return (size_t)2 * a.nhv_max * (v.bk * 2 + 16) + (size_t)2 * a.nhv_max * (8 + 4) + (size_t)cin_max * 4;
  const size_t main_loop =
      (size_t)2 * a.nhv_max * (v.bk * 2 + 16) + (size_t)a.nhv_max * (8 + 4) + (size_t)cin_max * 4;
  const int wn = v.bn == 32 ? 32 : 64;  // wave tile width of the instantiation
  const size_t epilogue = (size_t)v.nw * 32 * (wn + 4) * 4;
  return main_loop > epilogue ? main_loop : epilogue;
}

const char* conv_check(const ConvArgs& a) {
  if (a.nseg < 1 || a.nseg > 2) return "segment count";
  // the head with its x taps in the output columns (3x1 taps, video store)
  const bool headx = a.seg[0].KS == KS_3x1 && a.epi == EPI_VIDEO;
  if (headx ? (a.TF != 4 || a.TW != 16) : (a.seg[0].KS == KS_3x1 ? !wino_tile_shape_ok(a.TF, a.TW) : a.TW != kTileW))
    return "unsupported tile shape";
  if (headx && (a.Cout != 64 || a.nphase != 1 || a.tiles_x != (a.W + 13) / 14 || a.nseg != 1 ||
                a.nhv_max * (32 * 2 + 16) < kHeadXEpiBytes || conv_variant(a).mode != 5))
    return "the head's packed form: 64 columns, one phase, tiles of 14 output columns, staging rows";
  if (a.TF < 1 || a.TF * a.TH * a.TW != kTileM) return "tile TF*TH*TW != 256";
  if (a.F < 1 || a.H < 1 || a.W < 1 || a.Cout < 1) return "empty output grid";
  if (a.nphase != 1 && a.nphase != 4 && a.nphase != kWinoN) return "phase count";
  if (conv_lds_bytes(a) > 160 * 1024) return "LDS over 160 KiB";
  const int bk = conv_bk(a);
  for (int s = 0; s < a.nseg; ++s) {
    const ConvSeg& g = a.seg[s];
    const int hsy = g.KS == KS_1x1 ? 0 : 1;
    const int hsx = g.KS == KS_1x1 || g.KS == KS_3x1 ? 0 : 1;
    const int k2 = g.KS == KS_3x3 ? 9 : (g.KS == KS_PHASE ? 4 : (g.KS == KS_3x1 ? 3 : 1));
    const int st = g.stride == 2 ? 2 : 1;
    const int nhv = (a.TF + g.KT - 1) * (st * a.TH + 2 * hsy - (st - 1)) * (st * a.TW + 2 * hsx - (st - 1));
    const int nt = conv_variant(a).nw * 64;
    const int ipt = (nhv * (bk / 8) + nt - 1) / nt;
    const int ntaps = g.KT * k2;
    if (!g.x || !g.w) return "null operand";
    if (g.KT != 1 && g.KT != 3) return "KT must be 1 or 3";
    if (g.KS < KS_1x1 || g.KS > KS_3x1) return "unknown spatial tap code";
    if (g.KS == KS_PHASE && !(a.nphase == 4 || (a.nphase == 1 && a.epi == EPI_H16)))
      return "phase taps need 4 phases (or one, with a plain store)";
    if (a.epi == EPI_PHASE && (g.KS != KS_PHASE || a.nphase != 4)) return "the phase store needs 4 phases";
    if (g.KS == KS_3x1 && !headx && a.nphase != kWinoN) return "Winograd taps need one phase per xi plane";
    if (a.nphase != 1 && g.KS != KS_PHASE && g.KS != KS_3x1) return "phases need phase or Winograd taps";
    if (g.KS == KS_3x1 && !headx && (a.epi != EPI_WINO || conv_variant(a).mode != 4))
      return "3x1 taps run only as the Winograd-domain GEMM or the head";
    if (a.epi == EPI_WINO && g.KS != KS_3x1) return "EPI_WINO needs the 3x1 taps";
    if ((a.epi == EPI_WINO || g.KS == KS_PHASE) && a.nhv_max * (bk * 2 + 16) < kSwapEpiBytes)
      return "halo buffer below the epilogue's staging rows";
    if (g.KS == KS_PHASE && a.res) return "the phase-tap epilogue adds no residual";
    if (a.epi == EPI_WINO && (a.bias || a.res || a.scale != 1.0f))
      return "the Winograd-domain GEMM stores plain products (no bias, residual or scale)";
    if (a.bn != 0 && (a.epi != EPI_WINO || (a.bn != 128 && a.bn != 256) || a.Cout % a.bn))
      return "a tile width of 128 or 256 channels (dividing Cout) is the Winograd GEMM's choice";
    if (a.epi == EPI_WINO && (a.out_fstride < (long long)a.H * a.W * a.ldo ||
                              2LL * a.TF * a.out_fstride + 16 > 0x7fffffffLL))
      return "a Winograd product tile must span less than 2^31 bytes (32-bit store offsets)";
    if (nhv > a.nhv_max) return "halo larger than nhv_max";
    if ((g.KT == 3 && g.KS == 3 && a.TF == kTF333 && a.TH == kTH333 &&
         ((kNHV333 * (bk / 8) + 511) / 512) * 512 / (bk / 8) > a.nhv_max))
      return "nhv_max below the 3x3x3 item rows";
    if (g.wfrag && (g.w_bytes <= 0 || g.w_bytes > 0x7fffffffLL)) return "fragment weights need 0 < bytes < 2 GiB";
    if ((ipt + ntaps - 1) / ntaps > kMaxHaloItemsPerTap) return "halo items per tap over the register budget";
    if (g.Cin < 16 || g.Cin % 16) return "Cin must be a positive multiple of 16";
    if (g.Cin > a.zero_len) return "zero row shorter than Cin";
    if (g.lda % 8 || g.lda < g.Cin) return "input row stride must be a multiple of 8 and >= Cin";
    if (!g.wfrag && (g.ldw % 8 || g.ldw < g.Cin)) return "row-major operand stride";
    if (g.prologue != PRO_RAW && (g.Cin > kMaxCin || !g.rs || !g.gamma)) return "norm prologue operands";
    if (g.n_hist < 0 || g.n_hist > 2 || (g.n_hist > 0 && (!g.ring || g.KT != 3))) return "history ring";
    if (g.w_frame_stride && a.TF != 1) return "per-frame operands need TF == 1";
    if (g.stride != 0 && g.stride != 1 && g.stride != 2) return "stride must be 1 or 2";
    if (g.stride == 2 && (g.KT != 1 || g.KS != KS_3x3 || g.prologue != PRO_RAW || g.n_hist != 0 ||
                          conv_variant(a).mode != 0 || a.nphase != 1 || a.nseg != 1))
      return "stride 2 only for a raw one-segment 3x3 conv on the generic kernel";
    if (s > 0 && (g.KT != 1 || g.KS != 1) && conv_variant(a).mode != 0)
      return "the specialised kernels take only a 1x1x1 second segment";
    if (s > 0 && g.KS != KS_1x1) return "second segment must have 1x1 spatial taps";
  }
  if (a.epi == EPI_VIDEO && a.Cout != (headx ? 64 : 12))
    return "the video epilogue takes the head's 12 channels (64 packed columns)";
  if (a.epi == EPI_LATENT && (conv_persistent(a) || a.video_T < 1 || a.out_base < 0 || a.out_base + a.F > a.video_T))
    return "latent epilogue: generic kernel, frames inside the clip";
  if (!a.out || !a.zero_row) return "null output or zero row";
  return nullptr;
}

hipError_t launch_conv(const ConvArgs& a, hipStream_t stream) {
  if (conv_check(a)) return hipErrorInvalidValue;
  const Variant v = conv_variant(a);
  if (conv_persistent(a)) {
    const int pro = a.seg[0].prologue;
    if (v.mode == 2) return launch_persist_impl<256, 4, 2, PRO_RAW>(a, stream);
    if (v.mode == 3) return launch_persist_impl<256, 4, 3, PRO_RAW>(a, stream);
    if (v.mode == 5) return launch_persist_impl<64, 1, 5, PRO_RAW, 4, 16, 4>(a, stream);
    if (v.mode == 4) {  // one instantiation per Winograd tile shape (TF frames x TW column groups) and width
      if (a.bn == 128) {
        if (a.TF == 2 && a.TW == 8) return launch_persist_impl<128, 2, 4, PRO_RAW, 4, 8, 2>(a, stream);
        if (a.TF == 4 && a.TW == 8) return launch_persist_impl<128, 2, 4, PRO_RAW, 4, 8, 4>(a, stream);
        if (a.TF == 8 && a.TW == 4) return launch_persist_impl<128, 2, 4, PRO_RAW, 4, 4, 8>(a, stream);
        if (a.TF == 4 && a.TW == 4) return launch_persist_impl<128, 2, 4, PRO_RAW, 4, 4, 4>(a, stream);
        return launch_persist_impl<128, 2, 4, PRO_RAW, 4>(a, stream);
      }
      if (a.TF == 2 && a.TW == 8) return launch_persist_impl<256, 2, 4, PRO_RAW, 4, 8, 2>(a, stream);
      if (a.TF == 4 && a.TW == 8) return launch_persist_impl<256, 2, 4, PRO_RAW, 4, 8, 4>(a, stream);
      if (a.TF == 8 && a.TW == 4) return launch_persist_impl<256, 2, 4, PRO_RAW, 4, 4, 8>(a, stream);
      if (a.TF == 4 && a.TW == 4) return launch_persist_impl<256, 2, 4, PRO_RAW, 4, 4, 4>(a, stream);
      return launch_persist_impl<256, 2, 4, PRO_RAW, 4>(a, stream);
    }
    // the head (N = 32): 4 waves of 64 x 32, so each weight fragment feeds
    // two MFMAs (its one n32 block is the same for every wave, and eight
    // waves of 32 x 32 fetched every fragment eight times from L2)
    if (v.bn == 32) return launch_persist_impl<32, 1, 1, PRO_RAW, 4>(a, stream);
    if (pro == PRO_NORM_SILU) return launch_persist_impl<256, 2, 1, PRO_NORM_SILU, 4>(a, stream);
    return launch_persist_impl<256, 4, 1, PRO_RAW>(a, stream);
  }
  if (v.mode >= 3) return hipErrorInvalidValue;  // these tap sets exist only in the persistent kernel
  if (v.mode == 1) {
    const bool act = a.seg[0].prologue == PRO_NORM_SILU;
    if (v.nw == 8 && v.bn == 32) {
      if (act) return hipErrorInvalidValue;  // the narrow 3x3x3 variant is raw-only
      return launch_impl<32, 32, 1, 8, 1, PRO_RAW>(a, stream);
    }
    if (v.nw == 8)
      return act ? launch_impl<32, 256, 4, 8, 1, PRO_NORM_SILU>(a, stream)
                 : launch_impl<32, 256, 4, 8, 1, PRO_RAW>(a, stream);
    return act ? launch_impl<32, 128, 2, 4, 1, PRO_NORM_SILU>(a, stream)
               : launch_impl<32, 128, 2, 4, 1, PRO_RAW>(a, stream);
  }
  if (v.mode == 2) {
    if (v.nw == 8) return launch_impl<32, 256, 4, 8, 2, PRO_RAW>(a, stream);
    return launch_impl<32, 128, 2, 4, 2, PRO_RAW>(a, stream);
  }
  if (v.bk == 32 && v.bn == 128) return launch_impl<32, 128, 2, 4, 0, -1>(a, stream);
  if (v.bk == 32 && v.bn == 32) return launch_impl<32, 32, 1, 4, 0, -1>(a, stream);
  if (v.bk == 16 && v.bn == 128) return launch_impl<16, 128, 2, 4, 0, -1>(a, stream);
  return launch_impl<16, 32, 1, 4, 0, -1>(a, stream);
}

// Device address of this code object's range flags on the current device.
hipError_t conv_range_flags_addr(unsigned int** p) {
  return hipGetSymbolAddress(reinterpret_cast<void**>(p), HIP_SYMBOL(g_range_flags));
}

}  // namespace wvd
