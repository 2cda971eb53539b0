// Host side of the wvd library: the C ABI, the prepared-weight layout, the
// workspace plan and the pass scheduler that walks the decoder frames_per_pass
// latent frames at a time, carrying two history frames per causal conv in a
// ring (the "temporal caching" of the TensorRT-LLM norm-SiLU issue; the
// Wan2.2 VAE decoder page, "Performance and memory", decodes in passes of
// frames_per_pass latent frames without changing the video).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "wvd.h"
#include "wvd_internal.h"

using namespace wvd;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

enum ItemKind { K_CONV = 0, K_PHASE = 1, K_VEC = 2, K_WINO = 3, K_CONV_PART = 4, K_S2D = 5, K_HEADX = 6 };

// A 3x3x3 norm-SiLU conv runs in Winograd form (F(kWinoM,3) along x: input
// transform, kWinoN xi-plane GEMMs on the persistent kernel, output transform)
// when its widths suit the 256-wide persistent tiles and 32-channel chunks.
bool wino_ok(int cin, int cout) { return cin % 32 == 0 && cout % 256 == 0; }
// conv1 in Winograd form (wino_ok(cin, cout)), conv2 too (wino_ok(cout,
// cout), and a width-changing block's shortcut suits the 1x1 GEMM: K a
// multiple of 64).
bool rb_wino2(int cin, int cout) { return wino_ok(cout, cout) && (cin == cout || cin % 64 == 0); }
// Both convs of a ResBlock in Winograd form, conv1's output transform fused
// with conv2's input transform (wino_mid).
bool rb_fused(int cin, int cout) { return wino_ok(cin, cout) && rb_wino2(cin, cout) && wino_mid_ok(cout); }

// One canonical weight tensor and where its prepared form lives.
struct Item {
  int kind;
  int cout, cin, taps, cin_pad;  // conv: PyTorch [cout][cin][taps] -> [taps][cout][cin_pad]
  int n;                          // vec length
  float scale;                    // vec scale (sqrt(C) for gammas)
  size_t off;                     // byte offset in the prepared buffer
  size_t bytes;
  // K_CONV_PART: input channels [cin_off, cin_off + cin) of a tensor with
  // cin_src input channels, the canonical tensor `src` (-1: this item's own
  // index)
  int src = -1, cin_src = 0, cin_off = 0;
};

// Indices of the canonical tensors of one ResBlock.
struct RB {
  int norm1, conv1w, conv1b, norm2, conv2w, conv2b, scw = -1, scb = -1;
  int cin, cout;
  bool wino1 = false, wino2 = false;  // conv1 / conv2 prepared and run in Winograd form
};

constexpr int kMaxResPerStage = 3;

struct Layout {
  std::vector<Item> items;
  int nrb = 2;                  // ResBlocks per up stage (3 in the deep variant)
  int pre_w = -1, pre_b = -1;   // deep variant: 48 -> 48 1x1x1 conv on the latents (fp32 matrix, bias)
  int conv_in_w, conv_in_b;
  RB mid0, mid1, up[4][kMaxResPerStage];
  int attn_norm, qkv_w, qkv_b, proj_w, proj_b;
  int tc_w[2], tc_b[2], upc_w[3], upc_b[3];
  int head_norm, head_w, head_b;
  // The encoder (R13-R16): down stages, strided down-convs, and the temporal
  // down-convs of stages 1 and 2 as two K segments (the pair's first and
  // second frame) with a shared bias.
  bool encoder = false;
  RB down[4][2];
  int dc_w[3], dc_b[3];
  int td_w[2][2], td_b[2];
  size_t zero_off = 0;
  int zero_len = 0;
  size_t total = 0;
};

void add_conv(Layout& L, int cout, int cin, int taps, int cin_pad, int* wi, int* bi) {
  Item w{K_CONV, cout, cin, taps, cin_pad, 0, 1.0f, 0, 0};
  w.bytes = prep_frag_bytes(cout, cin_pad, taps);
  *wi = (int)L.items.size();
  L.items.push_back(w);
  Item b{K_VEC, 0, 0, 0, 0, cout, 1.0f, 0, (size_t)cout * 4};
  *bi = (int)L.items.size();
  L.items.push_back(b);
}
int add_vec(Layout& L, int n, float scale) {
  Item g{K_VEC, 0, 0, 0, 0, n, scale, 0, (size_t)n * 4};
  L.items.push_back(g);
  return (int)L.items.size() - 1;
}
RB add_rb(Layout& L, int cin, int cout) {
  RB r;
  r.cin = cin;
  r.cout = cout;
  r.norm1 = add_vec(L, cin, std::sqrt((float)cin));
  add_conv(L, cout, cin, 27, cin, &r.conv1w, &r.conv1b);
  r.norm2 = add_vec(L, cout, std::sqrt((float)cout));
  add_conv(L, cout, cout, 27, cout, &r.conv2w, &r.conv2b);
  if (cin != cout) add_conv(L, cout, cin, 1, cin, &r.scw, &r.scb);
  auto to_wino = [&](int item) {
    Item& it = L.items[item];
    it.kind = K_WINO;
    it.taps = kWinoN * 9;  // xi x 3 dt x 3 dy
    it.bytes = prep_frag_bytes(it.cout, it.cin_pad, it.taps);
  };
  r.wino1 = wino_ok(cin, cout);
  r.wino2 = rb_wino2(cin, cout);
  if (r.wino1) to_wino(r.conv1w);
  if (r.wino2) to_wino(r.conv2w);
  return r;
}

int lpad_of(int L);

Layout make_layout(int c, int h, int w, bool deep = false) {
  Layout L;
  const int c4 = 4 * c;
  const int widths[4] = {c4, c4, 2 * c, c};
  L.nrb = deep ? 3 : 2;
  if (deep) {
    L.pre_w = add_vec(L, 48 * 48, 1.0f);  // [out][in] as fp32
    L.pre_b = add_vec(L, 48, 1.0f);
  }
  add_conv(L, c4, 48, 27, 64, &L.conv_in_w, &L.conv_in_b);
  L.mid0 = add_rb(L, c4, c4);
  L.attn_norm = add_vec(L, c4, std::sqrt((float)c4));
  add_conv(L, 3 * c4, c4, 1, c4, &L.qkv_w, &L.qkv_b);
  add_conv(L, c4, c4, 1, c4, &L.proj_w, &L.proj_b);
  L.mid1 = add_rb(L, c4, c4);
  int prev = c4;
  for (int s = 0; s < 4; ++s) {
    const int cs = widths[s];
    L.up[s][0] = add_rb(L, prev, cs);
    for (int k = 1; k < L.nrb; ++k) L.up[s][k] = add_rb(L, cs, cs);
    if (s < 2) add_conv(L, 2 * cs, cs, 3, cs, &L.tc_w[s], &L.tc_b[s]);
    if (s < 3) {
      add_conv(L, cs, cs, 9, cs, &L.upc_w[s], &L.upc_b[s]);
      Item& it = L.items[L.upc_w[s]];
      it.kind = K_PHASE;
      it.taps = 16;  // 4 phases x 2x2 taps
      it.bytes = prep_frag_bytes(cs, cs, 16);
    }
    prev = cs;
  }
  L.head_norm = add_vec(L, c, std::sqrt((float)c));
  add_conv(L, 12, c, 27, c, &L.head_w, &L.head_b);
  if (c % 32 == 0) {  // the x taps in the output columns (the head's packed form)
    Item& it = L.items[L.head_w];
    it.kind = K_HEADX;
    it.bytes = prep_frag_bytes(64, c, 9);
  }
  size_t off = 0;
  for (auto& it : L.items) {
    it.off = off;
    off = align_up(off + it.bytes);
  }
  // fp16 zeros: the source of padding voxels; as long as the widest
  // reduction of any conv (the attention P.V contraction runs over h*w keys).
  L.zero_off = off;
  L.zero_len = std::max(kMaxCin, lpad_of(h * w));
  off = align_up(off + (size_t)L.zero_len * 2);
  L.total = off;
  return L;
}

// Workspace carve-up for a given maximum number of latent frames per pass.
struct Work {
  size_t X, H, Y, zt, zp, rs, qkv, S, Pm, Vt, O;
  size_t X_bytes, H_bytes, Y_bytes;  // capacities of X, H, Y (checked before every write into them)
  size_t kf, vf, st;         // attention on the batched GEMM: K, V^T fragments, score statistics
  size_t U, M;               // Winograd input planes and products
  std::vector<size_t> ring;  // 24 rings: offsets inside the ring block
  size_t rings;              // ring block offset in the workspace (npos: caller-owned state)
  size_t ring_bytes;         // ring block size
  size_t total;
};

constexpr size_t kNoRings = ~(size_t)0;

struct RingInfo {
  int cin;
  int level;
};

// Rings (the last two raw input frames of every temporal conv), in a fixed
// order: conv_in, the mid block's four convs, per up stage two per ResBlock
// and the time_conv of stages 0 and 1, then the head.
enum { R_CONV_IN = 0, R_MID0_1, R_MID0_2, R_MID1_1, R_MID1_2, R_UP_BASE };

int ring_up(int nrb, int s, int k, int conv) {  // conv 0: conv1's input, 1: conv2's input
  int id = R_UP_BASE;
  for (int t = 0; t < s; ++t) id += 2 * nrb + (t < 2 ? 1 : 0);
  return id + 2 * k + conv;
}
int ring_tc(int nrb, int s) { return ring_up(nrb, s, nrb, 0); }
int ring_head(int nrb) { return ring_up(nrb, 3, nrb, 0); }
int ring_count(int nrb) { return ring_head(nrb) + 1; }

RingInfo ring_info(int c, int nrb, int id) {
  const int c4 = 4 * c;
  const int widths[4] = {c4, c4, 2 * c, c};
  if (id < R_UP_BASE) return {id == R_CONV_IN ? 64 : c4, 0};
  if (id == ring_head(nrb)) return {c, 3};
  int prev = c4;
  for (int s = 0; s < 4; ++s) {
    for (int k = 0; k < nrb; ++k)
      for (int cv = 0; cv < 2; ++cv)
        if (id == ring_up(nrb, s, k, cv)) return {(k == 0 && cv == 0) ? prev : widths[s], s};
    if (s < 2 && id == ring_tc(nrb, s)) return {widths[s], s};
    prev = widths[s];
  }
  return {c, 3};
}

int lpad_of(int L) { return (L + 31) / 32 * 32; }

// The mid attention runs on the batched 256 x 256 GEMM (scores never stored:
// a score pass, then an in-place softmax of its output) when a frame has at least 256
// tokens and the width is a multiple of 256; smaller shapes use the generic
// conv kernel with stored fp32 scores.
bool attn_fast(int C, long long L) { return L >= 256 && C % 256 == 0; }
long long attn_np(long long L) { return (L + 255) / 256 * 256; }

// Attention buffers of F frames of L tokens at width C: the fp32 scores,
// probabilities and V^T of the generic path, or the probabilities, K and V^T
// fragments and score statistics of the batched-GEMM path.
template <class Take>
void take_attention(Work& W, Take& take, long long F, long long L, long long C) {
  const long long Lp = lpad_of((int)L), Np = attn_np(L);
  const bool fast = attn_fast((int)C, L);
  W.S = take(fast ? 0 : (size_t)F * L * Lp * 4);
  W.Pm = take((size_t)F * L * (fast ? Np : Lp) * 2);
  W.Vt = take(fast ? 0 : (size_t)F * C * Lp * 2);
  W.O = take((size_t)F * L * C * 2);
  W.kf = take(fast ? (size_t)F * Np * C * 2 : 0);
  W.vf = take(fast ? (size_t)F * Np * C * 2 : 0);
  W.st = take(fast ? (size_t)F * L * (Np / 64) * 8 : 0);
}

Work make_work(int c, int h, int w, int P, bool rings_in_workspace = true, int nrb = 2) {
  Work W;
  const long long r0 = (long long)h * w;
  const long long res[4] = {r0, 4 * r0, 16 * r0, 64 * r0};
  const long long c4 = 4 * c, c2 = 2 * c;
  const long long F0 = P, F1 = 2LL * P, F2 = 4LL * P;
  const long long L = r0;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  // X: conv_in's output and the up-convs' (the widest: level 3 at 2c).
  W.X_bytes = (size_t)std::max({F0 * r0 * c4, F1 * res[1] * c4, F2 * res[2] * c4, F2 * res[3] * c2}) * 2;
  W.X = take(W.X_bytes);
  // H holds a ResBlock's conv1 output h.  Where both convs run fused in
  // Winograd form (the output transform of conv1 feeds conv2's input
  // transform directly), h is stored only for the history ring, and into H
  // only by a one-frame pass; other blocks store all the pass's frames.  The
  // head's normalised input goes to H where the last ResBlock cannot write
  // it.  Levels 0..3 hold widths 4c, 4c, 4c -> 2c -> 2c, 2c -> c -> c.
  {
    const long long fl[4] = {F0, F1, F2, F2};
    const long long blk[6][3] = {{0, c4, c4}, {1, c4, c4}, {2, c4, c2}, {2, c2, c2}, {3, c2, c}, {3, c, c}};
    long long hsz = 0;
    for (const auto& b : blk) {
      const bool fused = rb_fused((int)b[1], (int)b[2]);
      hsz = std::max(hsz, (fused ? 1 : fl[b[0]]) * res[b[0]] * b[2]);
    }
    if (!rb_fused(c, c)) hsz = std::max(hsz, F2 * res[3] * c);
    W.H_bytes = (size_t)hsz * 2;
    W.H = take(W.H_bytes);
  }
  // Y: the time_convs' outputs and the width-changing ResBlocks' (4c -> 2c
  // at level 2, 2c -> c at level 3).
  W.Y_bytes = (size_t)std::max({F1 * r0 * c4, F2 * res[1] * c4, F2 * res[2] * c2, F2 * res[3] * c}) * 2;
  W.Y = take(W.Y_bytes);
  W.zt = take((size_t)F0 * r0 * 64 * 2);
  W.zp = take((size_t)F0 * r0 * 64 * 2);  // latents after the deep variant's 1x1x1 conv
  W.rs = take((size_t)(F2 + 2) * res[3] * 4);
  W.qkv = take((size_t)F0 * L * 3 * c4 * 2);
  take_attention(W, take, F0, L, c4);
  {
    // Winograd planes: U = [N][F+2][H][WQ][Cin], M = [N][F][H][WQ][Cout] with
    // N = kWinoN planes and WQ = ceil(W / kWinoM) column groups, per level
    // (Cin / Cout of that level's widest Winograd conv).
    const long long hl[4] = {h, 2LL * h, 4LL * h, 8LL * h};
    long long w2[4];
    for (int l = 0; l < 4; ++l) w2[l] = (((long long)w << l) + kWinoM - 1) / kWinoM;
    const long long fl[4] = {F0, F1, F2, F2};
    const long long ci[4] = {c4, c4, c4, c2};
    const long long co[4] = {c4, c4, c2, c};
    long long u = 0, m = 0;
    for (int l = 0; l < 4; ++l) {
      if (!wino_ok((int)ci[l], (int)co[l]) && !wino_ok((int)co[l], (int)co[l])) continue;
      u = std::max(u, kWinoN * (fl[l] + 2) * hl[l] * w2[l] * ci[l]);
      m = std::max(m, kWinoN * fl[l] * hl[l] * w2[l] * co[l]);
    }
    W.U = take((size_t)u * 2);
    W.M = take((size_t)m * 2);
  }
  // The causal history (two raw input frames of every temporal conv) lives
  // in one block: inside the workspace for a whole-clip decode, or in the
  // caller's stream state for chunked decodes.
  size_t roff = 0;
  for (int i = 0; i < ring_count(nrb); ++i) {
    RingInfo ri = ring_info(c, nrb, i);
    W.ring.push_back(roff);
    roff = align_up(roff + (size_t)2 * res[ri.level] * ri.cin * 2);
  }
  W.ring_bytes = roff;
  W.rings = rings_in_workspace ? take(roff) : kNoRings;
  W.total = off;
  return W;
}

// ---------------------------------------------------------------------------
// Encoder layout, rings and workspace (the decoder's mirror image, R13-R16)
// ---------------------------------------------------------------------------

int enc_width(int c, int s) { return s == 0 ? c : (s == 1 ? 2 * c : 4 * c); }

// Items 0..83 are the canonical tensors in order; the second halves of the
// two temporal down-convs' weights follow.
Layout make_layout_enc(int c, int h, int w) {
  Layout L;
  L.encoder = true;
  const int c4 = 4 * c;
  // 12 patch channels, padded to 32: one 32-channel chunk, so conv_in runs on
  // the specialised 3x3x3 kernel (16-channel chunks would take the generic one)
  add_conv(L, c, 12, 27, kEncInC, &L.conv_in_w, &L.conv_in_b);
  int prev = c;
  for (int s = 0; s < 4; ++s) {
    const int cs = enc_width(c, s);
    L.down[s][0] = add_rb(L, prev, cs);
    L.down[s][1] = add_rb(L, cs, cs);
    if (s < 3) {
      // the stride-2 down-conv runs in space-to-depth form: 2x2 taps over
      // the four phase images (4 cs input channels)
      add_conv(L, cs, cs, 9, cs, &L.dc_w[s], &L.dc_b[s]);
      Item& it = L.items[L.dc_w[s]];
      it.kind = K_S2D;
      it.taps = 4;
      it.bytes = prep_frag_bytes(cs, 4 * cs, 4);
    }
    if (s == 1 || s == 2) {
      const int k = s - 1;
      add_conv(L, cs, cs, 3, cs, &L.td_w[k][0], &L.td_b[k]);
      Item& it = L.items[L.td_w[k][0]];
      it.kind = K_CONV_PART;  // the pair's first frame: input channels [0, cs) of [cs, 2cs, 3, 1, 1]
      it.cin_src = 2 * cs;
      it.cin_off = 0;
    }
    prev = cs;
  }
  L.mid0 = add_rb(L, c4, c4);
  L.attn_norm = add_vec(L, c4, std::sqrt((float)c4));
  add_conv(L, 3 * c4, c4, 1, c4, &L.qkv_w, &L.qkv_b);
  add_conv(L, c4, c4, 1, c4, &L.proj_w, &L.proj_b);
  L.mid1 = add_rb(L, c4, c4);
  L.head_norm = add_vec(L, c4, std::sqrt((float)c4));
  add_conv(L, 48, c4, 27, c4, &L.head_w, &L.head_b);
  for (int k = 0; k < 2; ++k) {  // the pair's second frame: input channels [cs, 2cs)
    const int cs = enc_width(c, k + 1);
    Item it = L.items[L.td_w[k][0]];
    it.src = L.td_w[k][0];
    it.cin_off = cs;
    L.td_w[k][1] = (int)L.items.size();
    L.items.push_back(it);
  }
  size_t off = 0;
  for (auto& it : L.items) {
    it.off = off;
    off = align_up(off + it.bytes);
  }
  L.zero_off = off;
  // (the space-to-depth down-convs read 4 x their width per voxel)
  L.zero_len = std::max({kMaxCin, lpad_of(h * w), 4 * enc_width(c, 2)});
  off = align_up(off + (size_t)L.zero_len * 2);
  L.total = off;
  return L;
}

// Encoder rings: conv_in; per down stage s, ResBlock k, conv cv one each;
// the temporal down-convs' two segments (first / second frame of a pair);
// the mid block's four convs; the head.
enum {
  E_CONV_IN = 0,
  E_DOWN_BASE = 1,                 // + 4 s + 2 k + cv
  E_TD_BASE = E_DOWN_BASE + 16,    // + 2 k + half
  E_MID_BASE = E_TD_BASE + 4,      // mid0 conv1, conv2, mid1 conv1, conv2
  E_HEAD = E_MID_BASE + 4,
  E_RING_COUNT = E_HEAD + 1
};

int enc_ring_down(int s, int k, int cv) { return E_DOWN_BASE + 4 * s + 2 * k + cv; }

// Channels and level (0: h x w, ..., 3: 8h x 8w) of encoder ring id.
RingInfo enc_ring_info(int c, int id) {
  if (id == E_CONV_IN) return {kEncInC, 3};
  if (id < E_TD_BASE) {
    const int r = id - E_DOWN_BASE, s = r / 4, k = (r / 2) % 2, cv = r % 2;
    const int cin = (k == 0 && cv == 0) ? (s == 0 ? c : enc_width(c, s - 1)) : enc_width(c, s);
    return {cin, 3 - s};
  }
  if (id < E_MID_BASE) {
    const int k = (id - E_TD_BASE) / 2;  // stage k + 1, after its spatial down-conv
    return {enc_width(c, k + 1), 1 - k};
  }
  return {4 * c, 0};
}

Work make_work_enc(int c, int h, int w, int P) {
  Work W;
  const long long r0 = (long long)h * w;
  const long long res[4] = {r0, 4 * r0, 16 * r0, 64 * r0};
  const long long c4 = 4 * c, c2 = 2 * c;
  const long long F0 = P, F1 = 2LL * P, F2 = 4LL * P;
  const long long act = std::max({F2 * res[3] * std::max<long long>(c, kEncInC), F2 * res[2] * c2, F2 * res[1] * c2,
                                  F1 * res[1] * c4, F1 * res[0] * c4, F0 * res[0] * c4});
  const long long L = r0;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  W.X_bytes = W.H_bytes = W.Y_bytes = (size_t)act * 2;
  W.X = take(W.X_bytes);
  W.H = take(W.H_bytes);
  W.Y = take(W.Y_bytes);
  W.zt = W.zp = take(0);
  W.rs = take((size_t)(F2 + 2) * res[3] * 4);
  W.qkv = take((size_t)F0 * L * 3 * c4 * 2);
  take_attention(W, take, F0, L, c4);
  {
    // Winograd planes of the ResBlock convs of each level (frames, input and
    // output widths), as make_work does for the decoder.
    struct Lv { long long F, H, W; long long cin[4], cout[4]; };
    const Lv lv[4] = {
        {F2, 8LL * h, 8LL * w, {c, c, c, c}, {c, c, c, c}},
        {F2, 4LL * h, 4LL * w, {c, c2, c2, c2}, {c2, c2, c2, c2}},
        {F1, 2LL * h, 2LL * w, {c2, c4, c4, c4}, {c4, c4, c4, c4}},
        {F0, (long long)h, (long long)w, {c4, c4, c4, c4}, {c4, c4, c4, c4}},
    };
    long long u = 0, m = 0;
    for (const Lv& l : lv) {
      const long long wq = (l.W + kWinoM - 1) / kWinoM;
      for (int i = 0; i < 4; ++i) {
        if (!wino_ok((int)l.cin[i], (int)l.cout[i])) continue;
        u = std::max(u, kWinoN * (l.F + 2) * l.H * wq * l.cin[i]);
        m = std::max(m, kWinoN * l.F * l.H * wq * l.cout[i]);
      }
    }
    W.U = take((size_t)u * 2);
    W.M = take((size_t)m * 2);
  }
  size_t roff = 0;
  for (int i = 0; i < E_RING_COUNT; ++i) {
    RingInfo ri = enc_ring_info(c, i);
    W.ring.push_back(roff);
    roff = align_up(roff + (size_t)2 * res[ri.level] * ri.cin * 2);
  }
  W.ring_bytes = roff;
  W.rings = take(roff);
  W.total = off;
  return W;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

struct ProfRec {
  int cls;
  double flops;
  hipEvent_t e0, e1;
};

}  // namespace

struct wvd_plan {
  int c, h, w;
  Layout L;
  unsigned char* prep;
  bool profile = false;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  size_t pool_used = 0;

  long long launches = 0;  // kernel launches of the last wvd_decode
  int magic = 0x77766470;
};

namespace {

bool plan_ok(const wvd_plan* p) { return p && p->magic == 0x77766470; }
bool dec_plan_ok(const wvd_plan* p) { return plan_ok(p) && !p->L.encoder; }
bool enc_plan_ok(const wvd_plan* p) { return plan_ok(p) && p->L.encoder; }

int check_dims(int c, int h, int w) {
  if (c <= 0 || c % 16 != 0 || 4 * c > kMaxCin) return WVD_EUNSUPPORTED;
  if (h < 1 || w < 1 || h > 4096 || w > 4096) return WVD_EUNSUPPORTED;
  return WVD_OK;
}

// ---------------------------------------------------------------------------
// Decode-time scheduler
// ---------------------------------------------------------------------------

thread_local std::string g_last_error;

void set_error(const char* what, hipError_t e) {
  g_last_error = std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
}

struct Ctx {
  wvd_plan* plan;
  hipStream_t st;
  unsigned char* ws;
  const Work* W;
  hipError_t err = hipSuccess;
  const char* what = "";
  // The tensor (data pointer and frame count) whose pass-frame statistics the
  // rs buffer already holds (written by a Winograd output transform), or null.
  const h16_t* rs_tensor = nullptr;
  int rs_frames = 0;

  template <typename T>
  T* prep(int item) const { return reinterpret_cast<T*>(plan->prep + plan->L.items[item].off); }
  template <typename T>
  T* wsp(size_t off) const { return reinterpret_cast<T*>(ws + off); }
  unsigned char* ringbase = nullptr;  // the ring block (workspace or stream state)
  h16_t* ring(int id) const { return reinterpret_cast<h16_t*>(ringbase + W->ring[id]); }
  long long wbytes(int item) const { return (long long)plan->L.items[item].bytes; }

  hipEvent_t ev() {
    if (plan->pool_used == plan->pool.size()) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      plan->pool.push_back(e);
    }
    return plan->pool[plan->pool_used++];
  }
  // A host-side check failed: no launch; the decode returns WVD_EHIP with
  // the reason in wvd_last_error.
  void fail(const char* why) {
    if (err != hipSuccess) return;
    err = hipErrorInvalidValue;
    set_error(why, err);
  }
  // A write of `bytes` starting at p: where p is the start of the X, H or Y
  // buffer, the write must fit in that buffer's capacity.
  void check_fits(const void* p, size_t bytes, const char* what) {
    const size_t cap = p == wsp<unsigned char>(W->X)   ? W->X_bytes
                       : p == wsp<unsigned char>(W->H) ? W->H_bytes
                       : p == wsp<unsigned char>(W->Y) ? W->Y_bytes
                                                       : ~(size_t)0;
    if (bytes > cap) fail(what);
  }
  template <typename F>
  void run(int cls, double flops, F&& fn) {
    if (err != hipSuccess) return;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (plan->profile) {
      e0 = ev();
      e1 = ev();
      // a pair whose first record fails is not timed
      if (e0 && hipEventRecord(e0, st) != hipSuccess) e0 = nullptr;
    }
    err = fn();
    if (err != hipSuccess) set_error(what, err);
    ++plan->launches;
    if (plan->profile && e0 && e1 && hipEventRecord(e1, st) == hipSuccess) {
      plan->recs.push_back({cls, flops, e0, e1});
    }
  }
};

ConvSeg seg_basic(const h16_t* x, long long x_fstride, int lda, int Cin, const h16_t* w, int ldw,
                  long long tap_stride, int KT, int KS, long long w_bytes = 0) {
  ConvSeg s;
  std::memset(&s, 0, sizeof(s));
  s.x = x;
  s.x_fstride = x_fstride;
  s.lda = lda;
  s.Cin = Cin;
  s.w = w;
  s.ldw = ldw;
  s.w_tap_stride = tap_stride;
  s.KT = KT;
  s.KS = KS;
  s.prologue = PRO_RAW;
  s.wfrag = 1;
  s.w_bytes = w_bytes;
  return s;
}

void set_grid(ConvArgs& a, int F, int H, int W, int TF, int TW = kTileW) {
  a.F = F;
  a.H = H;
  a.W = W;
  a.TF = TF;
  a.TW = TW;
  a.TH = kTileM / TW / TF;
  a.tiles_x = (W + TW - 1) / TW;
  a.tiles_y = (H + a.TH - 1) / a.TH;
  a.tiles_f = (F + TF - 1) / TF;
  if (a.nphase == 0) a.nphase = 1;
  // Halo rows per LDS buffer: every segment's halo, rounded up so that whole
  // rounds of 16-byte items (one per thread) land on real (or spare) rows.
  int np = 4;
  for (int s = 0; s < a.nseg; ++s)
    if (a.seg[s].Cin % 32) np = 2;
  int rows = 0;
  for (int s = 0; s < a.nseg; ++s) {
    const ConvSeg& g = a.seg[s];
    const int hsy = g.KS == KS_1x1 ? 0 : 1;
    const int hsx = g.KS == KS_1x1 || g.KS == KS_3x1 ? 0 : 1;
    const int st = g.stride == 2 ? 2 : 1;
    const int nhv = (TF + g.KT - 1) * (st * a.TH + 2 * hsy - (st - 1)) * (st * TW + 2 * hsx - (st - 1));
    if (st == 2) np = 2;  // strided halos are staged in 16-channel chunks
    rows = std::max(rows, (nhv * np + 511) / 512 * 512 / np);  // whole rounds for 256 or 512 threads
    // the Winograd and up-conv epilogues stage their rows in one halo buffer
    if (g.KS == KS_3x1 || g.KS == KS_PHASE)
      rows = std::max(rows, (kSwapEpiBytes / (32 * 2 + 16) + 16) / 16 * 16);
  }
  a.nhv_max = rows;
}

ConvArgs args_init() {
  ConvArgs a;
  std::memset(&a, 0, sizeof(a));
  a.scale = 1.0f;
  a.TW = kTileW;
  a.nphase = 1;
  return a;
}

double conv_flops(const ConvArgs& a) {
  double f = 0;
  const double vox = (double)a.F * a.H * a.W * a.nphase;
  for (int s = 0; s < a.nseg; ++s) {
    const ConvSeg& g = a.seg[s];
    const int k2 = g.KS == KS_3x3 ? 9 : (g.KS == KS_PHASE ? 4 : (g.KS == KS_3x1 ? 3 : 1));
    f += 2.0 * vox * a.Cout * (double)g.KT * k2 * g.Cin;
  }
  return f;
}

void conv(Ctx& cx, ConvArgs& a, int cls) {
  a.zero_row = reinterpret_cast<const h16_t*>(cx.plan->prep + cx.plan->L.zero_off);
  a.zero_len = cx.plan->L.zero_len;
  const char* why = conv_check(a);
  if (why && cx.err == hipSuccess) {
    cx.err = hipErrorInvalidValue;
    g_last_error = std::string("conv launch check: ") + why;
    return;
  }
  cx.what = "conv";
  cx.rs_tensor = nullptr;  // any conv may overwrite the tensor whose statistics rs holds
  // Class 0 is exactly the dominant kernel instantiation; other convs of
  // the caller's class 0 are reported as class 1.
  if (cls == 0 && !conv_is_main(a)) cls = 1;
  cx.run(cls, conv_flops(a), [&] { return launch_conv(a, cx.st); });
}

struct Act {
  h16_t* p;
  int C;      // channels (= voxel stride)
  int F;      // frames in this pass
  int H, W;
  long long fstride() const { return (long long)H * W * C; }
};

// rs for the history slots and the F pass frames of x; the pass frames are
// skipped when the output transform that produced x already wrote them.
void stats(Ctx& cx, const Act& x, const h16_t* ring, int nh) {
  float* rs = cx.wsp<float>(cx.W->rs);
  const int F = (cx.rs_tensor == x.p && cx.rs_frames == x.F) ? 0 : x.F;
  cx.rs_tensor = nullptr;
  if (F + nh == 0) return;
  cx.what = "rms_stats";
  cx.run(3, 0, [&] { return launch_rms_stats(x.p, x.fstride(), x.C, ring, nh, x.C, F, x.H * x.W, rs, cx.st); });
}

void ring_update(Ctx& cx, h16_t* ring, const Act& x) {
  cx.what = "ring_update";
  cx.run(4, 0, [&] { return launch_ring_update(ring, x.p, x.fstride(), x.C, x.C, x.F, x.H * x.W, cx.st); });
}

// Temporal-3 convs use 2-frame tiles (a single-frame pass masks the second
// frame); the 1-frame, 16-row tile of a 3x3x3 conv would not fit in LDS.
int tf_for(int KT, int F) {
  (void)F;
  return KT == 3 ? 2 : 1;
}

// Tile shape of the Winograd-domain GEMM: TF frames x TH rows x TW column
// groups (256 positions).  The GEMM is power-limited, and its halo loads (U
// rows of the TF + 2 frames and TH + 2 rows around the tile) are much of the
// power: deeper tiles in t and y load fewer halo rows per output.  The choice
// minimises rounds of tiles over the CUs times (1 + 0.1 x halo rows per
// output), which also keeps the 20- and 39-column-group levels from mostly
// empty wide tiles.  A tile of 128 output channels takes half the time of
// one of 256 at about 1.15 times the cost per multiply-add (each A fragment
// feeds two MFMAs instead of four); it wins where 256-channel tiles would
// leave much of a last round idle (the 44x78 level: 384 tiles, 1.5 rounds).
struct WinoShape {
  int TF, TW, bn;
};

WinoShape wino_tile_shape(int F, int H, int WQ, int Cout) {
  static int slots = 0;
  if (!slots) {
    int dev = 0, n = 0;
    if (!g_dry_run && hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      slots = n;
    else
      slots = 256;
  }
  static const WinoShape cand[] = {{2, 16, 256}, {2, 8, 256}, {4, 8, 256}, {4, 4, 256}, {8, 4, 256},
                                   {2, 16, 128}, {2, 8, 128}, {4, 8, 128}, {4, 4, 128}, {8, 4, 128}};
  WinoShape best = cand[0];
  double best_cost = 1e300;
  for (const WinoShape& c : cand) {
    if (Cout % c.bn) continue;
    const int th = kTileM / c.TW / c.TF;
    const long long tiles = (long long)((WQ + c.TW - 1) / c.TW) * ((H + th - 1) / th) * ((F + c.TF - 1) / c.TF) *
                            kWinoN * (Cout / c.bn);
    const double halo = (double)(c.TF + 2) * (th + 2) / (c.TF * th);
    const double per_tile = c.bn == 256 ? 1.0 : 0.5 * 1.15;
    const double cost = (double)((tiles + slots - 1) / slots) * per_tile * (1.0 + 0.1 * halo);
    if (cost < best_cost) {
      best_cost = cost;
      best = c;
    }
  }
  return best;
}

// Causal 3x3x3 norm-SiLU conv in Winograd form along x:
//   U = F(kWinoM,3) input transform of SiLU(norm(x)) over the F frames and the
//       valid history frames (the transform computes the norm statistics),
//   M[xi] = causal (t, y) 3x3 conv of U[xi] with the transformed weights,
//   out = output transform of M + bias (+ res).
// Same function as conv333 + EPI_H16, with 4/9 of the multiply-adds (F(6,3):
// 8 planes x 9 (t, y) taps for 6 outputs x 27 taps).
// The Winograd GEMM over the U planes the input transform (or the fused
// transform) left for input x: M = the kWinoN planes of products.
void wino_gemm(Ctx& cx, const Act& x, int nh, int w_item, int Cout) {
  const int W2 = (x.W + kWinoM - 1) / kWinoM;  // column groups
  h16_t* U = cx.wsp<h16_t>(cx.W->U);
  h16_t* M = cx.wsp<h16_t>(cx.W->M);
  const long long uslot = (long long)x.H * W2 * x.C;     // elements per U frame
  const long long uplane = (long long)(x.F + 2) * uslot;  // per xi plane
  const long long mframe = (long long)x.H * W2 * Cout;
  ConvArgs a = args_init();
  ConvSeg& g = a.seg[0];
  g = seg_basic(U + 2 * uslot, uslot, x.C, x.C, cx.prep<h16_t>(w_item), x.C, 0, 3, KS_3x1, cx.wbytes(w_item));
  g.ring = U;  // slots 0 and 1 of every plane: the history frames
  g.n_hist = nh;
  g.x_pstride = uplane;
  a.nseg = 1;
  a.nphase = kWinoN;
  a.Cout = Cout;
  a.out = M;
  a.out_fstride = mframe;
  a.out_pstride = (long long)x.F * mframe;
  a.ldo = Cout;
  a.epi = EPI_WINO;
  const WinoShape ts = wino_tile_shape(x.F, x.H, W2, Cout);
  set_grid(a, x.F, x.H, W2, ts.TF, ts.TW);
  a.bn = ts.bn;
  conv(cx, a, 0);
}

// act_gamma >= 0: out receives SiLU(RMSNorm(v) * gamma) of the conv output v
// instead of v (and no norm statistics).
void wino_out(Ctx& cx, const Act& x, int b_item, int Cout, const Act& out, const h16_t* res, long long res_fstride,
              int ldr, int act_gamma = -1) {
  cx.what = "wino_out";
  cx.run(5, 0, [&] {
    return launch_wino_out(cx.wsp<h16_t>(cx.W->M), Cout, x.F, x.H, x.W, b_item >= 0 ? cx.prep<float>(b_item) : nullptr,
                           res, res_fstride, ldr, out.p, out.fstride(), out.C,
                           act_gamma >= 0 ? nullptr : cx.wsp<float>(cx.W->rs),
                           act_gamma >= 0 ? cx.prep<float>(act_gamma) : nullptr, cx.st);
  });
  cx.rs_tensor = act_gamma >= 0 ? nullptr : out.p;
  cx.rs_frames = x.F;
}

void conv_wino(Ctx& cx, const Act& x, h16_t* ring, int nh, int gamma_item, int w_item, int b_item, int Cout,
               const Act& out, const h16_t* res, long long res_fstride, int ldr) {
  cx.what = "wino_in";
  cx.run(5, 0, [&] {
    return launch_wino_in(x.p, x.fstride(), x.C, ring, nh, x.C, x.F, x.H, x.W, cx.prep<float>(gamma_item),
                          cx.wsp<h16_t>(cx.W->U), cx.st);
  });
  wino_gemm(cx, x, nh, w_item, Cout);
  wino_out(cx, x, b_item, Cout, out, res, res_fstride, ldr);
}

// Causal 3x3x3 conv with the fused RMSNorm+SiLU prologue.
ConvArgs conv333(Ctx& cx, const Act& x, h16_t* ring, int nh, int gamma_item, int w_item, int b_item, int Cout) {
  ConvArgs a = args_init();
  ConvSeg& s = a.seg[0];
  s = seg_basic(x.p, x.fstride(), x.C, x.C, cx.prep<h16_t>(w_item), x.C, (long long)Cout * x.C, 3, 3,
                cx.wbytes(w_item));
  s.ring = ring;
  s.n_hist = nh;
  s.rs = cx.wsp<float>(cx.W->rs);
  s.gamma = cx.prep<float>(gamma_item);
  s.prologue = PRO_NORM_SILU;
  a.nseg = 1;
  a.Cout = Cout;
  a.bias = cx.prep<float>(b_item);
  return a;
}

// True where resblock() can hand out SiLU(RMSNorm(output) * gamma) in
// place of its output (conv2 in Winograd form with the residual in place).
bool resblock_can_activate(const RB& rb) { return rb.wino1 && rb.wino2 && wino_mid_ok(rb.cout) && rb.cin == rb.cout; }

// ResBlock: x -> x (in place) when widths match, else x -> out.  With
// act_gamma >= 0 (only where resblock_can_activate) the block's output is
// replaced by SiLU(RMSNorm(output) * gamma), for a consumer that needs only
// that (the head).
Act resblock(Ctx& cx, const RB& rb, const Act& x, h16_t* hbuf, h16_t* obuf, int ring1, int ring2, int nh,
             int act_gamma = -1) {
  if (act_gamma >= 0 && !resblock_can_activate(rb)) {
    cx.fail("resblock activation");
    return x;
  }
  h16_t* r1 = cx.ring(ring1);
  h16_t* r2 = cx.ring(ring2);
  if (!rb.wino1) stats(cx, x, r1, nh);  // the Winograd input transform computes its own
  Act h{hbuf, rb.cout, x.F, x.H, x.W};
  const bool fused = rb.wino1 && rb.wino2 && wino_mid_ok(rb.cout);
  {
    // frames of h stored into hbuf (fused blocks: only a one-frame pass's)
    const long long hf = fused ? (x.F >= 2 ? 0 : x.F) : x.F;
    cx.check_fits(hbuf, (size_t)hf * x.H * x.W * rb.cout * 2, "resblock: conv1 output beyond its buffer");
    if (rb.cin != rb.cout)
      cx.check_fits(obuf, (size_t)x.F * x.H * x.W * rb.cout * 2, "resblock: output beyond its buffer");
    if (cx.err != hipSuccess) return x;
  }
  if (fused) {
    // conv1's products go straight into conv2's input planes: h is stored
    // only for the frames the next pass reads as history (its ring)
    cx.what = "wino_in";
    cx.run(5, 0, [&] {
      return launch_wino_in(x.p, x.fstride(), x.C, r1, nh, x.C, x.F, x.H, x.W, cx.prep<float>(rb.norm1),
                            cx.wsp<h16_t>(cx.W->U), cx.st);
    });
    wino_gemm(cx, x, nh, rb.conv1w, rb.cout);
    cx.what = "wino_in_history";
    cx.run(5, 0, [&] {
      return launch_wino_in(h.p, h.fstride(), h.C, r2, nh, h.C, h.F, h.H, h.W, cx.prep<float>(rb.norm2),
                            cx.wsp<h16_t>(cx.W->U), cx.st, true);
    });
    // With two or more frames in the pass the last two are exactly the next
    // pass's history: they go straight into the ring (slots 0, 1); a
    // one-frame pass stores its frame in h and shifts the ring below.
    const int tail = std::max(0, x.F - 2);
    cx.what = "wino_mid";
    cx.run(5, 0, [&] {
      return launch_wino_mid(cx.wsp<h16_t>(cx.W->M), cx.prep<float>(rb.conv1b), rb.cout, x.F, x.H, x.W,
                             cx.prep<float>(rb.norm2), cx.wsp<h16_t>(cx.W->U), x.F >= 2 ? r2 : h.p,
                             x.F >= 2 ? (long long)x.H * x.W * h.C : h.fstride(), h.C, tail, x.F >= 2 ? tail : 0,
                             cx.st);
    });
    cx.rs_tensor = nullptr;
  } else if (rb.wino1) {
    conv_wino(cx, x, r1, nh, rb.norm1, rb.conv1w, rb.conv1b, rb.cout, h, nullptr, 0, 0);
  } else {
    ConvArgs a = conv333(cx, x, r1, nh, rb.norm1, rb.conv1w, rb.conv1b, rb.cout);
    a.out = h.p;
    a.out_fstride = h.fstride();
    a.ldo = h.C;
    a.epi = EPI_H16;
    set_grid(a, x.F, x.H, x.W, tf_for(3, x.F));
    conv(cx, a, 0);
  }
  ring_update(cx, r1, x);
  if (!rb.wino2) stats(cx, h, r2, nh);
  Act out{rb.cin == rb.cout ? x.p : obuf, rb.cout, x.F, x.H, x.W};
  // conv2: input planes from its own transform, or already there (fused)
  auto conv2_wino = [&](int b_item, const h16_t* res, long long res_fstride, int ldr) {
    if (fused) {
      wino_gemm(cx, h, nh, rb.conv2w, rb.cout);
      wino_out(cx, h, b_item, rb.cout, out, res, res_fstride, ldr, act_gamma);
    } else {
      conv_wino(cx, h, r2, nh, rb.norm2, rb.conv2w, b_item, rb.cout, out, res, res_fstride, ldr);
    }
  };
  if (rb.wino2 && rb.cin == rb.cout) {  // residual x, written in place
    conv2_wino(rb.conv2b, x.p, x.fstride(), x.C);
  } else if (rb.wino2) {
    // shortcut first (1x1 GEMM over the raw input, with the pre-summed
    // biases of conv2 and the shortcut), then conv2 adds onto it in place
    const long long Mv = (long long)x.F * x.H * x.W;
    cx.rs_tensor = nullptr;
    if (Mv >= 256 && rb.cin % 128 == 0) {
      cx.what = "shortcut_gemm";
      cx.run(1, 2.0 * Mv * rb.cout * rb.cin, [&] {
        return launch_gemm1x1(x.p, Mv, x.C, rb.cin, cx.prep<h16_t>(rb.scw), cx.wbytes(rb.scw), rb.cout,
                              cx.prep<float>(rb.scb), out.p, out.C, cx.st);
      });
    } else {  // passes too small for a 256-row tile: the generic 1x1 conv
      ConvArgs a = args_init();
      a.seg[0] = seg_basic(x.p, x.fstride(), x.C, rb.cin, cx.prep<h16_t>(rb.scw), rb.cin, 0, 1, 1, cx.wbytes(rb.scw));
      a.nseg = 1;
      a.Cout = rb.cout;
      a.bias = cx.prep<float>(rb.scb);
      a.out = out.p;
      a.out_fstride = out.fstride();
      a.ldo = out.C;
      a.epi = EPI_H16;
      set_grid(a, x.F, x.H, x.W, 1);
      conv(cx, a, 1);
    }
    conv2_wino(-1, out.p, out.fstride(), out.C);
  } else {
    ConvArgs a = conv333(cx, h, r2, nh, rb.norm2, rb.conv2w, rb.conv2b, rb.cout);
    if (rb.cin == rb.cout) {
      a.res = x.p;
      a.res_fstride = x.fstride();
      a.ldr = x.C;
    } else {
      // 1x1x1 shortcut over the raw block input as a second K segment; its
      // bias is pre-summed with conv2's into the shortcut bias slot.
      a.seg[1] = seg_basic(x.p, x.fstride(), x.C, x.C, cx.prep<h16_t>(rb.scw), x.C, 0, 1, 1, cx.wbytes(rb.scw));
      a.nseg = 2;
      a.bias = cx.prep<float>(rb.scb);
    }
    a.out = out.p;
    a.out_fstride = out.fstride();
    a.ldo = out.C;
    a.epi = EPI_H16;
    set_grid(a, x.F, x.H, x.W, tf_for(3, x.F));
    conv(cx, a, 0);
  }
  if (!(fused && x.F >= 2)) ring_update(cx, r2, h);
  return out;
}

GemmArgs gemm_args() {
  GemmArgs g;
  std::memset(&g, 0, sizeof(g));
  g.scale = 1.0f;
  g.nF = 1;
  return g;
}

// Per-frame single-head attention on the batched 256 x 256 GEMM:
//   xn = RMSNorm(x); qkv = xn Wqkv^T + b;
//   per frame, with K and V^T in fragment order: the score pass computes
//   s = q.k / sqrt(C) and, per query and group g of 64 keys, the maximum
//   m_g; it stores e^(s - m_g) in fp16 (zero for the padding keys) and
//   (m_g, sum of e^(s - m_g)); a per-query pass takes the maximum M and the
//   sum S over the groups and scales the group's values by e^(m_g - M) / S,
//   which gives P = softmax(s) in place; O = P V; x += O Wp^T + bp.
// The fp32 scores are never stored, and each score is computed once.
void attention_fast(Ctx& cx, const Act& x) {
  const Layout& L = cx.plan->L;
  const int C = x.C, Lt = x.H * x.W;
  const long long Np = attn_np(Lt);
  h16_t* qkv = cx.wsp<h16_t>(cx.W->qkv);
  h16_t* O = cx.wsp<h16_t>(cx.W->O);  // also xn, which is dead before O is written
  h16_t* P = cx.wsp<h16_t>(cx.W->Pm);
  h16_t* kf = cx.wsp<h16_t>(cx.W->kf);
  h16_t* vf = cx.wsp<h16_t>(cx.W->vf);
  float* st = cx.wsp<float>(cx.W->st);
  const long long rows = (long long)x.F * Lt;
  cx.rs_tensor = nullptr;
  cx.what = "attention norm";
  cx.run(3, 0, [&] {
    return launch_norm_silu(x.p, x.fstride(), C, C, x.F, Lt, cx.prep<float>(L.attn_norm), O, (long long)Lt * C, C,
                            cx.st, false);
  });
  GemmArgs g = gemm_args();
  g.x = O;
  g.M = rows;
  g.lda = C;
  g.K = C;
  g.w = cx.prep<h16_t>(L.qkv_w);
  g.w_bytes = cx.wbytes(L.qkv_w);
  g.N = 3 * C;
  g.bias = cx.prep<float>(L.qkv_b);
  g.out = qkv;
  g.ldo = 3 * C;
  cx.what = "attention qkv";
  cx.run(2, 2.0 * rows * 3 * C * C, [&] { return launch_gemm_nt(g, G_H16, cx.st); });
  cx.what = "attention fragments";
  cx.run(4, 0, [&] { return launch_attn_frag(qkv, x.F, Lt, C, (int)Np, kf, vf, cx.st); });
  g = gemm_args();
  g.x = qkv;  // queries: the first third of each qkv row
  g.M = Lt;
  g.lda = 3 * C;
  g.K = C;
  g.w = kf;
  g.w_bytes = Np * C * 2;
  g.N = (int)Np;
  g.scale = 1.0f / std::sqrt((float)C);
  g.nF = x.F;
  g.a_fs = (long long)Lt * 3 * C;
  g.w_fs = Np * C;
  g.n_valid = Lt;
  g.stats = st;
  g.out = P;
  g.ldo = (int)Np;
  g.o_fs = Lt * Np;
  cx.what = "attention scores";
  cx.run(2, 2.0 * x.F * Lt * Np * C, [&] { return launch_gemm_nt(g, G_STATS, cx.st); });
  cx.what = "attention softmax";
  cx.run(4, 0, [&] { return launch_attn_rescale(P, st, rows, (int)Np, cx.st); });
  g = gemm_args();
  g.x = P;
  g.M = Lt;
  g.lda = (int)Np;
  g.K = (int)Np;
  g.w = vf;
  g.w_bytes = Np * C * 2;
  g.N = C;
  g.nF = x.F;
  g.a_fs = Lt * Np;
  g.w_fs = Np * C;
  g.out = O;
  g.ldo = C;
  g.o_fs = (long long)Lt * C;
  cx.what = "attention P V";
  cx.run(2, 2.0 * x.F * Lt * C * Np, [&] { return launch_gemm_nt(g, G_H16, cx.st); });
  g = gemm_args();
  g.x = O;
  g.M = rows;
  g.lda = C;
  g.K = C;
  g.w = cx.prep<h16_t>(L.proj_w);
  g.w_bytes = cx.wbytes(L.proj_w);
  g.N = C;
  g.bias = cx.prep<float>(L.proj_b);
  g.res = x.p;
  g.ldr = C;
  g.out = x.p;
  g.ldo = C;
  cx.what = "attention projection";
  cx.run(2, 2.0 * rows * C * C, [&] { return launch_gemm_nt(g, G_H16, cx.st); });
}

void attention(Ctx& cx, const Act& x) {
  if (attn_fast(x.C, (long long)x.H * x.W)) {
    attention_fast(cx, x);
    return;
  }
  const Layout& L = cx.plan->L;
  const int C = x.C, Lt = x.H * x.W, Lp = lpad_of(Lt);
  h16_t* qkv = cx.wsp<h16_t>(cx.W->qkv);
  float* S = cx.wsp<float>(cx.W->S);
  h16_t* Pm = cx.wsp<h16_t>(cx.W->Pm);
  h16_t* Vt = cx.wsp<h16_t>(cx.W->Vt);
  h16_t* O = cx.wsp<h16_t>(cx.W->O);
  stats(cx, x, nullptr, 0);
  {  // qkv = Wqkv RMSNorm(x) + b
    ConvArgs a = args_init();
    a.seg[0] = seg_basic(x.p, x.fstride(), C, C, cx.prep<h16_t>(L.qkv_w), C, 0, 1, 1, cx.wbytes(L.qkv_w));
    a.seg[0].rs = cx.wsp<float>(cx.W->rs);
    a.seg[0].gamma = cx.prep<float>(L.attn_norm);
    a.seg[0].prologue = PRO_NORM;
    a.nseg = 1;
    a.Cout = 3 * C;
    a.bias = cx.prep<float>(L.qkv_b);
    a.out = qkv;
    a.out_fstride = (long long)Lt * 3 * C;
    a.ldo = 3 * C;
    a.epi = EPI_H16;
    set_grid(a, x.F, x.H, x.W, 1);
    conv(cx, a, 1);
  }
  {  // S = Q K^T / sqrt(C), per frame
    ConvArgs a = args_init();
    a.seg[0] = seg_basic(qkv, (long long)Lt * 3 * C, 3 * C, C, qkv + C, 3 * C, 0, 1, 1);
    a.seg[0].w_frame_stride = (long long)Lt * 3 * C;
    a.seg[0].wfrag = 0;  // K rows of the qkv activations
    a.nseg = 1;
    a.Cout = Lt;
    a.scale = 1.0f / std::sqrt((float)C);
    a.out = S;
    a.out_fstride = (long long)Lt * Lp;
    a.ldo = Lp;
    a.epi = EPI_F32;
    set_grid(a, x.F, x.H, x.W, 1);
    conv(cx, a, 2);
  }
  cx.run(4, 0, [&] { return launch_softmax_rows(S, x.F * Lt, Lt, Lp, Pm, cx.st); });
  cx.run(4, 0, [&] { return launch_transpose_v(qkv, x.F, Lt, C, Lp, Vt, cx.st); });
  {  // O = P V
    ConvArgs a = args_init();
    a.seg[0] = seg_basic(Pm, (long long)Lt * Lp, Lp, Lp, Vt, Lp, 0, 1, 1);
    a.seg[0].w_frame_stride = (long long)C * Lp;
    a.seg[0].wfrag = 0;  // rows of V^T
    a.nseg = 1;
    a.Cout = C;
    a.out = O;
    a.out_fstride = (long long)Lt * C;
    a.ldo = C;
    a.epi = EPI_H16;
    set_grid(a, x.F, x.H, x.W, 1);
    conv(cx, a, 2);
  }
  {  // x += Wp O + bp
    ConvArgs a = args_init();
    a.seg[0] = seg_basic(O, (long long)Lt * C, C, C, cx.prep<h16_t>(L.proj_w), C, 0, 1, 1, cx.wbytes(L.proj_w));
    a.nseg = 1;
    a.Cout = C;
    a.bias = cx.prep<float>(L.proj_b);
    a.res = x.p;
    a.res_fstride = x.fstride();
    a.ldr = C;
    a.out = x.p;
    a.out_fstride = x.fstride();
    a.ldo = C;
    a.epi = EPI_H16;
    set_grid(a, x.F, x.H, x.W, 1);
    conv(cx, a, 1);
  }
}

// time_conv: x (F frames, first global frame g) -> y (interleaved frames).
Act time_upsample(Ctx& cx, int s, const Act& x, int g, h16_t* ybuf, int ring_id) {
  const Layout& L = cx.plan->L;
  h16_t* ring = cx.ring(ring_id);
  const bool first = g == 0;
  Act y{ybuf, x.C, first ? 2 * x.F - 1 : 2 * x.F, x.H, x.W};
  cx.check_fits(ybuf, (size_t)y.F * y.fstride() * 2, "time_conv: output beyond its buffer");
  if (first) {
    cx.run(4, 0, [&] { return launch_copy16(y.p, x.p, (size_t)x.fstride() * 2, cx.st); });
  }
  Act sx{first ? x.p + x.fstride() : x.p, x.C, first ? x.F - 1 : x.F, x.H, x.W};
  if (sx.F == 0) return y;
  const int nh = std::min(2, std::max(0, g - 1));
  ConvArgs a = args_init();
  a.seg[0] = seg_basic(sx.p, sx.fstride(), sx.C, sx.C, cx.prep<h16_t>(L.tc_w[s]), sx.C, 2LL * sx.C * sx.C, 3, 1,
                       cx.wbytes(L.tc_w[s]));
  a.seg[0].ring = ring;
  a.seg[0].n_hist = nh;
  a.nseg = 1;
  a.Cout = 2 * x.C;
  a.bias = cx.prep<float>(L.tc_b[s]);
  a.out = y.p;
  a.out_fstride = y.fstride();
  a.ldo = y.C;
  a.epi = EPI_TIME;
  a.out_base = first ? 1 : 0;
  set_grid(a, sx.F, sx.H, sx.W, tf_for(3, sx.F));
  conv(cx, a, 1);
  ring_update(cx, ring, sx);
  return y;
}

// Nearest-2x + Conv2d 3x3 in phase form: x [F][H][W][C] -> y [F][2H][2W][C].
Act up_conv(Ctx& cx, int s, const Act& x, h16_t* ybuf) {
  const Layout& L = cx.plan->L;
  Act y{ybuf, x.C, x.F, 2 * x.H, 2 * x.W};
  cx.check_fits(ybuf, (size_t)y.F * y.fstride() * 2, "up-conv: output beyond its buffer");
  ConvArgs a = args_init();
  a.seg[0] = seg_basic(x.p, x.fstride(), x.C, x.C, cx.prep<h16_t>(L.upc_w[s]), x.C, (long long)x.C * x.C, 1, 2,
                       cx.wbytes(L.upc_w[s]));
  a.nseg = 1;
  a.nphase = 4;
  a.Cout = x.C;
  a.bias = cx.prep<float>(L.upc_b[s]);
  a.out = y.p;
  a.out_fstride = y.fstride();
  a.ldo = y.C;
  a.epi = EPI_PHASE;
  set_grid(a, x.F, x.H, x.W, 1);
  conv(cx, a, 1);
  return y;
}

// Prepares every item of layout L from the canonical tensors and returns the
// plan (wvd_prepare and wvd_encoder_prepare).
int prepare_plan(int c, int h, int w, const Layout& L, const void* const* weights, int weight_dtype, void* prepared,
                 hipStream_t s, wvd_plan** plan_out) {
  wvd_plan* p = new (std::nothrow) wvd_plan();
  if (!p) return WVD_EINVAL;
  p->c = c;
  p->h = h;
  p->w = w;
  p->L = L;
  p->prep = static_cast<unsigned char*>(prepared);
  hipError_t e = hipSuccess;
  for (size_t i = 0; i < L.items.size() && e == hipSuccess; ++i) {
    const Item& it = L.items[i];
    const void* src = weights[it.src >= 0 ? it.src : (int)i];
    void* dst = p->prep + it.off;
    if (it.kind == K_WINO)
      e = launch_prep_wino_frag(src, weight_dtype, it.cout, it.cin, static_cast<h16_t*>(dst), s);
    else if (it.kind == K_CONV)
      e = launch_prep_frag(src, weight_dtype, it.cout, it.cin, it.taps, it.cin_pad, static_cast<h16_t*>(dst), s);
    else if (it.kind == K_CONV_PART)
      e = launch_prep_frag_part(src, weight_dtype, it.cout, it.cin_src, it.cin_off, it.cin, it.taps, it.cin_pad,
                                static_cast<h16_t*>(dst), s);
    else if (it.kind == K_PHASE)
      e = launch_prep_phase_frag(src, weight_dtype, it.cout, static_cast<h16_t*>(dst), s);
    else if (it.kind == K_S2D)
      e = launch_prep_s2d_frag(src, weight_dtype, it.cout, static_cast<h16_t*>(dst), s);
    else if (it.kind == K_HEADX)
      e = launch_prep_headx_frag(src, weight_dtype, it.cin, static_cast<h16_t*>(dst), s);
    else
      e = launch_prep_vec(src, weight_dtype, it.n, it.scale, static_cast<float*>(dst), s);
  }
  if (e == hipSuccess) e = launch_fill_zero(p->prep + L.zero_off, align_up((size_t)L.zero_len * 2), s);
  // Blocks with a shortcut add two biases; keep their sum in the shortcut slot.
  const RB* sc_blocks[2] = {L.encoder ? &L.down[1][0] : &L.up[2][0], L.encoder ? &L.down[2][0] : &L.up[3][0]};
  for (const RB* rb : sc_blocks) {
    if (e != hipSuccess) break;
    e = launch_prep_vec_add(weights[rb->conv2b], weights[rb->scb], weight_dtype, rb->cout,
                            reinterpret_cast<float*>(p->prep + L.items[rb->scb].off), s);
  }
  if (e != hipSuccess) {
    set_error(L.encoder ? "wvd_encoder_prepare" : "wvd_prepare", e);
    delete p;
    return WVD_EHIP;
  }
  *plan_out = p;
  return WVD_OK;
}

}  // namespace

extern "C" {

const char* wvd_status_string(int st) {
  switch (st) {
    case WVD_OK: return "ok";
    case WVD_EINVAL: return "invalid argument";
    case WVD_ESHAPE: return "shape inconsistent with the plan";
    case WVD_ENOSPACE: return "buffer smaller than required";
    case WVD_EUNSUPPORTED: return "unsupported configuration";
    case WVD_EHIP: return "HIP error";
    default: return "unknown status";
  }
}

int wvd_prepared_bytes(int c, int h, int w, size_t* bytes) {
  return wvd_prepared_bytes_n(c, h, w, WVD_NUM_WEIGHTS, bytes);
}

int wvd_prepared_bytes_n(int c, int h, int w, int n_weights, size_t* bytes) {
  if (!bytes) return WVD_EINVAL;
  if (n_weights != WVD_NUM_WEIGHTS && n_weights != WVD_NUM_WEIGHTS_DEEP) return WVD_EINVAL;
  int st = check_dims(c, h, w);
  if (st) return st;
  *bytes = make_layout(c, h, w, n_weights == WVD_NUM_WEIGHTS_DEEP).total;
  return WVD_OK;
}

int wvd_prepare(int c, int h, int w, const void* const* weights, int n_weights, int weight_dtype, void* prepared,
                size_t prepared_bytes, void* stream, wvd_plan** plan_out) {
  if (!weights || !prepared || !plan_out) return WVD_EINVAL;
  if (weight_dtype != WVD_DTYPE_BF16 && weight_dtype != WVD_DTYPE_F32) return WVD_EINVAL;
  int st = check_dims(c, h, w);
  if (st) return st;
  if (n_weights != WVD_NUM_WEIGHTS && n_weights != WVD_NUM_WEIGHTS_DEEP) return WVD_EINVAL;
  for (int i = 0; i < n_weights; ++i)
    if (!weights[i]) return WVD_EINVAL;
  if (!aligned16(prepared)) return WVD_EINVAL;
  Layout L = make_layout(c, h, w, n_weights == WVD_NUM_WEIGHTS_DEEP);
  if ((int)L.items.size() != n_weights) return WVD_EINVAL;
  if (prepared_bytes < L.total) return WVD_ENOSPACE;
  return prepare_plan(c, h, w, L, weights, weight_dtype, prepared, static_cast<hipStream_t>(stream), plan_out);
}

int wvd_workspace_bytes(const wvd_plan* plan, int T, int frames_per_pass, size_t* bytes) {
  if (!dec_plan_ok(plan) || !bytes || T < 1 || frames_per_pass < 1) return WVD_EINVAL;
  const int P = std::min(T, frames_per_pass);
  *bytes = make_work(plan->c, plan->h, plan->w, P, true, plan->L.nrb).total;
  return WVD_OK;
}

}  // extern "C"

namespace {

// Video frames of the first t latent frames.
long long video_frames(long long t) { return t > 0 ? 4 * t - 3 : 0; }

// Decode latent frames [t_begin, t_begin + T) (z holds just those) into their
// video frames [video_frames(t_begin), video_frames(t_begin + T)).  The rings
// carry the causal history: in the workspace (t_begin = 0, state = null) or
// in the caller's stream state.
int decode_impl(wvd_plan* plan, const void* z, int z_dtype, int T, int t_begin, int frames_per_pass, void* state,
                void* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int c = plan->c, h = plan->h, w = plan->w;
  const int P = std::min(T, frames_per_pass);
  Work W = make_work(c, h, w, P, state == nullptr, plan->L.nrb);
  if (workspace_bytes < W.total) return WVD_ENOSPACE;
  const Layout& L = plan->L;
  Ctx cx;
  cx.plan = plan;
  cx.st = stream;
  cx.ws = static_cast<unsigned char*>(workspace);
  cx.W = &W;
  cx.ringbase = state ? static_cast<unsigned char*>(state) : cx.ws + W.rings;
  plan->launches = 0;
  const int c4 = 4 * c;
  h16_t* X = cx.wsp<h16_t>(W.X);
  h16_t* Hb = cx.wsp<h16_t>(W.H);
  h16_t* Y = cx.wsp<h16_t>(W.Y);
  h16_t* const zt0 = cx.wsp<h16_t>(W.zt);
  const long long vbase = video_frames(t_begin);
  const int VT = (int)(video_frames((long long)t_begin + T) - vbase);

  for (int t0 = 0; t0 < T && cx.err == hipSuccess; t0 += P) {
    const int F0 = std::min(P, T - t0);
    const int G = t_begin + t0;  // global index of the pass's first latent frame
    const bool first = G == 0;
    const int g0 = G, g1 = first ? 0 : 2 * G - 1, g2 = first ? 0 : 4 * G - 3;
    const int nh0 = std::min(2, g0), nh1 = std::min(2, g1), nh2 = std::min(2, g2);
    // conv_in on the channels-last latents.
    cx.what = "latent_to_cl";
    h16_t* zt = zt0;
    cx.run(4, 0, [&] { return launch_latent_to_cl(z, z_dtype, T, t0, F0, h * w, zt, cx.st); });
    if (L.pre_w >= 0) {  // deep variant: the 48 -> 48 1x1x1 conv on the latents
      h16_t* zp = cx.wsp<h16_t>(W.zp);
      cx.what = "pre_conv";
      cx.run(1, 2.0 * F0 * h * w * 48 * 48, [&] {
        return launch_pre_conv(zt, F0 * h * w, cx.prep<float>(L.pre_w), cx.prep<float>(L.pre_b), zp, cx.st);
      });
      zt = zp;
    }
    Act za{zt, 64, F0, h, w};
    Act x{X, c4, F0, h, w};
    {
      h16_t* ring = cx.ring(R_CONV_IN);
      ConvArgs a = args_init();
      a.seg[0] = seg_basic(zt, za.fstride(), 64, 64, cx.prep<h16_t>(L.conv_in_w), 64, (long long)c4 * 64, 3, 3,
                           cx.wbytes(L.conv_in_w));
      a.seg[0].ring = ring;
      a.seg[0].n_hist = nh0;
      a.nseg = 1;
      a.Cout = c4;
      a.bias = cx.prep<float>(L.conv_in_b);
      a.out = x.p;
      a.out_fstride = x.fstride();
      a.ldo = c4;
      a.epi = EPI_H16;
      set_grid(a, F0, h, w, tf_for(3, F0));
      conv(cx, a, 0);
      ring_update(cx, ring, za);
    }
    x = resblock(cx, L.mid0, x, Hb, nullptr, R_MID0_1, R_MID0_2, nh0);
    attention(cx, x);
    x = resblock(cx, L.mid1, x, Hb, nullptr, R_MID1_1, R_MID1_2, nh0);
    const int nrb = L.nrb;
    // The last ResBlock hands the head its normalised input directly (in
    // place of the block output, which nothing else reads) where it can.
    const bool head_fused = resblock_can_activate(L.up[3][nrb - 1]);
    auto stage = [&](int s, int nh) {  // the stage's ResBlocks; the first may change the width
      for (int k = 0; k < nrb; ++k)
        x = resblock(cx, L.up[s][k], x, Hb, k == 0 && s >= 2 ? Y : nullptr, ring_up(nrb, s, k, 0),
                     ring_up(nrb, s, k, 1), nh, s == 3 && k == nrb - 1 && head_fused ? L.head_norm : -1);
    };
    // Stage 0 (h x w), time_conv, up-conv to 2h x 2w.
    stage(0, nh0);
    Act y = time_upsample(cx, 0, x, g0, Y, ring_tc(nrb, 0));
    x = up_conv(cx, 0, y, X);
    // Stage 1 (2h x 2w).
    stage(1, nh1);
    y = time_upsample(cx, 1, x, g1, Y, ring_tc(nrb, 1));
    x = up_conv(cx, 1, y, X);
    // Stage 2 (4h x 4w): 4c -> 2c.
    stage(2, nh2);
    x = up_conv(cx, 2, x, X);
    // Stage 3 (8h x 8w): 2c -> c.
    stage(3, nh2);
    // Head: RMSNorm + SiLU + conv c -> 12, pixel shuffle, clamp, NCTHW video.
    // With only 12 output channels the conv's halo staging would normalise
    // each voxel many times per output; the normalised input is written once
    // instead: by the last ResBlock's output transform (head_fused), else by
    // a norm-SiLU pass into the free H buffer.  The head's history ring
    // holds normalised frames.
    {
      h16_t* ring = cx.ring(ring_head(L.nrb));
      Act yn{head_fused ? x.p : Hb, x.C, x.F, x.H, x.W};
      if (!head_fused) cx.check_fits(Hb, (size_t)x.F * x.H * x.W * x.C * 2, "head: input beyond its buffer");
      if (!head_fused) {
        cx.what = "norm_silu";
        cx.run(3, 0, [&] {
          return launch_norm_silu(x.p, x.fstride(), x.C, x.C, x.F, x.H * x.W, cx.prep<float>(L.head_norm), yn.p,
                                  yn.fstride(), yn.C, cx.st);
        });
      }
      ConvArgs a = args_init();
      // Packed form (widths a multiple of 32): nine (t, y) taps over the
      // input columns, the three x taps as output columns 12 dx + co, tiles
      // of 4 frames x 4 rows x 16 columns making 14 output columns each.
      const bool packed = L.items[L.head_w].kind == K_HEADX;
      a.seg[0] = seg_basic(yn.p, yn.fstride(), yn.C, yn.C, cx.prep<h16_t>(L.head_w), yn.C, (long long)12 * yn.C, 3,
                           packed ? KS_3x1 : KS_3x3, cx.wbytes(L.head_w));
      a.seg[0].ring = ring;
      a.seg[0].n_hist = nh2;
      a.nseg = 1;
      a.Cout = packed ? 64 : 12;
      a.bias = cx.prep<float>(L.head_b);
      a.out = out;
      a.epi = EPI_VIDEO;
      a.out_base = (int)(g2 - vbase);
      a.video_T = VT;
      if (packed) {
        set_grid(a, x.F, x.H, x.W, 4, 16);
        a.tiles_x = (x.W + 13) / 14;
      } else {
        set_grid(a, x.F, x.H, x.W, tf_for(3, x.F));
      }
      conv(cx, a, 0);
      ring_update(cx, ring, yn);
    }
  }
  if (cx.err != hipSuccess) return WVD_EHIP;
  return WVD_OK;
}


// ---------------------------------------------------------------------------
// Encoder (R13-R16): video [1, 3, 4T-3, 16h, 16w] -> latents [1, 48, T, h, w]
// ---------------------------------------------------------------------------

// Spatial down-conv (R14): Conv2d 3x3, stride 2, zero pad 1, per frame:
// x [F][2H][2W][C] -> y [F][H][W][Cout].
Act down_conv(Ctx& cx, int s, const Act& x, h16_t* ybuf, h16_t* sbuf) {
  // 3x3 stride-2 conv (pad 1) in space-to-depth form: x's four phase images
  // side by side in channels (into sbuf), then a 2x2 conv over them at offsets
  // -1, 0 on the phase-tap kernel with one phase and a plain store.
  const Layout& L = cx.plan->L;
  Act y{ybuf, x.C, x.F, x.H / 2, x.W / 2};
  Act z{sbuf, 4 * x.C, x.F, y.H, y.W};
  cx.what = "space_to_depth";
  cx.run(4, 0, [&] { return launch_space_to_depth(x.p, x.fstride(), x.C, x.F, x.H, x.W, z.p, cx.st); });
  ConvArgs a = args_init();
  a.seg[0] = seg_basic(z.p, z.fstride(), z.C, z.C, cx.prep<h16_t>(L.dc_w[s]), z.C, 0, 1, KS_PHASE,
                       cx.wbytes(L.dc_w[s]));
  a.nseg = 1;
  a.nphase = 1;
  a.Cout = x.C;
  a.bias = cx.prep<float>(L.dc_b[s]);
  a.out = y.p;
  a.out_fstride = y.fstride();
  a.ldo = y.C;
  a.epi = EPI_H16;
  set_grid(a, y.F, y.H, y.W, 1);
  conv(cx, a, 1);
  return y;
}

// Temporal down-conv (R15) of stage k + 1: x (F frames, the clip's first
// frame first when `first`) -> y.  The clip's first frame is copied; the
// pairs (2s+1, 2s+2) after it (or (2s, 2s+1) in a later pass) are the two K
// segments of one causal 3x1x1 conv, each reading every second frame and
// carrying its own two history frames.
Act time_down(Ctx& cx, int k, const Act& x, bool first, h16_t* ybuf, int nh) {
  const Layout& L = cx.plan->L;
  const int npairs = first ? (x.F - 1) / 2 : x.F / 2;
  Act y{ybuf, x.C, npairs + (first ? 1 : 0), x.H, x.W};
  if (first) {
    cx.what = "copy";
    cx.run(4, 0, [&] { return launch_copy16(y.p, x.p, (size_t)x.fstride() * 2, cx.st); });
  }
  if (npairs == 0) return y;
  const h16_t* p0 = first ? x.p + x.fstride() : x.p;  // first frame of the first pair
  const long long pstride = 2 * x.fstride();
  ConvArgs a = args_init();
  for (int h = 0; h < 2; ++h) {
    a.seg[h] = seg_basic(p0 + h * x.fstride(), pstride, x.C, x.C, cx.prep<h16_t>(L.td_w[k][h]), x.C, 0, 3, KS_1x1,
                         cx.wbytes(L.td_w[k][h]));
    a.seg[h].ring = cx.ring(E_TD_BASE + 2 * k + h);
    a.seg[h].n_hist = nh;
  }
  a.nseg = 2;
  a.Cout = x.C;
  a.bias = cx.prep<float>(L.td_b[k]);
  a.out = y.p + (first ? y.fstride() : 0);
  a.out_fstride = y.fstride();
  a.ldo = y.C;
  a.epi = EPI_H16;
  set_grid(a, npairs, x.H, x.W, tf_for(3, npairs));
  conv(cx, a, 1);
  for (int h = 0; h < 2; ++h) {
    h16_t* ring = cx.ring(E_TD_BASE + 2 * k + h);
    cx.what = "ring_update";
    cx.run(4, 0, [&] {
      return launch_ring_update(ring, p0 + h * x.fstride(), pstride, x.C, x.C, npairs, x.H * x.W, cx.st);
    });
  }
  return y;
}

int encode_impl(wvd_plan* plan, const void* video, int v_dtype, int T, int frames_per_pass, float* latents,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int c = plan->c, h = plan->h, w = plan->w;
  const int P = std::min(T, frames_per_pass);
  Work W = make_work_enc(c, h, w, P);
  if (workspace_bytes < W.total) return WVD_ENOSPACE;
  const Layout& L = plan->L;
  Ctx cx;
  cx.plan = plan;
  cx.st = stream;
  cx.ws = static_cast<unsigned char*>(workspace);
  cx.W = &W;
  cx.ringbase = cx.ws + W.rings;
  plan->launches = 0;
  const int c4 = 4 * c;
  h16_t* X = cx.wsp<h16_t>(W.X);
  h16_t* Hb = cx.wsp<h16_t>(W.H);
  h16_t* Y = cx.wsp<h16_t>(W.Y);
  const int Tv = 4 * T - 3;
  for (int t0 = 0; t0 < T && cx.err == hipSuccess; t0 += P) {
    const int F0 = std::min(P, T - t0);
    const bool first = t0 == 0;
    const int vb = first ? 0 : 4 * t0 - 3;  // first video frame of the pass
    const int F2 = first ? 4 * F0 - 3 : 4 * F0;
    const int g2 = vb, g1 = first ? 0 : 2 * t0 - 1, g0 = t0;
    const int nh2 = std::min(2, g2), nh1 = std::min(2, g1), nh0 = std::min(2, g0);
    // 2x2 patchify into kEncInC channels (12 + zero pad), then conv_in 12 -> c.
    Act zt{Y, kEncInC, F2, 8 * h, 8 * w};
    cx.what = "patchify";
    cx.run(4, 0, [&] { return launch_patchify(video, v_dtype, Tv, vb, F2, 8 * h, 8 * w, Y, cx.st); });
    Act x{X, c, F2, 8 * h, 8 * w};
    {
      h16_t* ring = cx.ring(E_CONV_IN);
      ConvArgs a = args_init();
      a.seg[0] = seg_basic(zt.p, zt.fstride(), kEncInC, kEncInC, cx.prep<h16_t>(L.conv_in_w), kEncInC, 0, 3, KS_3x3,
                           cx.wbytes(L.conv_in_w));
      a.seg[0].ring = ring;
      a.seg[0].n_hist = nh2;
      a.nseg = 1;
      a.Cout = c;
      a.bias = cx.prep<float>(L.conv_in_b);
      a.out = x.p;
      a.out_fstride = x.fstride();
      a.ldo = c;
      a.epi = EPI_H16;
      set_grid(a, F2, x.H, x.W, tf_for(3, F2));
      conv(cx, a, 1);
      ring_update(cx, ring, zt);
    }
    // Stage 0 (8h x 8w, c), down to 4h x 4w.
    x = resblock(cx, L.down[0][0], x, Hb, nullptr, enc_ring_down(0, 0, 0), enc_ring_down(0, 0, 1), nh2);
    x = resblock(cx, L.down[0][1], x, Hb, nullptr, enc_ring_down(0, 1, 0), enc_ring_down(0, 1, 1), nh2);
    x = down_conv(cx, 0, x, Y, Hb);
    // Stage 1 (4h x 4w, c -> 2c), down to 2h x 2w, frames 4T-3 -> 2T-1.
    x = resblock(cx, L.down[1][0], x, Hb, X, enc_ring_down(1, 0, 0), enc_ring_down(1, 0, 1), nh2);
    x = resblock(cx, L.down[1][1], x, Hb, nullptr, enc_ring_down(1, 1, 0), enc_ring_down(1, 1, 1), nh2);
    x = down_conv(cx, 1, x, Y, Hb);
    x = time_down(cx, 0, x, first, X, first ? 0 : std::min(2, 2 * t0 - 2));
    // Stage 2 (2h x 2w, 2c -> 4c), down to h x w, frames 2T-1 -> T.
    x = resblock(cx, L.down[2][0], x, Hb, Y, enc_ring_down(2, 0, 0), enc_ring_down(2, 0, 1), nh1);
    x = resblock(cx, L.down[2][1], x, Hb, nullptr, enc_ring_down(2, 1, 0), enc_ring_down(2, 1, 1), nh1);
    x = down_conv(cx, 2, x, X, Hb);
    x = time_down(cx, 1, x, first, Y, first ? 0 : std::min(2, t0 - 1));
    // Stage 3 (h x w, 4c), then the mid block.
    x = resblock(cx, L.down[3][0], x, Hb, nullptr, enc_ring_down(3, 0, 0), enc_ring_down(3, 0, 1), nh0);
    x = resblock(cx, L.down[3][1], x, Hb, nullptr, enc_ring_down(3, 1, 0), enc_ring_down(3, 1, 1), nh0);
    x = resblock(cx, L.mid0, x, Hb, nullptr, E_MID_BASE, E_MID_BASE + 1, nh0);
    attention(cx, x);
    x = resblock(cx, L.mid1, x, Hb, nullptr, E_MID_BASE + 2, E_MID_BASE + 3, nh0);
    // Head: RMSNorm + SiLU in the conv prologue, causal 3x3x3 conv 4c -> 48,
    // fp32 NCTHW latents.
    {
      h16_t* ring = cx.ring(E_HEAD);
      stats(cx, x, ring, nh0);
      ConvArgs a = conv333(cx, x, ring, nh0, L.head_norm, L.head_w, L.head_b, 48);
      a.out = latents;
      a.epi = EPI_LATENT;
      a.out_base = t0;
      a.video_T = T;
      set_grid(a, x.F, x.H, x.W, tf_for(3, x.F));
      conv(cx, a, 1);
      ring_update(cx, ring, x);
    }
    (void)c4;
  }
  if (cx.err != hipSuccess) return WVD_EHIP;
  return WVD_OK;
}

}  // namespace

extern "C" {

int wvd_decode(const wvd_plan* cplan, const void* z, int z_dtype, int T, int frames_per_pass, void* out,
               void* workspace, size_t workspace_bytes, void* stream) {
  if (!dec_plan_ok(cplan) || !z || !out || !workspace || T < 1 || frames_per_pass < 1) return WVD_EINVAL;
  if (z_dtype != WVD_DTYPE_BF16 && z_dtype != WVD_DTYPE_F32) return WVD_EINVAL;
  if (!aligned16(workspace)) return WVD_EINVAL;
  return decode_impl(const_cast<wvd_plan*>(cplan), z, z_dtype, T, 0, frames_per_pass, nullptr, out, workspace,
                     workspace_bytes, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// Decode without allocation: the workspace is this file-scope device array
// (one copy per device, held until the process ends).  Host code never uses
// the array's name as an address: the device address of each device's copy is
// looked up once, with that device current, and kept in g_scratch_addr.
// ---------------------------------------------------------------------------

namespace {

constexpr size_t kStaticWorkspaceBytes = WVD_STATIC_WORKSPACE_BYTES;
constexpr int kMaxDevices = 64;
static_assert(kStaticWorkspaceBytes % kAlign == 0, "static workspace size");

__device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on the first call on
// each device).
int static_workspace(void** addr) {
  if (g_dry_run) {  // nothing is dereferenced: any aligned placeholder will do
    *addr = reinterpret_cast<void*>(static_cast<uintptr_t>(1) << 20);
    return WVD_OK;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error("wvd_decode_static: hipGetDevice", e);
    return WVD_EHIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    g_last_error = "wvd_decode_static: device index beyond the static table";
    return WVD_EUNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      set_error("wvd_decode_static: hipGetSymbolAddress(scratch)", e != hipSuccess ? e : hipErrorInvalidSymbol);
      return WVD_EHIP;
    }
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return WVD_OK;
}

}  // namespace

int wvd_decode_static(const wvd_plan* cplan, const void* z, int z_dtype, int T, int frames_per_pass, void* out,
                      void* stream) {
  if (!dec_plan_ok(cplan) || !z || !out || T < 1 || frames_per_pass < 1) return WVD_EINVAL;
  if (z_dtype != WVD_DTYPE_BF16 && z_dtype != WVD_DTYPE_F32) return WVD_EINVAL;
  const int P = std::min(T, frames_per_pass);
  const size_t need = make_work(cplan->c, cplan->h, cplan->w, P, true, cplan->L.nrb).total;
  if (need > kStaticWorkspaceBytes) {
    g_last_error = "wvd_decode_static: this decode needs " + std::to_string(need) +
                   " workspace bytes, more than the static workspace of " + std::to_string(kStaticWorkspaceBytes) +
                   " bytes (use wvd_decode with a caller-owned workspace, or a smaller frames_per_pass)";
    return WVD_ENOSPACE;
  }
  void* ws = nullptr;
  const int st = static_workspace(&ws);
  if (st != WVD_OK) return st;
  return decode_impl(const_cast<wvd_plan*>(cplan), z, z_dtype, T, 0, frames_per_pass, nullptr, out, ws,
                     kStaticWorkspaceBytes, static_cast<hipStream_t>(stream));
}

int wvd_state_bytes(const wvd_plan* plan, size_t* bytes) {
  if (!dec_plan_ok(plan) || !bytes) return WVD_EINVAL;
  *bytes = make_work(plan->c, plan->h, plan->w, 1, false, plan->L.nrb).ring_bytes;
  return WVD_OK;
}

int wvd_chunk_workspace_bytes(const wvd_plan* plan, int T, int frames_per_pass, size_t* bytes) {
  if (!dec_plan_ok(plan) || !bytes || T < 1 || frames_per_pass < 1) return WVD_EINVAL;
  *bytes = make_work(plan->c, plan->h, plan->w, std::min(T, frames_per_pass), false, plan->L.nrb).total;
  return WVD_OK;
}

int wvd_decode_chunk(const wvd_plan* cplan, const void* z, int z_dtype, int T, int t_begin, int frames_per_pass,
                     void* state, size_t state_bytes, void* out, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (!dec_plan_ok(cplan) || !z || !out || !workspace || !state || T < 1 || t_begin < 0 || frames_per_pass < 1)
    return WVD_EINVAL;
  if (z_dtype != WVD_DTYPE_BF16 && z_dtype != WVD_DTYPE_F32) return WVD_EINVAL;
  if (!aligned16(workspace) || !aligned16(state)) return WVD_EINVAL;
  if ((long long)t_begin + T > (1LL << 28)) return WVD_EINVAL;  // video frame indices stay in int
  size_t need = 0;
  wvd_state_bytes(cplan, &need);
  if (state_bytes < need) return WVD_ENOSPACE;
  return decode_impl(const_cast<wvd_plan*>(cplan), z, z_dtype, T, t_begin, frames_per_pass, state, out, workspace,
                     workspace_bytes, static_cast<hipStream_t>(stream));
}

const char* wvd_last_error(void) { return g_last_error.c_str(); }

int wvd_math_probe(const float* x, float* silu_out, float* exp_out, long long n, void* stream) {
  if (n < 0 || (n > 0 && (!x || !silu_out || !exp_out))) return WVD_EINVAL;
  if (n > (1LL << 31)) return WVD_EINVAL;
  hipError_t e = launch_math_probe(x, silu_out, exp_out, n, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_error("wvd_math_probe", e);
    return WVD_EHIP;
  }
  return WVD_OK;
}

int wvd_f16_probe(const float* x, unsigned short* h_out, float* rs_out, long long n, void* stream) {
  if (n < 0 || n % 8 || (n > 0 && (!x || !h_out || !rs_out))) return WVD_EINVAL;
  if (n > (1LL << 31)) return WVD_EINVAL;
  if (!aligned16(x) || !aligned16(h_out) || !aligned16(rs_out)) return WVD_EINVAL;
  hipError_t e = launch_f16_probe(x, h_out, rs_out, n, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_error("wvd_f16_probe", e);
    return WVD_EHIP;
  }
  return WVD_OK;
}

int wvd_range_flags(void* stream, int clear, unsigned int* flags) {
  if (!flags) return WVD_EINVAL;
  *flags = 0;
  if (g_dry_run) return WVD_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  unsigned int* addr[2] = {nullptr, nullptr};
  unsigned int host[2] = {0, 0};
  hipError_t e = conv_range_flags_addr(&addr[0]);
  if (e == hipSuccess) e = aux_range_flags_addr(&addr[1]);
  for (int i = 0; i < 2 && e == hipSuccess; ++i)
    e = hipMemcpyAsync(&host[i], addr[i], sizeof(unsigned int), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  for (int i = 0; i < 2 && e == hipSuccess && clear; ++i) e = hipMemsetAsync(addr[i], 0, sizeof(unsigned int), st);
  if (e == hipSuccess && clear) e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    set_error("wvd_range_flags", e);
    return WVD_EHIP;
  }
  *flags = host[0] | host[1];
  return WVD_OK;
}

void wvd_set_dry_run(int on) { g_dry_run = on != 0; }

long long wvd_last_launch_count(const wvd_plan* plan) { return plan_ok(plan) ? plan->launches : -1; }

void wvd_destroy(wvd_plan* plan) {
  if (!plan_ok(plan)) return;
  for (hipEvent_t e : plan->pool) (void)hipEventDestroy(e);
  plan->magic = 0;
  delete plan;
}

int wvd_profile_enable(wvd_plan* plan, int on) {
  if (!plan_ok(plan)) return WVD_EINVAL;
  plan->profile = on != 0;
  return WVD_OK;
}

int wvd_profile_read(const wvd_plan* cplan, double* ms, double* flops, long long* launches, int n_classes) {
  if (!plan_ok(cplan) || !ms || !flops || !launches || n_classes < 1) return WVD_EINVAL;
  wvd_plan* plan = const_cast<wvd_plan*>(cplan);
  if (!plan->recs.empty() && hipEventSynchronize(plan->recs.back().e1) != hipSuccess) return WVD_EHIP;
  double m[6] = {0, 0, 0, 0, 0, 0}, f[6] = {0, 0, 0, 0, 0, 0};
  long long n[6] = {0, 0, 0, 0, 0, 0};
  for (const ProfRec& r : plan->recs) {
    float t = 0;
    if (hipEventElapsedTime(&t, r.e0, r.e1) != hipSuccess) return WVD_EHIP;
    m[r.cls] += t;
    f[r.cls] += r.flops;
    n[r.cls] += 1;
  }
  for (int i = 0; i < n_classes && i < 6; ++i) {
    ms[i] = m[i];
    flops[i] = f[i];
    launches[i] = n[i];
  }
  plan->recs.clear();
  plan->pool_used = 0;
  return WVD_OK;
}

// ---- encoder ----

int wvd_encoder_prepared_bytes(int c, int h, int w, size_t* bytes) {
  if (!bytes) return WVD_EINVAL;
  int st = check_dims(c, h, w);
  if (st) return st;
  *bytes = make_layout_enc(c, h, w).total;
  return WVD_OK;
}

int wvd_encoder_prepare(int c, int h, int w, const void* const* weights, int n_weights, int weight_dtype,
                        void* prepared, size_t prepared_bytes, void* stream, wvd_plan** plan_out) {
  if (!weights || !prepared || !plan_out) return WVD_EINVAL;
  if (weight_dtype != WVD_DTYPE_BF16 && weight_dtype != WVD_DTYPE_F32) return WVD_EINVAL;
  int st = check_dims(c, h, w);
  if (st) return st;
  if (n_weights != WVD_NUM_WEIGHTS_ENCODER) return WVD_EINVAL;
  for (int i = 0; i < n_weights; ++i)
    if (!weights[i]) return WVD_EINVAL;
  if (!aligned16(prepared)) return WVD_EINVAL;
  Layout L = make_layout_enc(c, h, w);
  if (prepared_bytes < L.total) return WVD_ENOSPACE;
  return prepare_plan(c, h, w, L, weights, weight_dtype, prepared, static_cast<hipStream_t>(stream), plan_out);
}

int wvd_encode_workspace_bytes(const wvd_plan* plan, int T, int frames_per_pass, size_t* bytes) {
  if (!enc_plan_ok(plan) || !bytes || T < 1 || frames_per_pass < 1) return WVD_EINVAL;
  *bytes = make_work_enc(plan->c, plan->h, plan->w, std::min(T, frames_per_pass)).total;
  return WVD_OK;
}

int wvd_encode(const wvd_plan* cplan, const void* video, int video_dtype, int T, int frames_per_pass, float* latents,
               void* workspace, size_t workspace_bytes, void* stream) {
  if (!enc_plan_ok(cplan) || !video || !latents || !workspace || T < 1 || frames_per_pass < 1) return WVD_EINVAL;
  if (video_dtype != WVD_DTYPE_BF16 && video_dtype != WVD_DTYPE_F32) return WVD_EINVAL;
  if (!aligned16(workspace)) return WVD_EINVAL;
  if (T > (1 << 28)) return WVD_EINVAL;
  return encode_impl(const_cast<wvd_plan*>(cplan), video, video_dtype, T, frames_per_pass, latents, workspace,
                     workspace_bytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"
