// ssim_kernels.hip -- fused SSIM loss, forward and backward, for gfx950.
//
// What is computed ("Fully Fused Differentiable SSIM", opening section and
// Usage; "TriSSIM", How it works and Usage): the SSIM map of the 11x11
// Gaussian window, loss = 1 - mean(map), and its gradient with respect to
// both images through the adjoint B^T of the blur and the chain rule.
//
// Readings of the pages that keep the work and the rounding error down
// without changing the result:
//   * One blur pass serves several statistics ("Fully Fused Differentiable
//     SSIM", opening section).  SSIM needs the second moments only through
//     sigma_xy and sigma_x^2 + sigma_y^2 = 2 sigma_xy + var(x - y), so four
//     blurred quantities suffice: mu_x' = B(x'), mu_y' = B(y'),
//     P' = B(x' y') and R = B((x - y)^2), with x' = x - 1/2, y' = y - 1/2.
//     Then, with dmu = mu_x - mu_y,
//         A1 = 2 mu_x mu_y + C1,  D1 = dmu^2,            B1 = A1 + D1
//         A2 = 2 (P' - mu_x' mu_y') + C2,  D2 = R - dmu^2, B2 = A2 + D2
//         1 - S = (A1 D2 + D1 B2) / (B1 B2).
//     The shift by 1/2 leaves every variance unchanged and halves the
//     magnitudes that cancel in P' - mu_x' mu_y'; the difference basis makes
//     B1 - A1 and B2 - A2 exact by construction, so identical images give a
//     loss and gradients of exactly zero and near-identical images (SSIM
//     near 1, the end of a training run) keep full relative accuracy in
//     1 - S, which is what the loss sums.
//   * The pages send five upstream gradients through B^T (mu1, mu2, s11, s22,
//     s12); in the basis above there are four, m0..m3 = d loss /
//     d(mu_x', mu_y', R, P') (R's with the chain rule's 2 folded in), and
//         grad_x = dloss * (B^T m0 + y' * B^T m3 + (x - y) * B^T m2)
//         grad_y = dloss * (B^T m1 + x' * B^T m3 - (x - y) * B^T m2).
//   * The window is symmetric and B^T of a zero-filled correlation is a
//     correlation with the same taps shifted by the padding; so forward and
//     backward are one "blur with input offset" skeleton:
//         out[i][j] = sum_{a,b} g[a] g[b] in[i + a - off][j + b - off],
//     in = 0 outside its extent (for the forward: pixels x = y = 0 there, so
//     x' = y' = -1/2 -- load-then-shift produces exactly that).  Forward:
//     off = 0 (valid) or 5 (same); backward: off = 10 (valid: the "full"
//     correlation) or 5 (same).
//
// Skeleton (one workgroup = 4 wave64 = 256 lanes; one strip = 256 input
// columns -> 244 output columns):
//   column pass : lane t owns input column j0 - off + t.  It marches down the
//                 rows, loading its own pixel per row straight from HBM
//                 (coalesced across lanes), and keeps the last 11 rows of the
//                 four quantities in a 12-slot register ring; each new row
//                 gives one column-blurred row of the four quantities.
//   row pass    : batches of 4 column-blurred rows go through a double-
//                 buffered LDS tile [quantity][row][256] (32 KiB); wave w then
//                 takes row w of the batch and lane l produces the 4 adjacent
//                 outputs 4l..4l+3 from 4 aligned 16-byte LDS reads per
//                 quantity (conflict-free: lanes read consecutive 16 bytes).
//   consumer    : forward -> 1 - SSIM into the loss sum and, in training
//                 mode, the four blurred quantities stored as four map planes
//                 (16 bytes per plane per lane); backward -> chain rule and
//                 two gradient stores.  The backward's column pass forms the
//                 loss partials from the saved quantities as it reads them:
//                 the forward is ALU-bound and the backward memory-bound, so
//                 the partials' arithmetic sits where it is free.
// Work is split by strip-column ((plane, strip) pairs): on a grid of about
// one wave of resident workgroups, each strip-column is cut into equal row
// ranges, one per workgroup (or, with more strip-columns than workgroups,
// each workgroup takes whole strip-columns), so every workgroup gets the
// same work.  A workgroup marches down its range so that every input row is
// loaded and column-blurred once, plus a 10-row warm-up where the range
// starts.  Workgroup ids are remapped so that each of the 8 XCDs (separate
// L2s) owns one contiguous eighth of the grid.
//
// Loss reduction: the map entries of 1 - S are summed as per-lane fp32 sums
// of 4 outputs -> fp64 per lane -> wave64 shuffle tree -> LDS -> one fp64
// partial per workgroup -> the last workgroup (completion ticket) sums the
// partials in a fixed order and writes loss = sum / M.  Deterministic; no
// atomics on floating point.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "ssim_loss_amd.h"

#if defined(__HIP_DEVICE_COMPILE__)
#if !defined(__gfx950__)
#error "this library targets gfx950 (MI355X) only"
#endif
#endif

namespace {

constexpr int kWave = 64;        // gfx9 wavefront size; checked on the host at run time
constexpr int kThreads = 256;    // 4 waves per workgroup
constexpr int kWaves = kThreads / kWave;
constexpr int kTileW = 256;      // input columns per strip: one per lane
constexpr int kStripOut = 244;   // outputs per strip: 256 - 10, rounded down to a multiple of 4
constexpr int kRowLanes = kStripOut / 4;  // lanes active in the row pass (61)
constexpr int kRows = 4;         // rows per batch = waves (one row each in the row pass)
constexpr int kRing = 12;        // ring slots: 11 rows needed, 12 so 3 batches of 4 close the cycle
constexpr int kQ = 4;            // blurred quantities / maps
constexpr int kMaxBlocks = 4096; // bound on the grid (size of the partial-sum table)
constexpr int kMinRowsPerBlock = 8;

static_assert(kRows == kWaves, "row pass maps one batch row per wave");
static_assert(4 * (kRowLanes - 1) + 16 <= kTileW, "row-pass reads stay inside the tile");
static_assert(kStripOut + 10 <= kTileW, "a strip's halo fits the tile");
static_assert(kStripOut % 4 == 0, "strips start on 16-byte boundaries");

// 1-D Gaussian taps: exp(-(k-5)^2 / (2 * 1.5^2)) normalised to sum 1 (the
// original SSIM paper's window; "Fully Fused Differentiable SSIM" hard-codes
// its weights), written out to 17 significant digits and rounded once to
// fp32.  Symmetric: g[k] == g[10-k].
constexpr float kTap0 = 0.0010283800844791100f;
constexpr float kTap1 = 0.0075987581352391900f;
constexpr float kTap2 = 0.036000772128430830f;
constexpr float kTap3 = 0.10936068950970002f;
constexpr float kTap4 = 0.21300553771125370f;
constexpr float kTap5 = 0.26601172486179436f;

__host__ __device__ constexpr float tap(int k) {
  return (k == 0 || k == 10) ? kTap0
       : (k == 1 || k == 9)  ? kTap1
       : (k == 2 || k == 8)  ? kTap2
       : (k == 3 || k == 7)  ? kTap3
       : (k == 4 || k == 6)  ? kTap4
                             : kTap5;
}

constexpr float kC1 = 1.0e-4f;  // (0.01 * 1)^2
constexpr float kC2 = 9.0e-4f;  // (0.03 * 1)^2
constexpr float kShift = 0.5f;  // x' = x - 1/2 (see the file header)

struct Workspace {
  unsigned int ticket;
  unsigned int pad[63];
  double partial[kMaxBlocks];
};

enum Mode { kFwdInfer = 0, kFwdTrain = 1, kBwd = 2 };

struct Params {
  // blur geometry
  int in_h, in_w;       // extent of the blurred input (fwd: H x W, bwd: Ho x Wo)
  int in_pitch;         // row pitch of the input planes, elements
  int64_t in_plane;     // elements between consecutive planes of one input array
  int out_h, out_w;     // output extent (fwd: Ho x Wo, bwd: H x W)
  int off;              // in row = out row + a - off (same for columns)
  int strips;           // ceil(out_w / kStripOut)
  int64_t cols;         // strip-columns: planes * strips
  int parts;            // > 1: workgroups per strip-column (each takes a row range)
  int per_block;        // parts == 1: whole strip-columns per workgroup
  // images (fwd: the inputs; bwd: read by the chain rule)
  const float* x;
  const float* y;
  int64_t img_plane;    // H * W
  int img_w;            // W
  // maps (fwd: written in training mode; bwd: the blurred input)
  float* maps;
  int map_pitch;        // roundup(Wo, 4)
  int64_t map_plane;    // Ho * map_pitch floats per map plane
  // forward
  float k_m2;           // -2 / M
  double inv_m;         // 1 / M
  float* loss;
  Workspace* ws;
  // backward
  const float* dloss;
  float* gx;
  float* gy;
};

// ---------------------------------------------------------------------------
// Memory access through buffer descriptors
//
// Every global load and store goes through a raw buffer descriptor covering
// exactly one plane.  The hardware range-checks each access against the
// descriptor's size: an out-of-range load returns 0 and an out-of-range store
// is dropped.  Zero padding, the ragged right edge, rows above or below a
// plane and idle lanes are all expressed as out-of-range offsets (a negative
// row offset wraps to a large unsigned value; an invalid column uses the
// 2^31 marker), so the hot loop has no branches around memory operations and
// the compiler can keep loads in flight across the stores of a batch.
// Planes are limited to 2^27 elements so that every valid byte offset, and
// every marked one, stays on its side of 2^31.

using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr unsigned kOob = 0x80000000u;         // offset that is out of range for every plane
constexpr int kRsrcFlags = 0x00020000;          // gfx9 dword3: 32-bit data format, raw access

__device__ __forceinline__ rsrc_t make_rsrc(const float* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, (int)bytes, kRsrcFlags);
}
__device__ __forceinline__ float ld1(rsrc_t r, unsigned off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ float4 ld4(rsrc_t r, unsigned off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// Stores take a cache policy: kNt marks them non-temporal (streaming), for
// launches whose data cannot stay in the last-level cache anyway.
constexpr int kPolicyNt = 2;  // gfx950 cache-policy bit: non-temporal
template <bool kNt>
__device__ __forceinline__ void st1(rsrc_t r, unsigned off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, off, 0, kNt ? kPolicyNt : 0);
}
template <bool kNt>
__device__ __forceinline__ void st4(rsrc_t r, unsigned off, float4 v) {
  using u4 = unsigned __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, off, 0, kNt ? kPolicyNt : 0);
}

// ---------------------------------------------------------------------------
// SSIM at one map position

// The SSIM terms at one map position, from the blurred quantities
// mu_x', mu_y', R = B((x-y)^2), P' = B(x' y').
struct SsimTerms {
  float mux, muy, dm, a1, d1, b1, a2, d2, b2, inv;
};

__device__ __forceinline__ SsimTerms ssim_terms(float mxs, float mys, float rr, float pp) {
  SsimTerms t;
  t.mux = mxs + kShift;
  t.muy = mys + kShift;
  t.dm = mxs - mys;
  t.a1 = __builtin_fmaf(2.0f * t.mux, t.muy, kC1);
  t.d1 = t.dm * t.dm;
  t.b1 = t.a1 + t.d1;
  const float cov = __builtin_fmaf(-mxs, mys, pp);
  t.a2 = __builtin_fmaf(2.0f, cov, kC2);
  t.d2 = __builtin_fmaf(-t.dm, t.dm, rr);
  t.b2 = t.a2 + t.d2;
  t.inv = __builtin_amdgcn_rcpf(t.b1 * t.b2);
  return t;
}

// 1 - S = (A1 D2 + D1 B2) / (B1 B2)
__device__ __forceinline__ float one_minus_ssim(const SsimTerms& t) {
  return __builtin_fmaf(t.a1, t.d2, t.d1 * t.b2) * t.inv;
}

// The four loss partials at one map position (k_m2 = -2/M).  With
// S = A1 A2 inv, inv = 1/(B1 B2), and every term a multiple of D1, D2 or dmu
// (so all vanish when x = y):
//   dS/dmu_x' = 2 inv (mu_y T1 - mu_y' T2 + T3)
//   dS/dmu_y' = 2 inv (mu_x T1 - mu_x' T2 - T3)
//   dS/dP'    = 2 inv T2,      dS/dR = -S / B2 = -S B1 inv
// where T1 = A2 D1 / B1, T2 = A1 D2 / B2, T3 = S (B1 - B2) dmu.
// Maps (loss = mean of 1 - S over M entries, k = -(2/M) inv):
//   m0 = -(1/M) dS/dmu_x' = k (mu_y T1 - mu_y' T2 + T3)
//   m1 = -(1/M) dS/dmu_y' = k (mu_x T1 - mu_x' T2 - T3)
//   m2 = -(2/M) dS/dR     = -k S B1   (the chain rule's 2 folded in)
//   m3 = -(1/M) dS/dP'    = k T2
__device__ __forceinline__ void loss_partials(float mxs, float mys, const SsimTerms& t, float k_m2,
                                              float (&m)[4]) {
  const float s = t.a1 * t.a2 * t.inv;
  const float ib1 = t.b2 * t.inv;
  const float ib2 = t.b1 * t.inv;
  const float t1 = t.a2 * t.d1 * ib1;
  const float t2 = t.a1 * t.d2 * ib2;
  const float t3 = s * (t.b1 - t.b2) * t.dm;
  const float k = k_m2 * t.inv;
  m[0] = k * __builtin_fmaf(t.muy, t1, __builtin_fmaf(-mys, t2, t3));
  m[1] = k * __builtin_fmaf(t.mux, t1, __builtin_fmaf(-mxs, t2, -t3));
  m[2] = -(k * s) * t.b1;
  m[3] = k * t2;
}

// ---------------------------------------------------------------------------
// Per-segment context: one (plane, strip) and a run of its output rows

template <int MODE>
struct Seg {
  static constexpr int kIn = (MODE == kBwd) ? 4 : 2;
  rsrc_t in[kIn];       // fwd: x, y planes; bwd: the 4 map planes
  rsrc_t img[2];        // bwd: x, y planes (chain rule)
  rsrc_t out[4];        // fwd-train: the 4 map planes; bwd: grad_x, grad_y planes
  unsigned colbyte;     // this lane's input column in bytes, or kOob
  unsigned in_row;      // input row pitch, bytes
  unsigned out_row;     // output row pitch, bytes
  unsigned out_elem;    // bytes per output element (4)
  int r0;               // input row held by ring slot 0 (first output row - off)
  int row0, nrows;      // output rows [row0, row0 + nrows)
  int j0;               // first output column of the strip
};

template <int MODE>
struct Raw {
  float v[4];  // fwd: x, y; bwd: the four blurred quantities of a map entry
  bool in;     // the element lies inside the input extent
};

// This lane's input pixel(s) in input row r; 0 outside the input extent.
template <int MODE>
__device__ __forceinline__ void load_row(const Params& p, const Seg<MODE>& s, int r,
                                         Raw<MODE>& out) {
  const unsigned off = s.colbyte + (unsigned)r * s.in_row;
  if constexpr (MODE == kBwd) {
#pragma unroll
    for (int k = 0; k < 4; ++k) out.v[k] = ld1(s.in[k], off);
  } else {
    out.v[0] = ld1(s.in[0], off);
    out.v[1] = ld1(s.in[1], off);
  }
  out.in = (s.colbyte != kOob) && ((unsigned)r < (unsigned)p.in_h);
}

// Quantities blurred by the forward: x', y', (x - y)^2 and x' y' with
// x' = x - 1/2, y' = y - 1/2.  Quantities blurred by the backward: the four
// loss partials at each map entry, formed from the saved blurred quantities.
template <int MODE>
__device__ __forceinline__ void quantities(const Raw<MODE>& r, float k_m2, float (&q)[kQ]) {
  if constexpr (MODE == kBwd) {
    // the loss partials at this map entry; zero outside the map (the
    // adjoint's zero fill)
    float m[4];
    loss_partials(r.v[0], r.v[1], ssim_terms(r.v[0], r.v[1], r.v[2], r.v[3]), k_m2, m);
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = r.in ? m[k] : 0.0f;
  } else {
    (void)k_m2;
    const float x = r.v[0] - kShift, y = r.v[1] - kShift;
    const float d = r.v[0] - r.v[1];
    q[0] = x;
    q[1] = y;
    q[2] = d * d;
    q[3] = x * y;
  }
}

// ---------------------------------------------------------------------------
// Consumers (4 adjacent outputs of one row)

// Where this lane's output group lives: byte offset of its first output in
// the output planes, or kOob when the group is not real (row outside the
// segment, lane outside the strip, first column outside the output extent).
// The images read by the backward's chain rule are loaded here, at the start
// of a batch, so that their latency hides behind the batch's blur work.
template <int MODE, bool kVec>
struct Group {
  bool ok;
  int j;
  unsigned base;
  unsigned off[4];  // per-output offsets (kOob past the output extent)
  float xv[4], yv[4];
};

template <int MODE, bool kVec>
__device__ __forceinline__ void group_begin(const Params& p, const Seg<MODE>& s, int ri, int lane,
                                            Group<MODE, kVec>& g) {
  g.j = s.j0 + 4 * lane;
  g.ok = (ri < s.nrows) && (lane < kRowLanes) && (g.j < p.out_w);
  g.base = g.ok ? (unsigned)(s.row0 + ri) * s.out_row + (unsigned)g.j * s.out_elem : kOob;
#pragma unroll
  for (int t = 0; t < 4; ++t)
    g.off[t] = (g.ok && (g.j + t) < p.out_w) ? g.base + s.out_elem * t : kOob;
  if constexpr (MODE == kBwd) {
    if constexpr (kVec) {
      const float4 a = ld4(s.img[0], g.base);
      const float4 b = ld4(s.img[1], g.base);
      g.xv[0] = a.x; g.xv[1] = a.y; g.xv[2] = a.z; g.xv[3] = a.w;
      g.yv[0] = b.x; g.yv[1] = b.y; g.yv[2] = b.z; g.yv[3] = b.w;
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        g.xv[t] = ld1(s.img[0], g.off[t]);
        g.yv[t] = ld1(s.img[1], g.off[t]);
      }
    }
  }
}

template <int MODE, bool kVec, bool kNt>
__device__ __forceinline__ void consume(const Params& p, const Seg<MODE>& s,
                                        const Group<MODE, kVec>& g, const float (&o)[kQ][4],
                                        float dl, double& acc) {
  if constexpr (MODE != kBwd) {
    float s4 = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float ell = one_minus_ssim(ssim_terms(o[0][t], o[1][t], o[2][t], o[3][t]));
      s4 += (g.ok && (g.j + t) < p.out_w) ? ell : 0.0f;
    }
    acc += (double)s4;
    if constexpr (MODE == kFwdTrain) {
      // training: save the four blurred quantities, one map plane each (a
      // lane's 4 outputs are 16 contiguous bytes of a plane, so a wave writes
      // 1 KiB per plane per instruction); the backward forms the loss
      // partials from them as it reads them.  j is a multiple of 4 and the
      // pitch rounds Wo up to one, so the whole group lies inside the padded
      // row (entries past Wo land in the padding, which nothing reads).
#pragma unroll
      for (int q = 0; q < 4; ++q) st4<kNt>(s.out[q], g.base, make_float4(o[q][0], o[q][1], o[q][2], o[q][3]));
    }
  } else {
    float g1[4], g2[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // chain rule: d mu_x'/dx = B^T, d P'/dx = y' B^T, d R/dx = 2 (x - y) B^T
      const float xs = g.xv[t] - kShift, ys = g.yv[t] - kShift, d = g.xv[t] - g.yv[t];
      g1[t] = dl * __builtin_fmaf(d, o[2][t], __builtin_fmaf(ys, o[3][t], o[0][t]));
      g2[t] = dl * __builtin_fmaf(-d, o[2][t], __builtin_fmaf(xs, o[3][t], o[1][t]));
    }
    // a gradient the caller does not want has a zero-size descriptor: its
    // stores are dropped without a branch
    if constexpr (kVec) {
      st4<kNt>(s.out[0], g.base, make_float4(g1[0], g1[1], g1[2], g1[3]));
      st4<kNt>(s.out[1], g.base, make_float4(g2[0], g2[1], g2[2], g2[3]));
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        st1<kNt>(s.out[0], g.off[t], g1[t]);
        st1<kNt>(s.out[1], g.off[t], g2[t]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// One batch of kRows rows: column pass into the ring and the LDS tile, then
// the row pass and the consumer.  PH = batch index mod 3 fixes the ring slots
// at compile time.

template <int MODE, bool kVec, bool kNt, int PH>
__device__ __forceinline__ void batch(const Params& p, const Seg<MODE>& s,
                                      float (&tile)[2][kQ][kRows][kTileW],
                                      float (&ring)[kRing][kQ], Raw<MODE> (&pre)[kRows], int t,
                                      int buf, float dl, double& acc) {
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;

  Group<MODE, kVec> g;
  group_begin<MODE, kVec>(p, s, 4 * t + wave, lane, g);

  Raw<MODE> cur[kRows];
#pragma unroll
  for (int m = 0; m < kRows; ++m) cur[m] = pre[m];
  // prefetch the next batch (rows past the segment are harmless: in range
  // they are real pixels, out of range they read as 0)
#pragma unroll
  for (int m = 0; m < kRows; ++m) load_row<MODE>(p, s, s.r0 + 10 + 4 * (t + 1) + m, pre[m]);

  // column pass
#pragma unroll
  for (int m = 0; m < kRows; ++m) {
    const int base = 4 * PH + m;  // compile-time after unrolling
    quantities<MODE>(cur[m], p.k_m2, ring[(base + 10) % kRing]);
    float cs[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) cs[q] = tap(0) * ring[base % kRing][q];
#pragma unroll
    for (int a = 1; a < 11; ++a)
#pragma unroll
      for (int q = 0; q < kQ; ++q) cs[q] = __builtin_fmaf(tap(a), ring[(base + a) % kRing][q], cs[q]);
#pragma unroll
    for (int q = 0; q < kQ; ++q) tile[buf][q][m][tid] = cs[q];
  }
  __syncthreads();

  // row pass: wave w -> batch row w; lane l -> outputs 4l .. 4l+3.  Lanes
  // past the strip read the last real group and store out of range.
  const int lr = lane < kRowLanes ? lane : kRowLanes - 1;
  float o[kQ][4];  // [quantity][output]: the 4 outputs of a map plane are one register quad
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const float* src = &tile[buf][q][wave][4 * lr];
    float v[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 f = *reinterpret_cast<const float4*>(src + 4 * k);
      v[4 * k + 0] = f.x;
      v[4 * k + 1] = f.y;
      v[4 * k + 2] = f.z;
      v[4 * k + 3] = f.w;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float a = tap(0) * v[u];
#pragma unroll
      for (int b = 1; b < 11; ++b) a = __builtin_fmaf(tap(b), v[u + b], a);
      o[q][u] = a;
    }
  }
  consume<MODE, kVec, kNt>(p, s, g, o, dl, acc);
}

template <int MODE, bool kVec, bool kNt>
__device__ __forceinline__ void strip_body(const Params& p) {
  __shared__ float tile[2][kQ][kRows][kTileW];
  __shared__ double red[kWaves];
  __shared__ int is_last;

  const int tid = threadIdx.x;
  const int G = gridDim.x;
  // XCD-aware order: hardware hands consecutive workgroup ids to the 8 XCDs
  // in turn; give each XCD one contiguous eighth of the work.
  int lb = blockIdx.x;
  if ((G & 7) == 0) lb = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  // This workgroup's share: one row range of one strip-column, or a run of
  // whole strip-columns.  Every workgroup gets the same amount of work, so
  // the grid (one resident wave of workgroups) finishes together.
  int64_t sc_begin, sc_end;
  int row_begin, row_end;
  if (p.parts > 1) {
    sc_begin = lb / p.parts;
    sc_end = sc_begin + 1;
    const int part = lb - (int)sc_begin * p.parts;
    row_begin = (int)((int64_t)part * p.out_h / p.parts);
    row_end = (int)((int64_t)(part + 1) * p.out_h / p.parts);
  } else {
    sc_begin = (int64_t)lb * p.per_block;
    sc_end = sc_begin + p.per_block < p.cols ? sc_begin + p.per_block : p.cols;
    row_begin = 0;
    row_end = p.out_h;
  }

  float dl = 0.0f;
  if constexpr (MODE == kBwd) dl = *p.dloss;

  double acc = 0.0;
  int buf = 0;
  for (int64_t sc = sc_begin; sc < sc_end; ++sc) {
    Seg<MODE> s;
    const int64_t plane = sc / p.strips;
    const int strip = (int)(sc - plane * p.strips);
    s.row0 = row_begin;
    s.nrows = row_end - row_begin;
    s.j0 = strip * kStripOut;
    const int c = s.j0 - p.off + tid;  // this lane's input column
    s.colbyte = (c >= 0 && c < p.in_w) ? (unsigned)c * 4u : kOob;
    s.in_row = (unsigned)p.in_pitch * 4u;
    s.r0 = s.row0 - p.off;
    if constexpr (MODE == kBwd) {
      const float* mp = p.maps + plane * 4 * p.map_plane;
#pragma unroll
      for (int k = 0; k < 4; ++k) s.in[k] = make_rsrc(mp + k * p.map_plane, p.map_plane * 4);
      s.img[0] = make_rsrc(p.x + plane * p.img_plane, p.img_plane * 4);
      s.img[1] = make_rsrc(p.y + plane * p.img_plane, p.img_plane * 4);
      s.out[0] = make_rsrc(p.gx ? p.gx + plane * p.img_plane : p.x, p.gx ? p.img_plane * 4 : 0);
      s.out[1] = make_rsrc(p.gy ? p.gy + plane * p.img_plane : p.y, p.gy ? p.img_plane * 4 : 0);
      s.out_row = (unsigned)p.img_w * 4u;
      s.out_elem = 4u;
    } else {
      s.in[0] = make_rsrc(p.x + plane * p.in_plane, p.in_plane * 4);
      s.in[1] = make_rsrc(p.y + plane * p.in_plane, p.in_plane * 4);
      if constexpr (MODE == kFwdTrain) {
        const float* mp = p.maps + plane * 4 * p.map_plane;
#pragma unroll
        for (int k = 0; k < 4; ++k) s.out[k] = make_rsrc(mp + k * p.map_plane, p.map_plane * 4);
      }
      s.out_row = (unsigned)p.map_pitch * 4u;
      s.out_elem = 4u;
    }
    const int nb = (s.nrows + kRows - 1) / kRows;

    float ring[kRing][kQ];
    Raw<MODE> warm[10];
    Raw<MODE> pre[kRows];
#pragma unroll
    for (int k = 0; k < 10; ++k) load_row<MODE>(p, s, s.r0 + k, warm[k]);
#pragma unroll
    for (int m = 0; m < kRows; ++m) load_row<MODE>(p, s, s.r0 + 10 + m, pre[m]);
#pragma unroll
    for (int k = 0; k < 10; ++k) quantities<MODE>(warm[k], p.k_m2, ring[k]);

    for (int t = 0;;) {
      if (t >= nb) break;
      batch<MODE, kVec, kNt, 0>(p, s, tile, ring, pre, t, buf, dl, acc);
      buf ^= 1;
      if (++t >= nb) break;
      batch<MODE, kVec, kNt, 1>(p, s, tile, ring, pre, t, buf, dl, acc);
      buf ^= 1;
      if (++t >= nb) break;
      batch<MODE, kVec, kNt, 2>(p, s, tile, ring, pre, t, buf, dl, acc);
      buf ^= 1;
      ++t;
    }
  }

  if constexpr (MODE != kBwd) {
    // workgroup sum of the map of 1 - S, then the last workgroup finishes the mean
    const int wave = tid / kWave, lane = tid % kWave;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
    if (lane == 0) red[wave] = acc;
    __syncthreads();
    if (tid == 0) {
      double bs = 0.0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) bs += red[w];
      // Publish the partial with a device-coherent atomic store and wait for
      // its acknowledgement before taking the ticket: a release of exactly
      // this one value.  (A release fence would also write back every dirty
      // line of this XCD's L2 -- megabytes of map stores -- in every
      // workgroup.)
      __hip_atomic_store(&p.ws->partial[blockIdx.x], bs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
      const unsigned prev =
          __hip_atomic_fetch_add(&p.ws->ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      is_last = (prev == (unsigned)(G - 1));
    }
    __syncthreads();
    if (is_last && wave == 0) {
      double sum = 0.0;
      for (int k = lane; k < G; k += kWave)
        sum += __hip_atomic_load(&p.ws->partial[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) sum += __shfl_xor(sum, o, kWave);
      if (lane == 0) {
        *p.loss = (float)(sum * p.inv_m);
        __hip_atomic_store(&p.ws->ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// Entry kernels (one per direction, mode and store policy; named for
// profiles).  "stream" kernels mark their stores non-temporal.
__global__ __launch_bounds__(kThreads) void ssim_fwd_infer_kernel(const Params p) {
  strip_body<kFwdInfer, false, false>(p);
}
__global__ __launch_bounds__(kThreads) void ssim_fwd_train_kernel(const Params p) {
  strip_body<kFwdTrain, false, false>(p);
}
__global__ __launch_bounds__(kThreads) void ssim_fwd_train_stream_kernel(const Params p) {
  strip_body<kFwdTrain, false, true>(p);
}
__global__ __launch_bounds__(kThreads) void ssim_bwd_kernel(const Params p) {
  strip_body<kBwd, true, false>(p);
}
__global__ __launch_bounds__(kThreads) void ssim_bwd_stream_kernel(const Params p) {
  strip_body<kBwd, true, true>(p);
}
__global__ __launch_bounds__(kThreads) void ssim_bwd_unaligned_kernel(const Params p) {
  strip_body<kBwd, false, false>(p);
}

// ---------------------------------------------------------------------------
// Host side

enum KernelId { kKFwdInfer, kKFwdTrain, kKFwdTrainStream, kKBwd, kKBwdStream, kKBwdUnaligned, kKernels };
const void* const kKernelTable[kKernels] = {
    (const void*)ssim_fwd_infer_kernel, (const void*)ssim_fwd_train_kernel,
    (const void*)ssim_fwd_train_stream_kernel, (const void*)ssim_bwd_kernel,
    (const void*)ssim_bwd_stream_kernel, (const void*)ssim_bwd_unaligned_kernel};

// Bytes a training step touches in HBM (both images, the saved maps, both
// gradients).  Above this the step cannot stay in the 256 MB last-level
// cache between the forward and the backward, and the stores stream
// (non-temporal); below it they stay cacheable so that the backward finds
// the maps there.
constexpr size_t kStreamBytes = (size_t)256 << 20;

struct DeviceInfo {
  bool ready = false;
  int status = SSIM_OK;
  int cus = 0;
  int occ[kKernels] = {};  // resident workgroups per CU, per entry kernel
};

constexpr int kMaxDevices = 64;
std::mutex g_mu;
DeviceInfo g_dev[kMaxDevices];

int device_info(const DeviceInfo** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SSIM_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SSIM_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.ready) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SSIM_ERR_HIP;
    if (prop.warpSize != kWave || strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
      d.status = SSIM_ERR_DEVICE;
    } else {
      d.cus = prop.multiProcessorCount;
      for (int k = 0; k < kKernels; ++k) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kKernelTable[k], kThreads, 0) != hipSuccess)
          return SSIM_ERR_HIP;
        d.occ[k] = n > 0 ? n : 1;
      }
      d.status = SSIM_OK;
    }
    d.ready = true;
  }
  *out = &d;
  return d.status;
}

int64_t roundup4(int64_t v) { return (v + 3) & ~(int64_t)3; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return pa < pb + nb && pb < pa + na;
}

struct Shape {
  int64_t N, C, H, W, Ho, Wo, pitch, planes;
  size_t img_bytes, map_bytes;
};

int check_shape(int64_t N, int64_t C, int64_t H, int64_t W, int padding, Shape* s) {
  if (padding != SSIM_PAD_VALID && padding != SSIM_PAD_SAME) return SSIM_ERR_PADDING;
  if (N <= 0 || C <= 0 || H <= 0 || W <= 0) return SSIM_ERR_SHAPE;
  const int64_t Ho = padding == SSIM_PAD_VALID ? H - 10 : H;
  const int64_t Wo = padding == SSIM_PAD_VALID ? W - 10 : W;
  if (Ho <= 0 || Wo <= 0) return SSIM_ERR_SHAPE;
  // Buffer offsets are 32-bit: a plane (image, or map with its row pitch)
  // holds at most 2^27 elements and a row at most 2^20, so valid offsets
  // stay below 2^29 and the out-of-range ones (rows above the plane wrap to
  // just below 2^32; the 2^31 marker plus at most 14 rows of 4 MiB) stay
  // above 2^30.
  const int64_t lim = (int64_t)1 << 27;
  if (W > ((int64_t)1 << 20) || H > lim / W) return SSIM_ERR_OVERFLOW;
  const int64_t pitch = roundup4(Wo);
  if (H * W > lim || Ho * pitch > lim) return SSIM_ERR_OVERFLOW;
  if (N > (int64_t)1 << 40 || C > ((int64_t)1 << 40) / N) return SSIM_ERR_OVERFLOW;
  const int64_t planes = N * C;
  // bytes must fit comfortably in 64 bits
  if (planes > ((int64_t)1 << 58) / (H * W) || planes > ((int64_t)1 << 56) / (Ho * pitch))
    return SSIM_ERR_OVERFLOW;
  s->N = N; s->C = C; s->H = H; s->W = W; s->Ho = Ho; s->Wo = Wo; s->pitch = pitch;
  s->planes = planes;
  s->img_bytes = (size_t)(planes * H * W) * sizeof(float);
  s->map_bytes = (size_t)(planes * Ho * pitch) * 4 * sizeof(float);
  return SSIM_OK;
}

// Grid: one resident wave of workgroups (CUs x occupancy), or fewer when
// the work is small.  With fewer strip-columns than resident workgroups,
// each strip-column is split into `parts` equal row ranges of at least
// kMinRowsPerBlock rows; otherwise each workgroup takes `per_block` whole
// strip-columns.
int plan_grid(const DeviceInfo* d, int which, Params& p) {
  int64_t resident = (int64_t)d->cus * d->occ[which];
  if (resident > kMaxBlocks) resident = kMaxBlocks;
  if (p.cols >= resident) {
    p.parts = 1;
    p.per_block = (int)((p.cols + resident - 1) / resident);
    return (int)((p.cols + p.per_block - 1) / p.per_block);
  }
  int64_t parts = resident / p.cols;
  const int64_t max_parts = (p.out_h + kMinRowsPerBlock - 1) / kMinRowsPerBlock;
  if (parts > max_parts) parts = max_parts;
  if (parts < 1) parts = 1;
  p.parts = (int)parts;
  p.per_block = 1;
  return (int)(p.cols * parts);
}

void fill_geometry(Params& p, int in_h, int in_w, int in_pitch, int64_t in_plane, int out_h,
                   int out_w, int off, int64_t planes) {
  p.in_h = in_h;
  p.in_w = in_w;
  p.in_pitch = in_pitch;
  p.in_plane = in_plane;
  p.out_h = out_h;
  p.out_w = out_w;
  p.off = off;
  p.strips = (out_w + kStripOut - 1) / kStripOut;
  p.cols = planes * p.strips;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI

extern "C" {

int ssim_abi_version(void) { return SSIM_ABI_VERSION; }

const char* ssim_strerror(int code) {
  switch (code) {
    case SSIM_OK: return "success";
    case SSIM_ERR_NULL: return "a required pointer is NULL";
    case SSIM_ERR_SHAPE: return "bad shape: N, C, H, W must be positive and valid padding needs H, W >= 11";
    case SSIM_ERR_PADDING: return "padding must be SSIM_PAD_VALID (0) or SSIM_PAD_SAME (1)";
    case SSIM_ERR_OVERFLOW: return "a plane holds more than 2^27 elements, a row more than 2^20, or a size overflows";
    case SSIM_ERR_ALIAS: return "an output buffer overlaps an input or another output";
    case SSIM_ERR_HIP: return "a HIP runtime call failed";
    case SSIM_ERR_DEVICE: return "the current device is not a wave64 gfx950 GPU";
    default: return "unknown error code";
  }
}

void ssim_taps(float out[11]) {
  for (int k = 0; k < 11; ++k) out[k] = tap(k);
}

int ssim_map_shape(int64_t H, int64_t W, int padding, int64_t* Ho, int64_t* Wo) {
  if (!Ho || !Wo) return SSIM_ERR_NULL;
  Shape s;
  const int rc = check_shape(1, 1, H, W, padding, &s);
  if (rc != SSIM_OK) return rc;
  *Ho = s.Ho;
  *Wo = s.Wo;
  return SSIM_OK;
}

size_t ssim_saved_maps_bytes(int64_t N, int64_t C, int64_t H, int64_t W, int padding) {
  Shape s;
  if (check_shape(N, C, H, W, padding, &s) != SSIM_OK) return 0;
  return s.map_bytes;
}

size_t ssim_workspace_bytes(void) { return sizeof(Workspace); }

int ssim_forward(const float* img1, const float* img2, int64_t N, int64_t C, int64_t H,
                 int64_t W, int padding, float* loss, float* saved_maps, void* workspace,
                 void* stream) {
  if (!img1 || !img2 || !loss || !workspace) return SSIM_ERR_NULL;
  Shape s;
  int rc = check_shape(N, C, H, W, padding, &s);
  if (rc != SSIM_OK) return rc;
  if (saved_maps && ((uintptr_t)saved_maps & 15u)) return SSIM_ERR_SHAPE;
  const size_t wsb = sizeof(Workspace);
  const void* outs[3] = {loss, saved_maps, workspace};
  const size_t outb[3] = {sizeof(float), saved_maps ? s.map_bytes : 0, wsb};
  for (int k = 0; k < 3; ++k) {
    if (overlaps(outs[k], outb[k], img1, s.img_bytes) || overlaps(outs[k], outb[k], img2, s.img_bytes))
      return SSIM_ERR_ALIAS;
    for (int l = k + 1; l < 3; ++l)
      if (overlaps(outs[k], outb[k], outs[l], outb[l])) return SSIM_ERR_ALIAS;
  }

  const DeviceInfo* d = nullptr;
  rc = device_info(&d);
  if (rc != SSIM_OK) return rc;

  Params p;
  memset(&p, 0, sizeof(p));
  const int off = padding == SSIM_PAD_VALID ? 0 : 5;
  fill_geometry(p, (int)s.H, (int)s.W, (int)s.W, s.H * s.W, (int)s.Ho, (int)s.Wo, off, s.planes);
  p.x = img1;
  p.y = img2;
  p.img_plane = s.H * s.W;
  p.img_w = (int)s.W;
  p.maps = saved_maps;
  p.map_pitch = (int)s.pitch;
  p.map_plane = s.Ho * s.pitch;
  const double M = (double)s.planes * (double)s.Ho * (double)s.Wo;
  p.k_m2 = (float)(-2.0 / M);
  p.inv_m = 1.0 / M;
  p.loss = loss;
  p.ws = static_cast<Workspace*>(workspace);

  const bool stream_st = 4 * s.img_bytes + s.map_bytes > kStreamBytes;
  const int which = !saved_maps ? kKFwdInfer : stream_st ? kKFwdTrainStream : kKFwdTrain;
  const int G = plan_grid(d, which, p);
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* args[] = {&p};
  if (hipLaunchKernel(kKernelTable[which], dim3(G), dim3(kThreads), args, 0, st) != hipSuccess)
    return SSIM_ERR_HIP;
  return hipGetLastError() == hipSuccess ? SSIM_OK : SSIM_ERR_HIP;
}

int ssim_backward(const float* dloss, const float* img1, const float* img2, int64_t N,
                  int64_t C, int64_t H, int64_t W, int padding, const float* saved_maps,
                  float* grad_img1, float* grad_img2, void* stream) {
  if (!dloss || !img1 || !img2 || !saved_maps) return SSIM_ERR_NULL;
  Shape s;
  int rc = check_shape(N, C, H, W, padding, &s);
  if (rc != SSIM_OK) return rc;
  if ((uintptr_t)saved_maps & 15u) return SSIM_ERR_SHAPE;
  const void* ins[4] = {dloss, img1, img2, saved_maps};
  const size_t inb[4] = {sizeof(float), s.img_bytes, s.img_bytes, s.map_bytes};
  float* outs[2] = {grad_img1, grad_img2};
  for (int k = 0; k < 2; ++k)
    for (int l = 0; l < 4; ++l)
      if (overlaps(outs[k], s.img_bytes, ins[l], inb[l])) return SSIM_ERR_ALIAS;
  if (overlaps(grad_img1, s.img_bytes, grad_img2, s.img_bytes)) return SSIM_ERR_ALIAS;
  if (!grad_img1 && !grad_img2) return SSIM_OK;

  const DeviceInfo* d = nullptr;
  rc = device_info(&d);
  if (rc != SSIM_OK) return rc;

  Params p;
  memset(&p, 0, sizeof(p));
  const int off = padding == SSIM_PAD_VALID ? 10 : 5;
  fill_geometry(p, (int)s.Ho, (int)s.Wo, (int)s.pitch, s.Ho * s.pitch * 4, (int)s.H, (int)s.W,
                off, s.planes);
  p.x = img1;
  p.y = img2;
  p.img_plane = s.H * s.W;
  p.img_w = (int)s.W;
  p.maps = const_cast<float*>(saved_maps);
  p.map_pitch = (int)s.pitch;
  p.map_plane = s.Ho * s.pitch;
  p.dloss = dloss;
  p.gx = grad_img1;
  p.gy = grad_img2;
  p.k_m2 = (float)(-2.0 / ((double)s.planes * (double)s.Ho * (double)s.Wo));

  const bool vec = (s.W % 4 == 0) && ((uintptr_t)img1 % 16 == 0) && ((uintptr_t)img2 % 16 == 0) &&
                   ((uintptr_t)grad_img1 % 16 == 0) && ((uintptr_t)grad_img2 % 16 == 0);
  const bool stream_st = 4 * s.img_bytes + s.map_bytes > kStreamBytes;
  const int which = !vec ? kKBwdUnaligned : stream_st ? kKBwdStream : kKBwd;
  const int G = plan_grid(d, which, p);
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* args[] = {&p};
  if (hipLaunchKernel(kKernelTable[which], dim3(G), dim3(kThreads), args, 0, st) != hipSuccess)
    return SSIM_ERR_HIP;
  return hipGetLastError() == hipSuccess ? SSIM_OK : SSIM_ERR_HIP;
}

}  // extern "C"
