// ssim_fused.hpp -- the recomputing kernels: image -> blurred statistics ->
// loss partials -> adjoint blur -> gradients in one pass over the images,
// with no map written to or read from memory.
//
// The gradient is the one of "TriSSIM", How it works (the adjoint B^T of the
// blur applied to the loss partials, then the chain rule), in the basis of
// ssim_device.hpp.  Instead of saving the blurred statistics in the forward
// and reading them back, one kernel forms them again from the images and
// keeps every intermediate on chip: per step it moves the images and the
// gradients only (and, with the loss, that is the whole training step).
//
// Two stencil stages run in one strip of 256 lanes:
//   stage 1 : lane t owns image column v0 - 10 + t (v0: the strip's first
//             gradient column); the column pass of the four quantities runs
//             through a 12-slot register ring, the row pass through the LDS
//             tile, as in the two-kernel design.  Each
//             row-pass lane forms the SSIM terms and the four loss partials
//             at 4 adjacent map entries and writes the partials back into the
//             same tile row it read (zero outside the map: the adjoint's zero
//             fill).  246 map columns feed the strip's gradients.
//   stage 2 : lane t owns map column v0 - off2 + t; it reads its column of
//             the partials from the tile, runs the adjoint's column pass
//             through a second register ring, writes the result back into
//             the same column, and the row pass gives 4 adjacent gradient
//             entries per lane: 236 gradient columns per strip.
// Strips run over the N*C planes laid side by side, each followed by a gap
// of zero columns (Params::vpitch): a strip may end in one plane and go on
// into the next, so planes whose width is not a multiple of 236 share their
// last strips instead of each paying a mostly empty one.
// Row pipeline: image row r enters stage 1; it completes map row
// r + off - 10, whose partials complete gradient row r - 10 in stage 2.  A
// row range of n gradient rows therefore reads n + 20 image rows, each once:
// stage 1 also keeps the rows it loads in an LDS ring, from which stage 2
// takes x and y for the chain rule.  Map entries shared by two strips or two
// row ranges are computed by both, and the loss counts each exactly once, in
// the strip and range that own it.
//
// The tile is double-buffered per batch of 4 rows; within a batch it holds,
// in turn, the column-blurred quantities, the partials (written over the row
// each wave read) and the adjoint's column pass (written over the column
// each lane read), with a barrier between the phases.

#pragma once

#include "ssim_device.hpp"

namespace ssim_dev {

constexpr int kFOut = 236;                          // gradient columns per strip
constexpr int kFMapCols = kFOut + 10;               // map columns they need
constexpr int kFMapLanes = (kFMapCols + 3) / 4;     // stage-1 row-pass lanes (62)
constexpr int kFGradLanes = kFOut / 4;              // stage-2 row-pass lanes (59)
constexpr int kFTileW = kTileW + 4;                 // 256 lanes + the last lane's 4-column overhang
constexpr int kFThreads = 2 * kThreads;             // two groups of 4 waves, one per stage
constexpr int kFWaves = kFThreads / kWave;
// Rows of x and y kept in LDS between the two stages: stage 2 needs image
// row r for the chain rule 14 to 17 rows after stage 1 loaded it, and stage 1
// writes 4 new rows per tick, so 20 slots hold every row until its last use
// and are never written in the tick that reads them.
constexpr int kXYRing = 20;
constexpr int kXYOff = 2;  // column t at index t + 2: stage 2's 4-column groups start 16-byte aligned

static_assert(kFMapCols + 10 == kTileW, "a strip's image columns are one per lane");
static_assert(4 * (kFMapLanes - 1) + 16 <= kFTileW, "stage-1 row-pass reads stay in the tile row");
static_assert(4 * (kFGradLanes - 1) + 16 <= 4 * kFMapLanes,
              "stage-2 row-pass reads stay in the columns stage 1 wrote");
static_assert(kFOut % 4 == 0 && (kFTileW * 4) % 16 == 0, "16-byte aligned tile rows and groups");
static_assert(kXYOff + kTileW <= kFTileW && (kXYOff + 10) % 4 == 0,
              "the row ring holds a strip row; gradient groups read it 16-byte aligned");
static_assert(kXYRing % kRows == 0 && kXYRing >= 18, "ring depth covers the stage-1 to stage-2 lag");

struct FSeg {
  rsrc_t img[2];        // x, y from plane p0 on (at most two planes)
  rsrc_t out[2];        // grad_x, grad_y from plane p0 (zero-size when not wanted)
  unsigned colbyte;     // this lane's image column (stage 1): byte offset from plane p0, or kOob
  unsigned row_bytes;   // image row pitch, bytes
  unsigned plane_bytes; // image plane, bytes
  int img_h;            // image rows
  int u0, nrows;        // gradient rows [u0, u0 + nrows)
  int rv0;              // first gradient column of the strip, relative to plane p0's column 0
  bool p1;              // plane p0 + 1 exists
  bool last;            // the last strip: it owns the map columns right of its own range
  int i0;               // map row completed by the first batch row: u0 - off2
  int own_r1;           // the loss counts map rows [i0, own_r1)
  rsrc_t ref;           // cached reference statistics: B(y) map planes from p0
  unsigned ref_row;     // their row pitch, bytes
  unsigned ref_plane;   // their plane, bytes
};

// Where relative column rc (from plane p0's column 0) lies: its offset in
// bytes of eb-byte elements from plane p0's start (plane p0 or p0 + 1), or
// kOob for the gap between planes, left of the first and right of the last.
__device__ __forceinline__ unsigned plane_col(const Params& p, const FSeg& s, int rc, int w,
                                              unsigned plane_bytes, unsigned eb) {
  if ((unsigned)rc < (unsigned)w) return (unsigned)rc * eb;
  const int r2 = rc - p.vpitch;
  return (s.p1 && (unsigned)r2 < (unsigned)w) ? plane_bytes + (unsigned)r2 * eb : kOob;
}

// Per segment and row-pass lane: bit c (c < 4) when the lane's map entry c
// lies in a map (outside, the partials are the adjoint's zero fill), bit
// 4 + c when this strip also owns it for the loss (its own 236 map columns,
// and everything to the right for the last strip; rows are checked per
// batch).
__device__ __forceinline__ unsigned fused_masks(const Params& p, const FSeg& s, int lane) {
  const int lr = lane < kFMapLanes ? lane : kFMapLanes - 1;
  unsigned mk = 0u;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int jl = 4 * lr + c;  // map column within the strip
    const bool in_map =
        jl < kFMapCols && plane_col(p, s, s.rv0 - p.off2 + jl, p.map_w, 0u, 1u) != kOob;
    const bool own = in_map && lane < kFMapLanes && (jl < kFOut || s.last);
    mk |= (in_map ? 1u << c : 0u) | (own ? 1u << (4 + c) : 0u);
  }
  return mk;
}

// This lane's pixel of x and y in image row r (0 outside the image).
template <int T>
__device__ __forceinline__ void fload_row(const FSeg& s, int r, float (&v)[2]) {
  // rows outside the image are checked here: with two planes behind one
  // descriptor, a row past one plane's edge would be a valid offset into the
  // other
  const unsigned off = (unsigned)r < (unsigned)s.img_h ? s.colbyte + (unsigned)r * s.row_bytes : kOob;
  v[0] = ld_img<T>(s.img[0], off);
  v[1] = ld_img<T>(s.img[1], off);
}

// The quantities the forward blurs: y, x - y, (x - y)^2 and x' y'
// (x' = x - 1/2, y' = y - 1/2).
__device__ __forceinline__ void image_quantities(const float (&v)[2], float (&q)[kQ]) {
  const float d = v[0] - v[1];
  q[0] = v[1];
  q[1] = d;
  q[2] = d * d;
  q[3] = (v[0] - kShift) * (v[1] - kShift);
}

// Stage 1's column pass of one image row through a 12-slot ring: the row's
// quantities nq go into slot (base + 10) % 12 and the output is the 11-tap
// blur over slots base .. base + 10.  Quantities 0 .. kByParts - 1 are kept
// as differences from the row before (prev: that row's values) and blurred
// by parts; quantity kSkip (if any) is not blurred.
template <int kBase, int kSkip>
__device__ __forceinline__ void ring_column_fwd(float (&ring)[kRing][kQ],
                                                float (&prev)[kByParts], const float (&nq)[kQ],
                                                float (&cs)[kQ]) {
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    if (q == kSkip) {
      cs[q] = 0.0f;
    } else if (q < kByParts) {
      ring[(kBase + 10) % kRing][q] = nq[q] - prev[q];
      prev[q] = nq[q];
      cs[q] = blur11_by_parts(nq[q], [&](int j) { return ring[(kBase + j) % kRing][q]; });
    } else {
      ring[(kBase + 10) % kRing][q] = nq[q];
      cs[q] = blur11_plain([&](int a) { return ring[(kBase + a) % kRing][q]; });
    }
  }
}

// Stage 2's column pass (the adjoint's, over the partials already in the
// ring): plain 11-tap blurs over slots base .. base + 10.  Quantity kSkip
// (if any) is not blurred.
template <int kBase, int kSkip = -1>
__device__ __forceinline__ void ring_column(float (&ring)[kRing][kQ], float (&cs)[kQ]) {
#pragma unroll
  for (int q = 0; q < kQ; ++q)
    cs[q] = q == kSkip ? 0.0f : blur11_plain([&](int a) { return ring[(kBase + a) % kRing][q]; });
}

// row pass: 4 adjacent outputs of each of the 4 quantities from 16 columns of
// a tile row starting at column c (16-byte aligned); quantity kSkip (if any)
// is left alone.  kFwd: stage 1's image quantities (0 .. kByParts - 1 by
// parts); otherwise plain.
template <int kSkip = -1, bool kFwd = false>
__device__ __forceinline__ void row_pass(const float* row0, int c, float (&o)[kQ][4]) {
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    if (q == kSkip) continue;
    const float* src = row0 + q * (kRows * kFTileW) + c;
    float v[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 f = *reinterpret_cast<const float4*>(src + 4 * k);
      v[4 * k + 0] = f.x;
      v[4 * k + 1] = f.y;
      v[4 * k + 2] = f.z;
      v[4 * k + 3] = f.w;
    }
    if (kFwd && q < kByParts) blur4<true>(v, o[q]);
    else blur4<false>(v, o[q]);
  }
}

// Which gradients a kernel forms: kBoth, or one of them (the other pointer
// is NULL); a cached reference implies grad_x alone.  The loss partial, and
// the adjoint blur, that only the missing gradient needs are skipped:
// grad_x = B^T m0 + y' B^T m3 + d B^T m2 never uses m1, and grad_y = B^T m1 +
// x' B^T m3 - d B^T m2 never uses m0.
constexpr int kBoth = -1, kOnlyX = 0, kOnlyY = 1;
__host__ __device__ constexpr int unused_partial(bool ref, int grads) {
  return (ref || grads == kOnlyX) ? 1 : grads == kOnlyY ? 0 : -1;
}

// Stage 1 of batch t (PH = t mod 3): the column pass of image rows u0 + 4t
// .. +3 into the tile, then the row pass of tile row `wave` -> SSIM terms,
// loss and partials, written back over that row.  Two barriers.
template <bool kLoss, int T, int PH, bool kRef, int kGrads>
__device__ __forceinline__ void stage1_batch(const Params& p, const FSeg& s,
                                             float (&tile)[2][kQ][kRows][kFTileW],
                                             float (&xyr)[kXYRing][2][kFTileW],
                                             float (&ring)[kRing][kQ], float (&prev)[kByParts],
                                             float (&pre)[kRows][2], unsigned mk, int t, int buf,
                                             int col, int wave, int lane, double& acc) {
  // with a cached reference, B(y) (quantity 0) is read, not blurred; the
  // partial that only a missing gradient needs is not passed on
  constexpr int kSkip = kRef ? 0 : -1;
  constexpr int kSkipPart = unused_partial(kRef, kGrads);
  const int i = s.i0 + 4 * t + wave;
  const bool irow = (unsigned)i < (unsigned)p.map_h;
  const int lr = lane < kFMapLanes ? lane : kFMapLanes - 1;
  float cur[kRows][2];
#pragma unroll
  for (int m = 0; m < kRows; ++m) {
    cur[m][0] = pre[m][0];
    cur[m][1] = pre[m][1];
  }
  // prefetch the next batch's image rows (past the plane they read as 0)
#pragma unroll
  for (int m = 0; m < kRows; ++m) fload_row<T>(s, s.u0 + 4 * (t + 1) + m, pre[m]);

  // this batch's rows of x and y, kept for stage 2's chain rule (ring slot
  // = row within the range mod kXYRing)
  const int xslot = kRows * (t % (kXYRing / kRows));
#pragma unroll
  for (int m = 0; m < kRows; ++m) {
    xyr[xslot + m][0][col + kXYOff] = cur[m][0];
    xyr[xslot + m][1][col + kXYOff] = cur[m][1];
  }
#pragma unroll
  for (int m = 0; m < kRows; ++m) {
    constexpr int kB0 = 4 * PH;
    float cs[kQ], nq[kQ];
    image_quantities(cur[m], nq);
    switch (m) {  // m is a compile-time constant after unrolling
      case 0: ring_column_fwd<kB0 + 0, kSkip>(ring, prev, nq, cs); break;
      case 1: ring_column_fwd<kB0 + 1, kSkip>(ring, prev, nq, cs); break;
      case 2: ring_column_fwd<kB0 + 2, kSkip>(ring, prev, nq, cs); break;
      default: ring_column_fwd<kB0 + 3, kSkip>(ring, prev, nq, cs); break;
    }
#pragma unroll
    for (int q = 0; q < kQ; ++q)
      if (q != kSkip) tile[buf][q][m][col] = cs[q];
  }
  __syncthreads();

  // row pass: wave w -> map row i0 + 4t + w; lane l -> map columns
  // jm0 + 4l .. 4l+3.  The partials go back into the row just read.
  float muy_ref[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (kRef) {
    // the cached B(y) at this lane's 4 map entries (0 outside the map)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const unsigned cb = plane_col(p, s, s.rv0 - p.off2 + 4 * lr + c, p.map_w, s.ref_plane, 4u);
      muy_ref[c] = ld1(s.ref, irow && cb != kOob ? (unsigned)i * s.ref_row + cb : kOob);
    }
  }
  float part[kQ][4];
  if (irow) {
    float o[kQ][4];
    row_pass<kSkip, true>(&tile[buf][0][wave][0], 4 * lr, o);
    if constexpr (kRef) {
#pragma unroll
      for (int c = 0; c < 4; ++c) o[0][c] = muy_ref[c];
    }
    const bool own_row = kLoss && i < s.own_r1;
    float s4 = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool in_map = (mk >> c) & 1u;
      const SsimTerms st = ssim_terms(o[0][c], o[1][c], o[2][c], o[3][c]);
      float m4[4];
      // outside the map the partials are the adjoint's zero fill (a zero
      // scale: every input of the row pass is finite, the overhang included)
      loss_partials(st, in_map ? p.k_m2 : 0.0f, m4);
#pragma unroll
      for (int k = 0; k < kQ; ++k) part[k][c] = m4[k];
      if constexpr (kLoss) {
        const float ell = one_minus_ssim(st);
        s4 += (own_row && ((mk >> (4 + c)) & 1u)) ? ell : 0.0f;
      }
    }
    if constexpr (kLoss) acc += (double)s4;
  } else {
#pragma unroll
    for (int k = 0; k < kQ; ++k)
#pragma unroll
      for (int c = 0; c < 4; ++c) part[k][c] = 0.0f;
  }
  if (lane < kFMapLanes) {
#pragma unroll
    for (int k = 0; k < kQ; ++k)
      if (k != kSkipPart)
        *reinterpret_cast<float4*>(&tile[buf][k][wave][4 * lane]) =
            make_float4(part[k][0], part[k][1], part[k][2], part[k][3]);
  }
  __syncthreads();
}

// Stage 2 of batch t: the adjoint's column pass over the partials stage 1
// left in the tile (lane t owns map column jm0 + t; written back into the
// same column), then the row pass of tile row `wave` and the chain rule for
// gradient row u0 + 4t + wave - 10.  Two barriers.
template <bool kVec, bool kNt, int T, int PH, bool kRef, int kGrads>
__device__ __forceinline__ void stage2_batch(const Params& p, const FSeg& s,
                                             float (&tile)[2][kQ][kRows][kFTileW],
                                             const float (&xyr)[kXYRing][2][kFTileW],
                                             float (&ring)[kRing][kQ], int t, int buf, int col,
                                             int wave, int lane, float dl) {
  // with a cached reference only grad_x is formed; the partial that only a
  // missing gradient needs is neither blurred nor used
  constexpr int kSkip = unused_partial(kRef, kGrads);
  constexpr bool kG1 = kSkip != 0, kG2 = kSkip != 1;
  constexpr unsigned kEb = img_bytes<T>();
  // the gradient row this wave finishes; its x and y come from the row ring
  // that stage 1 filled (no second read of the images).  Stores are never
  // under a branch: groups that are not real use out-of-range offsets.
  const int gr = 4 * t + wave - 10;  // row within the range; < 0 while the adjoint warms up
  const bool grow = gr >= 0 && gr < s.nrows;
  // (with W and the plane pitch multiples of 4 a vector group lies wholly in
  // one plane or wholly in a gap, so its first column decides)
  const int gc = s.rv0 + 4 * lane;  // relative column of the lane's first gradient
  const unsigned rowoff = (unsigned)(s.u0 + gr) * s.row_bytes;
  unsigned goff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const unsigned cb = plane_col(p, s, gc + c, p.img_w, s.plane_bytes, kEb);
    goff[c] = (grow && lane < kFGradLanes && cb != kOob) ? rowoff + cb : kOob;
  }
  const unsigned gbase = goff[0];

#pragma unroll
  for (int m = 0; m < kRows; ++m) {
    constexpr int kB0 = 4 * PH;
#pragma unroll
    for (int q = 0; q < kQ; ++q)
      if (q != kSkip) ring[(kB0 + m + 10) % kRing][q] = tile[buf][q][m][col];
    float cs[kQ];
    switch (m) {
      case 0: ring_column<kB0 + 0, kSkip>(ring, cs); break;
      case 1: ring_column<kB0 + 1, kSkip>(ring, cs); break;
      case 2: ring_column<kB0 + 2, kSkip>(ring, cs); break;
      default: ring_column<kB0 + 3, kSkip>(ring, cs); break;
    }
#pragma unroll
    for (int q = 0; q < kQ; ++q)
      if (q != kSkip) tile[buf][q][m][col] = cs[q];
  }
  __syncthreads();

  // the arithmetic is skipped, wave-uniformly, while the adjoint warms up
  float g1[4] = {0.0f, 0.0f, 0.0f, 0.0f}, g2[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (grow) {
    const int lr = lane < kFGradLanes ? lane : kFGradLanes - 1;
    // stage-1 lane 10 + 4 lr + c held image column v0 + 4 lr + c
    const float4 xq = *reinterpret_cast<const float4*>(&xyr[gr % kXYRing][0][4 * lr + 10 + kXYOff]);
    const float4 yq = *reinterpret_cast<const float4*>(&xyr[gr % kXYRing][1][4 * lr + 10 + kXYOff]);
    const float xv[4] = {xq.x, xq.y, xq.z, xq.w};
    const float yv[4] = {yq.x, yq.y, yq.z, yq.w};
    float o[kQ][4];
    row_pass<kSkip>(&tile[buf][0][wave][0], 4 * lr, o);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float xs = xv[c] - kShift, ys = yv[c] - kShift, d = xv[c] - yv[c];
      if constexpr (kG1)
        g1[c] = dl * __builtin_fmaf(d, o[2][c], __builtin_fmaf(ys, o[3][c], o[0][c]));
      if constexpr (kG2)
        g2[c] = dl * __builtin_fmaf(-d, o[2][c], __builtin_fmaf(xs, o[3][c], o[1][c]));
    }
  }
  if constexpr (kVec) {
    if constexpr (kG1) st_img4<T, kNt>(s.out[0], gbase, g1);
    if constexpr (kG2) st_img4<T, kNt>(s.out[1], gbase, g2);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if constexpr (kG1) st_img<T, kNt>(s.out[0], goff[c], g1[c]);
      if constexpr (kG2) st_img<T, kNt>(s.out[1], goff[c], g2[c]);
    }
  }
  __syncthreads();
}

// This workgroup's share: a contiguous run of a sequence in which each
// strip-column counts as its kWarm warm-up rows followed by its gradient
// rows, so a share that starts a strip-column is charged for the warm-up it
// pays; a share that starts inside one pays at most kWarm more.  The share is
// taken as one segment per strip-column it touches.
//
// With two workgroups per CU (a grid of 2 x CUs, every workgroup resident at
// once), the one dispatched first onto a CU issues ahead of the other, which
// takes the issue slots left over, so the pair would finish far apart and the
// second would run its last part alone (per tick, a lone workgroup gets 0.62
// of what the pair does together).  The first therefore takes first_w / 100
// times the second's share.  Dispatch hands consecutive workgroup ids to the
// 8 XCDs in turn and, within an XCD, to its CUs in turn: ids below G / 2 are
// the first on their CU, which logical_block makes the first half of each
// XCD's run.  first_w == 100 gives equal shares.
struct FShare {
  int64_t v, v_end, vlen;
};
constexpr int kWarm = 20;

__device__ __forceinline__ FShare fused_share(const Params& p) {
  FShare w;
  w.vlen = (int64_t)p.out_h + kWarm;
  const int64_t total = p.cols * w.vlen;
  const int64_t lb = logical_block();
  const int64_t G = gridDim.x;
  if (p.first_w == 100 || G % 8 != 0) {
    w.v = lb * total / G;
    w.v_end = (lb + 1) * total / G;
    return w;
  }
  const int64_t m = G / 8, h = m / 2;  // workgroups per XCD, of which first on a CU
  const int64_t x = lb / m, k = lb - x * m;
  const int64_t fw = p.first_w;
  // weight of the first kk workgroups of an XCD's run
  const auto cum = [&](int64_t kk) { return fw * (kk < h ? kk : h) + 100 * (kk > h ? kk - h : 0); };
  const int64_t per = cum(m);
  w.v = (x * per + cum(k)) * total / (8 * per);
  w.v_end = (x * per + cum(k + 1)) * total / (8 * per);
  return w;
}

// The next segment of the share: false when the share is done.  A segment
// with no gradient rows (a share's tail inside a warm-up) is skipped.
template <int T>
__device__ __forceinline__ bool next_segment(const Params& p, FShare& w, FSeg& s, int col) {
  constexpr unsigned kEb = img_bytes<T>();
  for (;;) {
    if (w.v >= w.v_end) return false;
    const int64_t sc = w.v / w.vlen;
    const int64_t col_end = (sc + 1) * w.vlen;
    const int64_t seg_end = col_end < w.v_end ? col_end : w.v_end;
    const int64_t r0 = w.v - sc * w.vlen - kWarm, r1 = seg_end - sc * w.vlen - kWarm;
    const int row_begin = (int)(r0 > 0 ? r0 : 0);
    const int row_end = (int)(r1 > 0 ? r1 : 0);
    w.v = seg_end;
    if (row_end <= row_begin) continue;
    // strip sc of the planes laid side by side: plane p0 holds its first
    // image column (the halo's), and it reaches at most plane p0 + 1
    const int64_t v0 = sc * kFOut;
    const int64_t p0 = v0 >= 10 ? (v0 - 10) / p.vpitch : 0;
    const int64_t np = p.planes - p0 < 2 ? p.planes - p0 : 2;
    s.u0 = row_begin;
    s.nrows = row_end - row_begin;
    s.rv0 = (int)(v0 - p0 * p.vpitch);
    s.p1 = np > 1;
    s.last = sc == p.cols - 1;
    s.i0 = s.u0 - p.off2;
    s.row_bytes = (unsigned)p.img_w * kEb;
    s.plane_bytes = (unsigned)(p.img_plane * kEb);
    s.img_h = p.in_h;
    s.colbyte = plane_col(p, s, s.rv0 - 10 + col, p.img_w, s.plane_bytes, kEb);
    const int64_t pb = p0 * p.img_plane * kEb;
    const int64_t span = np * p.img_plane * kEb;
    s.img[0] = make_rsrc(byte_ptr(p.x, pb), span);
    s.img[1] = make_rsrc(byte_ptr(p.y, pb), span);
    s.out[0] = make_rsrc(p.gx ? byte_ptr(p.gx, pb) : p.x, p.gx ? span : 0);
    s.out[1] = make_rsrc(p.gy ? byte_ptr(p.gy, pb) : p.y, p.gy ? span : 0);
    // the last row range owns the map's remaining rows (same padding: the map
    // reaches 5 past the last gradient row range's own share)
    s.own_r1 = (row_end == p.out_h) ? p.map_h : row_end - p.off2;
    // cached reference statistics (the map buffer with its row pitch), if any
    s.ref = make_rsrc(p.maps ? p.maps + p0 * p.map_plane : p.x,
                      p.maps ? np * p.map_plane * 4 : 0);
    s.ref_row = (unsigned)p.map_pitch * 4u;
    s.ref_plane = (unsigned)(p.map_plane * 4);
    return true;
  }
}

// batches of a segment: n gradient rows need n + 10 rows of partials
__device__ __forceinline__ int segment_batches(const FSeg& s) {
  return (s.nrows + 10 + kRows - 1) / kRows;
}

// kLoss: also form loss = 1 - mean SSIM (the whole training step in one
// launch); otherwise gradients only (a backward that needs no saved maps).
//
// Eight waves: waves 0-3 run stage 1 on batch t while waves 4-7 run stage 2
// on batch t-1, so each wave holds one register ring and the workgroup keeps
// more waves resident per SIMD.  Batch t lives in tile buffer (number of
// batches before it in this workgroup) mod 2; per segment each group passes
// 2 (nb + 1) barriers (stage 2 idles through the first tick, stage 1
// through the last), so the two loops meet at every barrier.
// kRef: B(y) comes from a cached map (p.maps, the layout the
// reference-statistics kernel writes) and only grad_x is formed.
// kGrads: both gradients, or grad_x (kOnlyX) or grad_y (kOnlyY) alone.
template <bool kLoss, bool kVec, bool kNt, int T, bool kRef = false, int kGrads = kBoth>
__device__ __forceinline__ void fused_body(const Params& p) {
  __shared__ float tile[2][kQ][kRows][kFTileW];
  __shared__ float xyr[kXYRing][2][kFTileW];
  __shared__ double red[kFWaves];

  // wave index as a scalar, so the split below is a scalar branch: each wave
  // runs exactly one of the two loops
  const int wave_id = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  // the tile rows' 4-column overhang past the 256 lanes is read by the last
  // stage-1 row-pass lane but written by no stage: zero it once, so that
  // the entries it feeds (outside the map) stay finite and scale to zero
  if (threadIdx.x < 2 * kQ * kRows * (kFTileW - kTileW)) {
    const int k = threadIdx.x % (kFTileW - kTileW), r = threadIdx.x / (kFTileW - kTileW);
    (&tile[0][0][0][0])[r * kFTileW + kTileW + k] = 0.0f;
  }
  FShare w = fused_share(p);
  double acc = 0.0;
  int gb = 0;  // batches of earlier segments

  if (wave_id < kWaves) {
    // stage 1
    const int col = threadIdx.x;
    FSeg s;
    while (next_segment<T>(p, w, s, col)) {
      const int nb = segment_batches(s);
      const unsigned mk = fused_masks(p, s, lane);
      float ring[kRing][kQ];
      float prev[kByParts];
      float pre[kRows][2];
      {
        float warm[10][2];
#pragma unroll
        for (int k = 0; k < 10; ++k) fload_row<T>(s, s.u0 - 10 + k, warm[k]);
#pragma unroll
        for (int m = 0; m < kRows; ++m) fload_row<T>(s, s.u0 + m, pre[m]);
        // the first 10 rows of the window; for the quantities blurred by
        // parts, each row's difference from the one before (slot 0's is
        // never read)
#pragma unroll
        for (int k = 0; k < 10; ++k) {
          float nq[kQ];
          image_quantities(warm[k], nq);
#pragma unroll
          for (int q = 0; q < kQ; ++q) {
            if (q < kByParts) {
              ring[k][q] = k > 0 ? nq[q] - prev[q] : 0.0f;
              prev[q] = nq[q];
            } else {
              ring[k][q] = nq[q];
            }
          }
        }
      }
      for (int t = 0;;) {
        if (t >= nb) break;
        stage1_batch<kLoss, T, 0, kRef, kGrads>(p, s, tile, xyr, ring, prev, pre, mk, t, (gb + t) & 1, col, wave_id,
                                          lane,
                                          acc);
        if (++t >= nb) break;
        stage1_batch<kLoss, T, 1, kRef, kGrads>(p, s, tile, xyr, ring, prev, pre, mk, t, (gb + t) & 1, col, wave_id,
                                          lane,
                                          acc);
        if (++t >= nb) break;
        stage1_batch<kLoss, T, 2, kRef, kGrads>(p, s, tile, xyr, ring, prev, pre, mk, t, (gb + t) & 1, col, wave_id,
                                          lane,
                                          acc);
        ++t;
      }
      // last tick: stage 2 finishes the segment's last batch
      __syncthreads();
      __syncthreads();
      gb += nb;
    }
  } else {
    // stage 2
    const int col = threadIdx.x - kWaves * kWave;
    const int wave = wave_id - kWaves;
    const float dl = *p.dloss;
    FSeg s;
    while (next_segment<T>(p, w, s, col)) {
      const int nb = segment_batches(s);
      float ring[kRing][kQ];
#pragma unroll
      for (int k = 0; k < kRing; ++k)
#pragma unroll
        for (int q = 0; q < kQ; ++q) ring[k][q] = 0.0f;
      // first tick: stage 1 forms the segment's first batch
      __syncthreads();
      __syncthreads();
      for (int t = 0;;) {
        if (t >= nb) break;
        stage2_batch<kVec, kNt, T, 0, kRef, kGrads>(p, s, tile, xyr, ring, t, (gb + t) & 1, col, wave, lane, dl);
        if (++t >= nb) break;
        stage2_batch<kVec, kNt, T, 1, kRef, kGrads>(p, s, tile, xyr, ring, t, (gb + t) & 1, col, wave, lane, dl);
        if (++t >= nb) break;
        stage2_batch<kVec, kNt, T, 2, kRef, kGrads>(p, s, tile, xyr, ring, t, (gb + t) & 1, col, wave, lane, dl);
        ++t;
      }
      gb += nb;
    }
  }
  if constexpr (kLoss) finish_loss<kFWaves>(p, acc, red);
}

}  // namespace ssim_dev
