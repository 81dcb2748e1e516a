// ssim_vol.hpp -- SSIM loss of volumes (NCDHW), forward and backward.
//
// "Fully Fused Differentiable SSIM", 3D data: the 2-D computation is kept on
// each XY slice and the Z axis is handled by a buffer along depth, one
// depth row per thread.  Here: the window is g g g (the same 11 taps on each
// axis), the SSIM terms and loss partials are those of ssim_device.hpp, and
// forward and backward are one skeleton,
//     out[k][i][j] = sum_{a,b,c} g[a] g[b] g[c] in[k+a-off][i+b-off][j+c-off],
// with off = 0 / 5 (forward, valid / same) and 10 / 5 (backward, the adjoint).
//
// One workgroup (256 lanes) owns a 16 x 16 tile of output (i, j) positions of
// one volume and marches along depth.  Per depth step it stages the 26 x 26
// input tile of one slice in LDS (loaded one step ahead into registers), runs the X pass (26 x 16 partial sums) and
// the Y pass (16 x 16) through LDS, and each lane shifts its four XY-blurred
// values into an 11-deep register window whose 11-tap sum is the Z pass (a
// shift keeps the register indices fixed without unrolling the depth loop,
// whose per-step invariants would otherwise be hoisted and spilled).
//
// Training forward: the loss partials m0..m3 (ssim_device.hpp) are saved at
// every map voxel, four planes per volume; the backward blurs them with the
// adjoint offset and applies the chain rule.  The loss is reduced as in the
// 2-D kernels (deterministic, last-workgroup finalize).

#pragma once

#include "ssim_device.hpp"

namespace ssim_dev {

constexpr int kVT = 16;           // output tile side (i and j)
constexpr int kVIn = kVT + 10;    // input tile side
constexpr int kVInP = kVIn + 1;   // LDS row pitch of the input tile
constexpr int kVMinSlices = 24;   // shortest depth range of one workgroup
static_assert(kVT * kVT == kThreads, "one output position per lane");

struct VolParams {
  int D, H, W;          // volume extent
  int Do, Ho, Wo;       // map extent
  int off;              // in index = out index + a - off, on every axis
  int out_d, out_h, out_w;  // extent of this kernel's outputs (map or volume)
  int in_d, in_h, in_w;     // extent of this kernel's blurred input
  int tiles_x, tiles_y;
  int64_t cols;         // tile-columns: volumes * tiles_y * tiles_x
  int parts, per_block;
  const void* x;        // volumes, of the kernel's image type
  const void* y;
  int64_t vol;          // D * H * W
  float* maps;          // training forward: written; backward: read
  int64_t map_vol;      // Do * Ho * Wo
  float k_m2;           // -2 / M
  double inv_m;         // 1 / M
  float* loss;
  Workspace* ws;
  const float* dloss;
  void* gx;
  void* gy;
};

// This workgroup's share of (tile-column, output slice) work, as in the 2-D
// kernels: a depth range of one tile-column, or whole tile-columns.
__device__ __forceinline__ Share vol_share(const VolParams& p) {
  const int lb = logical_block();
  Share w;
  if (p.parts > 1) {
    w.sc_begin = lb / p.parts;
    w.sc_end = w.sc_begin + 1;
    const int part = lb - (int)w.sc_begin * p.parts;
    w.row_begin = (int)((int64_t)part * p.out_d / p.parts);
    w.row_end = (int)((int64_t)(part + 1) * p.out_d / p.parts);
  } else {
    w.sc_begin = (int64_t)lb * p.per_block;
    w.sc_end = w.sc_begin + p.per_block < p.cols ? w.sc_begin + p.per_block : p.cols;
    w.row_begin = 0;
    w.row_end = p.out_d;
  }
  return w;
}

struct VolSeg {
  rsrc_t in[4];         // forward: x, y volumes; backward: the 4 partial maps
  rsrc_t img[2];        // backward: x, y (chain rule)
  rsrc_t out[4];        // training forward: 4 partial maps; backward: grad_x, grad_y
  int i0, j0;           // first output (i, j) of the tile
  int k0, nk;           // output slices [k0, k0 + nk)
};

// One slice's input tile, held in registers between its loads and its LDS
// store: each lane owns up to kVIters positions of the 26 x 26 tile (the
// last iteration is partial).  Forward: x and y; backward: the 4 partials.
constexpr int kVIters = (kVIn * kVIn + kThreads - 1) / kThreads;
template <int MODE>
struct VolPre {
  float v[kVIters][MODE == kBwd ? 4 : 2];
};

// Issue the loads of input slice kin's tile (rows i0 - off .., columns
// j0 - off ..).  Outside the blurred input's extent a load reads 0 (an
// out-of-range offset): for the forward x = y = 0, for the backward a zero
// partial.  Every lane runs every iteration; positions past the tile use an
// out-of-range offset too.
template <int MODE, int T>
__device__ __forceinline__ void vol_load(const VolParams& p, const VolSeg& s, int kin,
                                         VolPre<MODE>& pre) {
  constexpr unsigned kEb = img_bytes<T>();
  const bool kok = (unsigned)kin < (unsigned)p.in_d;
#pragma unroll
  for (int it = 0; it < kVIters; ++it) {
    const int t = threadIdx.x + it * kThreads;
    const bool in_tile = t < kVIn * kVIn;
    const int tt = in_tile ? t : 0;
    const int r = tt / kVIn, c = tt - r * kVIn;
    const int ii = s.i0 - p.off + r, jj = s.j0 - p.off + c;
    const bool ok = in_tile && kok && (unsigned)ii < (unsigned)p.in_h &&
                    (unsigned)jj < (unsigned)p.in_w;
    const unsigned e = ok ? (unsigned)(((int64_t)kin * p.in_h + ii) * p.in_w + jj) : 0u;
    if constexpr (MODE == kBwd) {
      const unsigned off = ok ? e * 4u : kOob;
#pragma unroll
      for (int q = 0; q < kQ; ++q) pre.v[it][q] = ld1(s.in[q], off);
    } else {
      const unsigned off = ok ? e * kEb : kOob;
      pre.v[it][0] = ld_img<T>(s.in[0], off);
      pre.v[it][1] = ld_img<T>(s.in[1], off);
    }
  }
}

// Store a loaded tile into LDS as the four quantities to be blurred.
template <int MODE>
__device__ __forceinline__ void vol_store(const VolPre<MODE>& pre, float (&A)[kQ][kVIn][kVInP]) {
#pragma unroll
  for (int it = 0; it < kVIters; ++it) {
    const int t = threadIdx.x + it * kThreads;
    if (t < kVIn * kVIn) {
      const int r = t / kVIn, c = t - r * kVIn;
      if constexpr (MODE == kBwd) {
#pragma unroll
        for (int q = 0; q < kQ; ++q) A[q][r][c] = pre.v[it][q];
      } else {
        const float xv = pre.v[it][0], yv = pre.v[it][1];
        const float xs = xv - kShift, ys = yv - kShift, d = xv - yv;
        A[0][r][c] = xs;
        A[1][r][c] = ys;
        A[2][r][c] = d * d;
        A[3][r][c] = xs * ys;
      }
    }
  }
}

// One depth step on input slice kin, whose tile `pre` holds: store it to LDS,
// issue the loads of slice kin + 1 into `pre` (their latency hides behind
// this step), blur in X and Y, shift the lane's window down by one slice with
// the new values in slot 10, and return the Z-pass sum over slots 0 .. 10 in
// o.
template <int MODE, int T>
__device__ __forceinline__ void vol_step(const VolParams& p, const VolSeg& s, int kin,
                                         VolPre<MODE>& pre, float (&A)[kQ][kVIn][kVInP],
                                         float (&Bx)[kQ][kVIn][kVT], float (&win)[11][kQ],
                                         float (&o)[kQ]) {
  vol_store<MODE>(pre, A);
  vol_load<MODE, T>(p, s, kin + 1, pre);
  __syncthreads();
  // X pass: 26 rows x 16 columns of partial sums
  constexpr int kXIters = (kVIn * kVT + kThreads - 1) / kThreads;
#pragma unroll
  for (int it = 0; it < kXIters; ++it) {
    const int t = threadIdx.x + it * kThreads;
    if (t < kVIn * kVT) {
      const int r = t / kVT, c = t % kVT;
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        float a = tap(0) * A[q][r][c];
#pragma unroll
        for (int b = 1; b < 11; ++b) a = __builtin_fmaf(tap(b), A[q][r][c + b], a);
        Bx[q][r][c] = a;
      }
    }
  }
  __syncthreads();
  // Y pass at this lane's (i, j), then the Z window
  const int ty = threadIdx.x / kVT, tx = threadIdx.x % kVT;
#pragma unroll
  for (int k = 0; k < 10; ++k)
#pragma unroll
    for (int q = 0; q < kQ; ++q) win[k][q] = win[k + 1][q];
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    float a = tap(0) * Bx[q][ty][tx];
#pragma unroll
    for (int b = 1; b < 11; ++b) a = __builtin_fmaf(tap(b), Bx[q][ty + b][tx], a);
    win[10][q] = a;
  }
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    float a = tap(0) * win[0][q];
#pragma unroll
    for (int c = 1; c < 11; ++c) a = __builtin_fmaf(tap(c), win[c][q], a);
    o[q] = a;
  }
}

// Consume the four blurred values of output slice k at this lane's (i, j).
template <int MODE, bool kNt, int T>
__device__ __forceinline__ void vol_consume(const VolParams& p, const VolSeg& s, int k,
                                            const float (&o)[kQ], float dl, double& acc) {
  const int ty = threadIdx.x / kVT, tx = threadIdx.x % kVT;
  const int i = s.i0 + ty, j = s.j0 + tx;
  const bool ok = (unsigned)k < (unsigned)p.out_d && i < p.out_h && j < p.out_w;
  const unsigned e = ok ? (unsigned)(((int64_t)k * p.out_h + i) * p.out_w + j) : 0u;
  if constexpr (MODE == kBwd) {
    constexpr unsigned kEb = img_bytes<T>();
    const unsigned off = ok ? e * kEb : kOob;
    const float xv = ld_img<T>(s.img[0], off), yv = ld_img<T>(s.img[1], off);
    const float xs = xv - kShift, ys = yv - kShift, d = xv - yv;
    const float g1 = dl * __builtin_fmaf(d, o[2], __builtin_fmaf(ys, o[3], o[0]));
    const float g2 = dl * __builtin_fmaf(-d, o[2], __builtin_fmaf(xs, o[3], o[1]));
    st_img<T, kNt>(s.out[0], off, g1);
    st_img<T, kNt>(s.out[1], off, g2);
  } else {
    const SsimTerms st = ssim_terms(o[0], o[1], o[2], o[3]);
    acc += ok ? (double)one_minus_ssim(st) : 0.0;
    if constexpr (MODE == kFwdTrain) {
      float m[4];
      loss_partials(o[0], o[1], st, p.k_m2, m);
      const unsigned off = ok ? e * 4u : kOob;
#pragma unroll
      for (int q = 0; q < kQ; ++q) st1<kNt>(s.out[q], off, m[q]);
    }
  }
}

template <int MODE, bool kNt, int T>
__device__ __forceinline__ void vol_body(const VolParams& p) {
  __shared__ float A[kQ][kVIn][kVInP];
  __shared__ float Bx[kQ][kVIn][kVT];
  __shared__ double red[kWaves];
  __shared__ int is_last;
  constexpr unsigned kEb = img_bytes<T>();

  float dl = 0.0f;
  if constexpr (MODE == kBwd) dl = *p.dloss;
  const Share w = vol_share(p);
  double acc = 0.0;
  for (int64_t sc = w.sc_begin; sc < w.sc_end; ++sc) {
    VolSeg s;
    const int64_t tiles = (int64_t)p.tiles_x * p.tiles_y;
    const int64_t v = sc / tiles;
    const int tt = (int)(sc - v * tiles);
    s.i0 = (tt / p.tiles_x) * kVT;
    s.j0 = (tt % p.tiles_x) * kVT;
    s.k0 = w.row_begin;
    s.nk = w.row_end - w.row_begin;
    const int64_t vb = v * p.vol * kEb;
    if constexpr (MODE == kBwd) {
      const float* mp = p.maps + v * 4 * p.map_vol;
#pragma unroll
      for (int q = 0; q < kQ; ++q) s.in[q] = make_rsrc(mp + q * p.map_vol, p.map_vol * 4);
      s.img[0] = make_rsrc(byte_ptr(p.x, vb), p.vol * kEb);
      s.img[1] = make_rsrc(byte_ptr(p.y, vb), p.vol * kEb);
      s.out[0] = make_rsrc(p.gx ? byte_ptr(p.gx, vb) : p.x, p.gx ? p.vol * kEb : 0);
      s.out[1] = make_rsrc(p.gy ? byte_ptr(p.gy, vb) : p.y, p.gy ? p.vol * kEb : 0);
    } else {
      s.in[0] = make_rsrc(byte_ptr(p.x, vb), p.vol * kEb);
      s.in[1] = make_rsrc(byte_ptr(p.y, vb), p.vol * kEb);
      if constexpr (MODE == kFwdTrain) {
        float* mp = p.maps + v * 4 * p.map_vol;
#pragma unroll
        for (int q = 0; q < kQ; ++q) s.out[q] = make_rsrc(mp + q * p.map_vol, p.map_vol * 4);
      }
    }

    // warm-up: input slices k0 - off .. k0 - off + 9 enter the window; output
    // slice k0 + n then takes input slices kin0 + n .. kin0 + n + 10
    float win[11][kQ];
#pragma unroll
    for (int k = 0; k < 11; ++k)
#pragma unroll
      for (int q = 0; q < kQ; ++q) win[k][q] = 0.0f;
    float o[kQ];
    const int kin0 = s.k0 - p.off;
    VolPre<MODE> pre;
    vol_load<MODE, T>(p, s, kin0, pre);
    for (int k = 0; k < 10; ++k) vol_step<MODE, T>(p, s, kin0 + k, pre, A, Bx, win, o);
    for (int n = 0; n < s.nk; ++n) {
      vol_step<MODE, T>(p, s, kin0 + 10 + n, pre, A, Bx, win, o);
      vol_consume<MODE, kNt, T>(p, s, s.k0 + n, o, dl, acc);
    }
  }
  if constexpr (MODE != kBwd) {
    // finish_loss reads p.ws, p.loss, p.inv_m through a Params view
    Params q;
    q.ws = p.ws;
    q.loss = p.loss;
    q.inv_m = p.inv_m;
    finish_loss<kWaves>(q, acc, red, is_last);
  }
}

}  // namespace ssim_dev
