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
// One workgroup (512 lanes) owns a 32 x 16 tile of output (i, j) positions of
// one volume and marches along depth.  Each input slice is staged as a
// 42 x 26 tile in LDS (loaded one step ahead into registers), blurred in X
// (42 x 16 partial sums, through LDS) and in Y (32 x 16: each lane forms 4
// outputs of one quantity down one column, and writes them to a transpose
// tile), and each lane then takes the four XY-blurred quantities at its own
// position and feeds them to 11 running sums per quantity that form the Z
// pass (each sum moves one tap per slice inside its multiply-add, so the
// register indices stay fixed without unrolling the depth loop).  The four
// LDS stages of consecutive slices are software-pipelined over
// double-buffered tiles, one barrier per slice.
//
// Training forward: the loss partials m0..m3 (ssim_device.hpp) are saved at
// every map voxel, four planes per volume; the backward blurs them with the
// adjoint offset and applies the chain rule.  The loss is reduced as in the
// 2-D kernels (deterministic, last-workgroup finalize).

#pragma once

#include "ssim_device.hpp"

namespace ssim_dev {

constexpr int kVT = 16;           // output tile columns (j)
constexpr int kVTy = 32;          // output tile rows (i)
constexpr int kVIn = kVT + 10;    // input tile columns
constexpr int kVInY = kVTy + 10;  // input tile rows
constexpr int kVInP = kVIn + 2;   // LDS row pitch of the input tile (16-byte rows)
constexpr int kVByP = (kVInY + 3) / 4 * 4;  // column pitch of the X-blurred tile (16-byte columns)
constexpr int kVAq = (kVInY * kVInP + 63) / 64 * 64;  // quantity stride of the input tile
constexpr int kVCq = kVTy * kVT + 16;       // quantity stride of the transpose tile
constexpr int kVThreads = kVT * kVTy;    // one output position per lane
constexpr int kVWaves = kVThreads / kWave;
constexpr int kVMinSlices = 16;   // shortest depth range of one workgroup
constexpr int kXOut = 8;          // outputs of one X-pass task
constexpr int kXGroups = kVT / kXOut;
constexpr int kXRows = (kVInY + 15) / 16 * 16;  // X-pass rows per quantity, 16-lane aligned
constexpr int kXTasks = kXGroups * kQ * kXRows;
constexpr int kVHalf = 28;        // staged elements per half-wave
static_assert(kVThreads % kWave == 0, "whole waves");
static_assert(kXTasks <= kVThreads && (kQ * kXRows) % kWave == 0,
              "one X-pass task per lane at most; each column group starts a wave");
static_assert(kVAq % 64 == 0 && (kXRows * kVInP) % 64 == 0,
              "X-pass lanes 16 apart read the same bank groups, across quantities too");
static_assert(kVHalf + 4 <= 32 && 2 * kVIn >= kVHalf && kVInP == kVIn + 2,
              "28 consecutive staged elements span at most 32 words of the tile");
static_assert(kVInP % 4 == 0 && kXOut % 4 == 0 && kXOut * (kXGroups - 1) + kXOut + 12 <= kVInP,
              "X-pass tasks read whole 16-byte words inside a tile row");
static_assert(kVT == 16 && kQ == 4 && kVTy / 4 == kVWaves,
              "Y pass: a wave's lanes are 16 columns x 4 quantities, one 4-row group per wave");
static_assert(kVByP % 4 == 0 && (kVByP / 4) % 2 == 1 && 4 * (kVTy / 4 - 1) + 14 <= kVInY &&
                  4 * (kVTy / 4 - 1) + 16 <= kVByP,
              "Y-pass tasks read 16-byte words inside a column, of rows the X pass wrote, "
              "at an odd number of 16-byte words per column");
static_assert(kVCq % 32 == 16, "the transpose tile's quantities sit 16 banks apart");

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
// kernels: a depth range of one tile-column, or whole tile-columns.  dir is
// the direction the range is walked in: the odd ranges of a tile-column walk
// down, so that neighbouring ranges reach the 10 input slices they share at
// about the same time (both at their ends, or both at their starts), while
// those are still in the cache.
__device__ __forceinline__ Share vol_share(const VolParams& p, int& dir) {
  const int lb = logical_block();
  Share w;
  dir = 1;
  if (p.parts > 1) {
    w.sc_begin = lb / p.parts;
    w.sc_end = w.sc_begin + 1;
    const int part = lb - (int)w.sc_begin * p.parts;
    w.row_begin = (int)((int64_t)part * p.out_d / p.parts);
    w.row_end = (int)((int64_t)(part + 1) * p.out_d / p.parts);
    if (part & 1) dir = -1;
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
// store: each lane owns up to kVIters positions of the 42 x 26 tile (the
// last iteration is partial).  Forward: x and y; backward: the 4 partials.
constexpr int kVIters = (kVInY * kVIn + kVThreads / 32 * kVHalf - 1) / (kVThreads / 32 * kVHalf);

// The element of the row-major 42 x 26 tile that this lane stages in
// iteration it, or kVInY * kVIn (none).  A half-wave takes 28 consecutive
// elements (lanes 28 .. 31 idle): with the tile's 26-element rows at a
// 28-word pitch they span at most 32 consecutive words, so the half-wave's
// single-word LDS stores fall on 32 distinct banks.
__device__ __forceinline__ int vol_stage_elem(int it) {
  const int l = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int j = l % 32;
  const int h = (it * kVWaves + w) * 2 + l / 32;
  const int e = h * kVHalf + j;
  return j < kVHalf && e < kVInY * kVIn ? e : kVInY * kVIn;
}
template <int MODE>
struct VolPre {
  float v[kVIters][MODE == kBwd ? 4 : 2];
};

// This lane's staged-tile positions as element offsets within one input
// slice (kOob outside the tile or the slice), once per segment.
__device__ __forceinline__ void vol_tile_offsets(const VolParams& p, const VolSeg& s,
                                                 unsigned (&eo)[kVIters]) {
#pragma unroll
  for (int it = 0; it < kVIters; ++it) {
    const int t = vol_stage_elem(it);
    const bool in_tile = t < kVInY * kVIn;
    const int tt = in_tile ? t : 0;
    const int r = tt / kVIn, c = tt - r * kVIn;
    const int ii = s.i0 - p.off + r, jj = s.j0 - p.off + c;
    const bool ok = in_tile && (unsigned)ii < (unsigned)p.in_h && (unsigned)jj < (unsigned)p.in_w;
    eo[it] = ok ? (unsigned)(ii * p.in_w + jj) : kOob;
  }
}

// Issue the loads of input slice kin's tile.  Outside the blurred input's
// extent a load reads 0 (an out-of-range offset): for the forward x = y = 0,
// for the backward a zero partial.
template <int MODE, int T>
__device__ __forceinline__ void vol_load(const VolParams& p, const VolSeg& s, int kin,
                                         const unsigned (&eo)[kVIters], VolPre<MODE>& pre) {
  constexpr unsigned kEb = img_bytes<T>();
  const bool kok = (unsigned)kin < (unsigned)p.in_d;
  const unsigned slice = kok ? (unsigned)kin * (unsigned)(p.in_h * p.in_w) : 0u;
#pragma unroll
  for (int it = 0; it < kVIters; ++it) {
    const bool ok = kok && eo[it] != kOob;
    if constexpr (MODE == kBwd) {
      const unsigned off = ok ? (slice + eo[it]) * 4u : kOob;
#pragma unroll
      for (int q = 0; q < kQ; ++q) pre.v[it][q] = ld1(s.in[q], off);
    } else {
      const unsigned off = ok ? (slice + eo[it]) * kEb : kOob;
      pre.v[it][0] = ld_img<T>(s.in[0], off);
      pre.v[it][1] = ld_img<T>(s.in[1], off);
    }
  }
}

// Store a loaded tile into LDS as the four quantities to be blurred.
template <int MODE>
__device__ __forceinline__ void vol_store(const VolPre<MODE>& pre, float (&A)[kQ][kVAq]) {
#pragma unroll
  for (int it = 0; it < kVIters; ++it) {
    const int t = vol_stage_elem(it);
    if (t < kVInY * kVIn) {
      const int r = t / kVIn, c = t - r * kVIn;
      const int a = r * kVInP + c;
      if constexpr (MODE == kBwd) {
#pragma unroll
        for (int q = 0; q < kQ; ++q) A[q][a] = pre.v[it][q];
      } else {
        const float xv = pre.v[it][0], yv = pre.v[it][1];
        const float d = xv - yv;
        A[0][a] = yv;
        A[1][a] = d;
        A[2][a] = d * d;
        A[3][a] = (xv - kShift) * (yv - kShift);
      }
    }
  }
}

// X pass of one staged slice: 42 rows x 16 columns of partial sums, stored
// column-major (Bx[q][column][row], columns padded to 44 words).  A task is
// 8 adjacent outputs of one quantity in one row, formed from 20 columns read
// as five 16-byte words (the last two unused).  Tasks run (column group,
// quantity, row) with rows padded to 48, one pass of the first six waves:
// each 16 lanes take 16 consecutive rows of one quantity, whose 16-byte
// reads (7 words of 16 bytes per row) fall on distinct bank groups, and
// lanes 16 apart read the same bank group (16 rows, or the quantity stride
// minus 32 rows, are whole multiples of 64 words); a column group starts a
// wave.
// kFwd: the forward's quantities, blurred by parts in every pass (all four
// here, so that no wave splits between the two forms); otherwise plain.
template <bool kFwd>
__device__ __forceinline__ void vol_xpass(const float (&A)[kQ][kVAq],
                                          float (&Bx)[kQ][kVT][kVByP]) {
  const int t = threadIdx.x;
  const int g = t / (kQ * kXRows);
  const int rem = t - g * (kQ * kXRows);
  const int q = rem / kXRows, r = rem - q * kXRows;
  if (g < kXGroups && r < kVInY) {
    const float* src = &A[q][r * kVInP + kXOut * g];
    float v[kXOut + 12];
#pragma unroll
    for (int k = 0; k < (kXOut + 12) / 4; ++k) {
      const float4 f = *reinterpret_cast<const float4*>(src + 4 * k);
      v[4 * k + 0] = f.x;
      v[4 * k + 1] = f.y;
      v[4 * k + 2] = f.z;
      v[4 * k + 3] = f.w;
    }
    float o[kXOut];
    blur_row<kFwd>(v, o);
#pragma unroll
    for (int u = 0; u < kXOut; ++u) Bx[q][kXOut * g + u][r] = o[u];
  }
}

// Y pass of one X-blurred slice.  Wave w forms output rows 4w .. 4w + 3 of
// every quantity: lane (q, column) reads the 14 words of its column starting
// at row 4w as four 16-byte words (the last two words unused), 4 reads per 4
// outputs.  The 16 columns of one quantity sit an odd number of 16-byte words
// apart (44-word pitch), so a wave's 16-byte reads are free of bank
// conflicts.  The outputs go to the transpose tile C[q][row * 16 + column],
// whose quantities are 16 banks apart, so that each half-wave's stores (two
// quantities, 16 columns) cover 32 distinct banks.
template <bool kFwd>
__device__ __forceinline__ void vol_ypass(const float (&Bx)[kQ][kVT][kVByP],
                                          float (&C)[kQ][kVCq]) {
  const int t = threadIdx.x;
  const int tx = t % kVT, q = (t / kVT) % kQ, g = t / (kVT * kQ);
  const float* src = &Bx[q][tx][4 * g];
  float v[16];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 f = *reinterpret_cast<const float4*>(src + 4 * k);
    v[4 * k + 0] = f.x;
    v[4 * k + 1] = f.y;
    v[4 * k + 2] = f.z;
    v[4 * k + 3] = f.w;
  }
  float o[4];
  blur4<kFwd>(v, o);
#pragma unroll
  for (int u = 0; u < 4; ++u) C[q][(4 * g + u) * kVT + tx] = o[u];
}

// The four XY-blurred quantities at this lane's (i, j), from the transpose
// tile the Y pass wrote (a half-wave reads two 16-word rows: 32 banks).
__device__ __forceinline__ void vol_ytake(const float (&C)[kQ][kVCq], float (&a)[kQ]) {
#pragma unroll
  for (int q = 0; q < kQ; ++q) a[q] = C[q][threadIdx.x];
}

// Z pass as running sums: acc[c] holds the partial sum, over the slices seen
// so far, of the output whose window has the newest slice at tap c.  Each new
// XY-blurred value a moves every sum one tap on, acc[c] <- acc[c - 1] +
// g[c] a, and acc[10] is then the complete sum, in tap order, of the output
// whose window ends at the new slice.
//
// Each move is one v_fmamk_f32 (d = s0 * literal + s1, fused, with its own
// destination), taken in descending c so that acc[c] is overwritten only
// after acc[c + 1] has read it: the sums then stay in their registers across
// the depth loop.  Written with the accumulate form (d += s0 * literal) the
// compiler computed each new sum in its predecessor's register and rotated
// all 40 back with register copies on every slice.  The literals are the fp32
// bits of the taps, checked against them below.
#define SSIM_TAP0_BITS 0x3a86cab6
#define SSIM_TAP1_BITS 0x3bf8ff01
#define SSIM_TAP2_BITS 0x3d13758c
#define SSIM_TAP3_BITS 0x3ddff87f
#define SSIM_TAP4_BITS 0x3e5a1e20
#define SSIM_TAP5_BITS 0x3e8832b0
static_assert(__builtin_bit_cast(unsigned, kTap0) == SSIM_TAP0_BITS &&
                  __builtin_bit_cast(unsigned, kTap1) == SSIM_TAP1_BITS &&
                  __builtin_bit_cast(unsigned, kTap2) == SSIM_TAP2_BITS &&
                  __builtin_bit_cast(unsigned, kTap3) == SSIM_TAP3_BITS &&
                  __builtin_bit_cast(unsigned, kTap4) == SSIM_TAP4_BITS &&
                  __builtin_bit_cast(unsigned, kTap5) == SSIM_TAP5_BITS,
              "the Z pass's literals are the taps' fp32 bits");
#define SSIM_STR_(x) #x
#define SSIM_STR(x) SSIM_STR_(x)
#define SSIM_ZMOVE(c, BITS)                                                  \
  asm("v_fmamk_f32 %0, %1, " SSIM_STR(BITS) ", %2"                           \
      : "=v"(acc[c][q])                                                      \
      : "v"(a[q]), "v"(acc[c - 1][q]))
__device__ __forceinline__ void vol_zpass(float (&acc)[11][kQ], const float (&a)[kQ]) {
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    SSIM_ZMOVE(10, SSIM_TAP0_BITS);  // tap 10 = tap 0
    SSIM_ZMOVE(9, SSIM_TAP1_BITS);
    SSIM_ZMOVE(8, SSIM_TAP2_BITS);
    SSIM_ZMOVE(7, SSIM_TAP3_BITS);
    SSIM_ZMOVE(6, SSIM_TAP4_BITS);
    SSIM_ZMOVE(5, SSIM_TAP5_BITS);
    SSIM_ZMOVE(4, SSIM_TAP4_BITS);
    SSIM_ZMOVE(3, SSIM_TAP3_BITS);
    SSIM_ZMOVE(2, SSIM_TAP2_BITS);
    SSIM_ZMOVE(1, SSIM_TAP1_BITS);
    acc[0][q] = tap(0) * a[q];
  }
}

// The forward's Z pass, by parts: the output whose window has slices
// z0 .. z0 + 10 is v(z0) + sum_{j=1}^{10} T_j (v(z0 + j) - v(z0 + j - 1)),
// T_j = g_j + ... + g_10 (the taps sum to 1), exact for a window that is
// constant along depth.  acc[c] holds that sum for the window whose oldest
// slice arrived c slices ago, with its first c differences in; a new value a
// with difference dl = a - prev (prev: the value before it) moves every sum
// one difference on, acc[c] <- acc[c - 1] + T_c dl, and starts the newest,
// acc[1] = prev + T_1 dl, in descending c as above.  acc[10] is then the
// complete sum of the window that ends at the new slice.
#define SSIM_TAIL1_BITS 0x3f7fbc9b
#define SSIM_TAIL2_BITS 0x3f7dca9d
#define SSIM_TAIL3_BITS 0x3f749344
#define SSIM_TAIL4_BITS 0x3f589434
#define SSIM_TAIL5_BITS 0x3f220cac
#define SSIM_TAIL6_BITS 0x3ebbe6a8
#define SSIM_TAIL7_BITS 0x3e1daf30
#define SSIM_TAIL8_BITS 0x3d36cbc1
#define SSIM_TAIL9_BITS 0x3c0d58d7
#define SSIM_TAIL10_BITS 0x3a86cab6
static_assert(__builtin_bit_cast(unsigned, tail(1)) == SSIM_TAIL1_BITS &&
                  __builtin_bit_cast(unsigned, tail(2)) == SSIM_TAIL2_BITS &&
                  __builtin_bit_cast(unsigned, tail(3)) == SSIM_TAIL3_BITS &&
                  __builtin_bit_cast(unsigned, tail(4)) == SSIM_TAIL4_BITS &&
                  __builtin_bit_cast(unsigned, tail(5)) == SSIM_TAIL5_BITS &&
                  __builtin_bit_cast(unsigned, tail(6)) == SSIM_TAIL6_BITS &&
                  __builtin_bit_cast(unsigned, tail(7)) == SSIM_TAIL7_BITS &&
                  __builtin_bit_cast(unsigned, tail(8)) == SSIM_TAIL8_BITS &&
                  __builtin_bit_cast(unsigned, tail(9)) == SSIM_TAIL9_BITS &&
                  __builtin_bit_cast(unsigned, tail(10)) == SSIM_TAIL10_BITS,
              "the by-parts Z pass's literals are the tail sums' fp32 bits");
#define SSIM_ZPART(c, BITS)                                                  \
  asm("v_fmamk_f32 %0, %1, " SSIM_STR(BITS) ", %2"                           \
      : "=v"(acc[c][q])                                                      \
      : "v"(dl), "v"(acc[c - 1][q]))
__device__ __forceinline__ void vol_zpass_by_parts(float (&acc)[11][kQ], const float (&a)[kQ],
                                                   float (&prev)[kQ]) {
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const float dl = a[q] - prev[q];
    SSIM_ZPART(10, SSIM_TAIL10_BITS);
    SSIM_ZPART(9, SSIM_TAIL9_BITS);
    SSIM_ZPART(8, SSIM_TAIL8_BITS);
    SSIM_ZPART(7, SSIM_TAIL7_BITS);
    SSIM_ZPART(6, SSIM_TAIL6_BITS);
    SSIM_ZPART(5, SSIM_TAIL5_BITS);
    SSIM_ZPART(4, SSIM_TAIL4_BITS);
    SSIM_ZPART(3, SSIM_TAIL3_BITS);
    SSIM_ZPART(2, SSIM_TAIL2_BITS);
    asm("v_fmamk_f32 %0, %1, " SSIM_STR(SSIM_TAIL1_BITS) ", %2"
        : "=v"(acc[1][q])
        : "v"(dl), "v"(prev[q]));
    prev[q] = a[q];
  }
}
#undef SSIM_ZPART
#undef SSIM_TAIL1_BITS
#undef SSIM_TAIL2_BITS
#undef SSIM_TAIL3_BITS
#undef SSIM_TAIL4_BITS
#undef SSIM_TAIL5_BITS
#undef SSIM_TAIL6_BITS
#undef SSIM_TAIL7_BITS
#undef SSIM_TAIL8_BITS
#undef SSIM_TAIL9_BITS
#undef SSIM_TAIL10_BITS
#undef SSIM_ZMOVE
#undef SSIM_STR
#undef SSIM_STR_
#undef SSIM_TAP0_BITS
#undef SSIM_TAP1_BITS
#undef SSIM_TAP2_BITS
#undef SSIM_TAP3_BITS
#undef SSIM_TAP4_BITS
#undef SSIM_TAP5_BITS

// This lane's (i, j) as an element offset within one output slice, or kOob
// outside the output extent (once per segment).
__device__ __forceinline__ unsigned vol_out_pos(const VolParams& p, const VolSeg& s) {
  const int ty = threadIdx.x / kVT, tx = threadIdx.x % kVT;
  const int i = s.i0 + ty, j = s.j0 + tx;
  return (i < p.out_h && j < p.out_w) ? (unsigned)(i * p.out_w + j) : kOob;
}

// Where output slice k at this lane's (i, j) lives: its byte offset for
// elements of eb bytes, or kOob outside the output extent.
__device__ __forceinline__ unsigned vol_out_off(const VolParams& p, int k, unsigned oo,
                                                unsigned eb) {
  const bool ok = (unsigned)k < (unsigned)p.out_d && oo != kOob;
  return ok ? ((unsigned)k * (unsigned)(p.out_h * p.out_w) + oo) * eb : kOob;
}

// Backward: x and y at output slice k of this lane (issued a step before the
// chain rule needs them).
template <int T>
__device__ __forceinline__ void vol_load_xy(const VolParams& p, const VolSeg& s, int k,
                                            unsigned oo, float (&xy)[2]) {
  const unsigned off = vol_out_off(p, k, oo, img_bytes<T>());
  xy[0] = ld_img<T>(s.img[0], off);
  xy[1] = ld_img<T>(s.img[1], off);
}

// Consume the four blurred values of output slice k at this lane's (i, j):
// forward, the loss term and (training) the saved partials; backward, the
// chain rule with this voxel's x, y (xy) and both gradients.
template <int MODE, bool kNt, int T>
__device__ __forceinline__ void vol_consume(const VolParams& p, const VolSeg& s, int k,
                                            unsigned oo, const float (&o)[kQ],
                                            const float (&xy)[2], float dl, double& acc) {
  if constexpr (MODE == kBwd) {
    const unsigned off = vol_out_off(p, k, oo, img_bytes<T>());
    const float xv = xy[0], yv = xy[1];
    const float xs = xv - kShift, ys = yv - kShift, d = xv - yv;
    const float g1 = dl * __builtin_fmaf(d, o[2], __builtin_fmaf(ys, o[3], o[0]));
    const float g2 = dl * __builtin_fmaf(-d, o[2], __builtin_fmaf(xs, o[3], o[1]));
    st_img<T, kNt>(s.out[0], off, g1);
    st_img<T, kNt>(s.out[1], off, g2);
  } else {
    const unsigned off = vol_out_off(p, k, oo, 4u);
    const SsimTerms st = ssim_terms(o[0], o[1], o[2], o[3]);
    acc += off != kOob ? (double)one_minus_ssim(st) : 0.0;
    if constexpr (MODE == kFwdTrain) {
      float m[4];
      loss_partials(st, p.k_m2, m);
#pragma unroll
      for (int q = 0; q < kQ; ++q) st1<kNt>(s.out[q], off, m[q]);
    }
  }
}

template <int MODE, bool kNt, int T>
__device__ __forceinline__ void vol_body(const VolParams& p) {
  __shared__ __align__(16) float A[2][kQ][kVAq];
  __shared__ __align__(16) float Bx[2][kQ][kVT][kVByP];
  __shared__ float C[2][kQ][kVCq];
  __shared__ double red[kVWaves];
  constexpr unsigned kEb = img_bytes<T>();

  float dl = 0.0f;
  if constexpr (MODE == kBwd) dl = *p.dloss;
  int dir;
  const Share w = vol_share(p, dir);
  double acc = 0.0;
  for (int64_t sc = w.sc_begin; sc < w.sc_end; ++sc) {
    VolSeg s;
    const int64_t tiles = (int64_t)p.tiles_x * p.tiles_y;
    const int64_t v = sc / tiles;
    const int tt = (int)(sc - v * tiles);
    s.i0 = (tt / p.tiles_x) * kVTy;
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

    // Input slices kin0 .. kin0 + nsl - 1 pass through the lane's running
    // sums, upwards (dir 1) or downwards (dir -1, the taps are symmetric);
    // the first 10 only start them, and the (10 + n)-th completes the n-th
    // output slice of the range in the same direction.  Four stages per
    // slice, one step apart, each
    // step ending in the only barrier: in step j the tile of slice j goes
    // into A[j & 1] (its loads were issued in step j - 1), slice j - 1 is
    // blurred in X from A[(j - 1) & 1] into Bx[(j - 1) & 1], slice j - 2 in
    // Y from Bx[j & 1] into C[j & 1], and slice j - 3 is taken from
    // C[(j - 1) & 1] into the Z sums.  No buffer is written in the step that
    // reads its other use, and each stage reads what an earlier step wrote.
    float acc_z[11][kQ];
    float zprev[kQ] = {0.0f, 0.0f, 0.0f, 0.0f};  // the forward's by-parts Z pass
#pragma unroll
    for (int k = 0; k < 11; ++k)
#pragma unroll
      for (int q = 0; q < kQ; ++q) acc_z[k][q] = 0.0f;
    const int kin0 = s.k0 - p.off;
    const int nsl = 10 + s.nk;
    const int kin_first = dir > 0 ? kin0 : kin0 + nsl - 1;
    const int kout_first = dir > 0 ? s.k0 : s.k0 + s.nk - 1;
    unsigned eo[kVIters];
    vol_tile_offsets(p, s, eo);
    const unsigned oo = vol_out_pos(p, s);
    VolPre<MODE> pre;
    vol_load<MODE, T>(p, s, kin_first, eo, pre);
    float xy[2] = {0.0f, 0.0f};
    for (int j = 0; j < nsl + 3; ++j) {
      if (j < nsl) {
        vol_store<MODE>(pre, A[j & 1]);
        vol_load<MODE, T>(p, s, kin_first + dir * (j + 1), eo, pre);
      }
      if (j >= 1 && j <= nsl) vol_xpass<MODE != kBwd>(A[(j - 1) & 1], Bx[(j - 1) & 1]);
      if (j >= 2 && j <= nsl + 1) vol_ypass<MODE != kBwd>(Bx[j & 1], C[j & 1]);
      // (before slice 0 reaches the Z pass the sums take zeros, which leave
      // them unchanged but keep their update out of any branch)
      float a[kQ] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (j >= 3) vol_ytake(C[(j - 1) & 1], a);
      if constexpr (MODE == kBwd) vol_zpass(acc_z, a);
      else vol_zpass_by_parts(acc_z, a, zprev);
      const int n = j - 13;  // the range's n-th output slice, once its 11 slices are in
      if (n >= 0)
        vol_consume<MODE, kNt, T>(p, s, kout_first + dir * n, oo, acc_z[10], xy, dl, acc);
      // the chain rule's x, y for the next step's output slice
      if constexpr (MODE == kBwd) {
        if (j >= 12 && j < nsl + 2) vol_load_xy<T>(p, s, kout_first + dir * (j - 12), oo, xy);
      }
      __syncthreads();
    }
  }
  if constexpr (MODE != kBwd) {
    // finish_loss reads p.ws, p.loss, p.inv_m through a Params view
    Params q;
    q.ws = p.ws;
    q.loss = p.loss;
    q.inv_m = p.inv_m;
    finish_loss<kVWaves>(q, acc, red);
  }
}

}  // namespace ssim_dev
