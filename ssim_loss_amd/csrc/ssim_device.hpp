// ssim_device.hpp -- device side of the fused SSIM loss (forward and
// backward) for gfx950: constants, kernel parameters and the strip-marching
// skeleton, templated on direction, store policy and image storage type.
// Each ssim_kernels_<type>.hip instantiates the entry kernels for one image
// type; ssim_api.hip is the host side (C ABI, argument checks, launches).
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
//     blurred quantities suffice: mu_y = B(y), mu_d = B(x - y),
//     R = B((x - y)^2) and P' = B(x' y'), with x' = x - 1/2, y' = y - 1/2.
//     Then mu_x = mu_y + mu_d, dmu = mu_d, mu' = mu - 1/2 and
//         A1 = 2 mu_x mu_y + C1,  D1 = dmu^2,            B1 = A1 + D1
//         A2 = 2 (P' - mu_x' mu_y') + C2,  D2 = R - dmu^2, B2 = A2 + D2
//         1 - S = (A1 D2 + D1 B2) / (B1 B2).
//     The shift by 1/2 leaves every covariance unchanged and halves the
//     magnitudes that cancel in P' - mu_x' mu_y'; the difference basis makes
//     B1 - A1 and B2 - A2 exact by construction, so identical images give a
//     loss and gradients of exactly zero and near-identical images (SSIM
//     near 1, the end of a training run) keep full relative accuracy in
//     1 - S, which is what the loss sums.  The forward blurs all four by
//     parts (blur11_by_parts), which is exact on a constant window; why that
//     matters is at ssim_terms.
//   * The pages send five upstream gradients through B^T (mu1, mu2, s11, s22,
//     s12); here there are four, m0..m3 = d loss / d(mu_x, mu_y, R, P') (R's
//     with the chain rule's 2 folded in), and
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
//                 four quantities in a 12-slot register ring (the forward's
//                 as differences from the row before, for the blur by
//                 parts); each new row gives one column-blurred row of the
//                 four quantities.
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
// partial per workgroup -> one 64-bit atomic add of the partial in fixed
// point together with a completion count (finish_loss); the last workgroup
// writes loss = sum / M.  Deterministic; no atomics on floating point.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#if defined(__HIP_DEVICE_COMPILE__)
#if !defined(__gfx950__)
#error "this library targets gfx950 (MI355X) only"
#endif
#endif

namespace ssim_dev {

constexpr int kWave = 64;        // gfx9 wavefront size; checked on the host at run time
constexpr int kThreads = 256;    // 4 waves per workgroup
constexpr int kWaves = kThreads / kWave;
constexpr int kTileW = 256;      // input columns per strip: one per lane
constexpr int kStripOut = 244;   // outputs per strip: 256 - 10, rounded down to a multiple of 4
constexpr int kRowLanes = kStripOut / 4;  // lanes active in the row pass (61)
constexpr int kRows = 4;         // rows per batch = waves (one row each in the row pass)
constexpr int kRing = 12;        // ring slots: 11 rows needed, 12 so 3 batches of 4 close the cycle
constexpr int kQ = 4;            // blurred quantities / maps
constexpr int kMaxBlocks = 4096; // bound on the grid
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

// Partial sums of the taps, H_j = g_0 + ... + g_{j-1} for j = 1 .. 10, from
// the fp64 Gaussian, rounded once to fp32.  By symmetry the tail sums
// g_j + ... + g_10 are H_{11-j}.
constexpr float kHead1 = 0.0010283800844791101f;
constexpr float kHead2 = 0.0086271382197182951f;
constexpr float kHead3 = 0.044627910348149127f;
constexpr float kHead4 = 0.15398859985784913f;
constexpr float kHead5 = 0.36699413756910282f;
constexpr float kHead6 = 0.63300586243089718f;
constexpr float kHead7 = 0.84601140014215082f;
constexpr float kHead8 = 0.95537208965185094f;
constexpr float kHead9 = 0.99137286178028172f;
constexpr float kHead10 = 0.99897161991552086f;

__host__ __device__ constexpr float head(int j) {
  return j == 1 ? kHead1 : j == 2 ? kHead2 : j == 3 ? kHead3 : j == 4 ? kHead4
       : j == 5 ? kHead5 : j == 6 ? kHead6 : j == 7 ? kHead7 : j == 8 ? kHead8
       : j == 9 ? kHead9 : kHead10;
}
// tail sum g_j + ... + g_10, j = 1 .. 10
__host__ __device__ constexpr float tail(int j) { return head(11 - j); }

// The forward blurs some quantities by parts.  For a window w(0) .. w(10),
//   sum_a g_a w(a) = w(10) - sum_{j=1}^{10} H_j (w(j) - w(j-1))
// (the taps sum to 1), so the blur takes the window's newest value and its
// ten differences.  A constant window has zero differences and comes out
// exactly as its value, where the plain sum g_0 w(0) + g_1 w(1) + ... rounds
// the partial sums; and each difference is formed once per input and shared
// by every window that contains it.  See ssim_terms for why the forward needs
// exact constant windows.
template <typename D>
__device__ __forceinline__ float blur11_by_parts(float newest, const D& dlt) {
  float acc = newest;
#pragma unroll
  for (int j = 1; j < 11; ++j) acc = __builtin_fmaf(-head(j), dlt(j), acc);
  return acc;
}

// The plain 11-tap blur of a window w(0) .. w(10): g_0 w(0), then ten fused
// multiply-adds in tap order.
template <typename W>
__device__ __forceinline__ float blur11_plain(const W& w) {
  float acc = tap(0) * w(0);
#pragma unroll
  for (int a = 1; a < 11; ++a) acc = __builtin_fmaf(tap(a), w(a), acc);
  return acc;
}

// N adjacent outputs of one row from the N + 10 inputs v[0] .. v[N + 9]
// (output u reads v[u] .. v[u + 10]), by parts (kParts: the N + 9
// differences shared by the N outputs) or plain.
template <bool kParts, int N, int M>
__device__ __forceinline__ void blur_row(const float (&v)[M], float (&o)[N]) {
  static_assert(M >= N + 10, "N outputs read N + 10 inputs");
  if constexpr (kParts) {
    // tap by tap across the outputs (the order blur11_by_parts takes), so
    // that each difference is formed once and only a few are live
#pragma unroll
    for (int u = 0; u < N; ++u) o[u] = v[u + 10];
#pragma unroll
    for (int j = 1; j < 11; ++j)
#pragma unroll
      for (int u = 0; u < N; ++u) o[u] = __builtin_fmaf(-head(j), v[u + j] - v[u + j - 1], o[u]);
  } else {
#pragma unroll
    for (int u = 0; u < N; ++u) o[u] = blur11_plain([&](int a) { return v[u + a]; });
  }
}

// Four adjacent outputs from v[0] .. v[13] (the last two of the 16 unused).
template <bool kParts>
__device__ __forceinline__ void blur4(const float (&v)[16], float (&o)[4]) {
  blur_row<kParts>(v, o);
}

// The forward's four quantities (y, x - y, (x - y)^2 and x' y') are blurred
// by parts, the backward's partials plainly.
constexpr int kByParts = 4;

constexpr float kC1 = 1.0e-4f;  // (0.01 * 1)^2
constexpr float kC2 = 9.0e-4f;  // (0.03 * 1)^2
constexpr float kShift = 0.5f;  // x' = x - 1/2 (see the file header)

// The loss reduction's accumulator (finish_loss): fixed-point sum and
// completion count in one word, zero between launches.
struct Workspace {
  unsigned long long acc;
  unsigned long long pad[31];
};

// kRef: blur a reference image alone and store its blurred mean B(y)
// (the statistic that depends on the reference only), for reuse across steps
enum Mode { kFwdInfer = 0, kFwdTrain = 1, kBwd = 2, kRef = 3 };

// Storage type of images and gradients (the arithmetic is fp32 throughout;
// maps are always fp32).
enum ImgType { kImgF32 = 0, kImgF16 = 1, kImgBF16 = 2 };
template <int T>
constexpr unsigned img_bytes() {
  return T == kImgF32 ? 4u : 2u;
}

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
  // images (fwd: the inputs; bwd: read by the chain rule), of the kernel's
  // image type
  const void* x;
  const void* y;
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
  void* gx;             // of the kernel's image type
  void* gy;
  // recomputing kernels (image -> map -> gradient in one pass): off is the
  // forward's offset, off2 the adjoint's; the map extent.  Their strips run
  // over the planes laid side by side, plane p's columns starting at virtual
  // column p * vpitch (vpitch >= W + 10 and >= 256, a multiple of 4: the gap
  // reads as zeros, and a strip spans at most two planes); cols counts
  // those strips.
  int off2;
  int map_h, map_w;
  int vpitch;
  int64_t planes;
  // share of a workgroup dispatched first onto its CU, against one dispatched
  // second, in hundredths (100: equal shares); see fused_share
  int first_w;
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

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcFlags);
}
__device__ __forceinline__ const char* byte_ptr(const void* p, int64_t bytes) {
  return static_cast<const char*>(p) + bytes;
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

// Image elements: fp32, fp16 or bf16 in memory, fp32 in registers.  bf16 is
// the top half of an fp32; fp32 -> bf16 rounds to nearest even.
template <int T>
__device__ __forceinline__ float half_bits_to_float(unsigned h) {
  if constexpr (T == kImgF16) return (float)__builtin_bit_cast(_Float16, (unsigned short)h);
  else return __builtin_bit_cast(float, h << 16);
}
template <int T>
__device__ __forceinline__ unsigned float_to_half_bits(float v) {
  if constexpr (T == kImgF16) {
    return __builtin_bit_cast(unsigned short, (_Float16)v);
  } else {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  }
}
// one element at byte offset off
template <int T>
__device__ __forceinline__ float ld_img(rsrc_t r, unsigned off) {
  if constexpr (T == kImgF32) return ld1(r, off);
  else return half_bits_to_float<T>(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}
// four consecutive elements at byte offset off (aligned to 4 elements)
template <int T>
__device__ __forceinline__ void ld_img4(rsrc_t r, unsigned off, float (&v)[4]) {
  if constexpr (T == kImgF32) {
    const float4 a = ld4(r, off);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  } else {
    using u2 = unsigned __attribute__((ext_vector_type(2)));
    const u2 w = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    v[0] = half_bits_to_float<T>(w.x & 0xffffu);
    v[1] = half_bits_to_float<T>(w.x >> 16);
    v[2] = half_bits_to_float<T>(w.y & 0xffffu);
    v[3] = half_bits_to_float<T>(w.y >> 16);
  }
}
template <int T, bool kNt>
__device__ __forceinline__ void st_img(rsrc_t r, unsigned off, float v) {
  if constexpr (T == kImgF32) {
    st1<kNt>(r, off, v);
  } else {
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)float_to_half_bits<T>(v), r, off, 0,
                                          kNt ? kPolicyNt : 0);
  }
}
template <int T, bool kNt>
__device__ __forceinline__ void st_img4(rsrc_t r, unsigned off, const float (&v)[4]) {
  if constexpr (T == kImgF32) {
    st4<kNt>(r, off, make_float4(v[0], v[1], v[2], v[3]));
  } else {
    using u2 = unsigned __attribute__((ext_vector_type(2)));
    u2 w;
    w.x = float_to_half_bits<T>(v[0]) | (float_to_half_bits<T>(v[1]) << 16);
    w.y = float_to_half_bits<T>(v[2]) | (float_to_half_bits<T>(v[3]) << 16);
    __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, kNt ? kPolicyNt : 0);
  }
}

// ---------------------------------------------------------------------------
// SSIM at one map position

// The SSIM terms at one map position, from the blurred quantities
// mu_y = B(y), mu_d = B(x - y), R = B((x - y)^2) and P' = B(x' y')
// (x' = x - 1/2, y' = y - 1/2), with mu_x = mu_y + mu_d.  The first three are
// blurred by parts, exact on constant windows:
//   * a window on which y is constant gives mu_y = y, so mu_y' = mu_y - 1/2 is
//     the very y' in P', and the covariance P' - mu_x' mu_y' carries no bias
//     from a misrounded mean (an 8-bit flat region of a reference image, say:
//     otherwise the same few-ulp error would enter every such window and,
//     divided by C2 = 9e-4, bias the loss);
//   * dmu = mu_d is blurred from the differences themselves, with no
//     cancellation between two means where the images nearly agree;
//   * where both images are constant, dmu is the d = x - y of R, so
//     D2 = R - dmu^2 is exactly 0 (R holds the rounded d^2 and D1 the rounded
//     dmu^2).
struct SsimTerms {
  float mux, muy, mxs, mys, dm, a1, d1, b1, a2, d2, b2, inv;
};

__device__ __forceinline__ SsimTerms ssim_terms(float muy, float mud, float rr, float pp) {
  SsimTerms t;
  t.muy = muy;
  t.dm = mud;
  t.mux = muy + mud;
  t.mxs = t.mux - kShift;
  t.mys = muy - kShift;
  t.a1 = __builtin_fmaf(2.0f * t.mux, t.muy, kC1);
  t.d1 = t.dm * t.dm;
  t.b1 = t.a1 + t.d1;
  const float cov = __builtin_fmaf(-t.mxs, t.mys, pp);
  t.a2 = __builtin_fmaf(2.0f, cov, kC2);
  t.d2 = rr - t.d1;
  t.b2 = t.a2 + t.d2;
  t.inv = __builtin_amdgcn_rcpf(t.b1 * t.b2);
  return t;
}

// 1 - S = (A1 D2 + D1 B2) / (B1 B2)
__device__ __forceinline__ float one_minus_ssim(const SsimTerms& t) {
  return __builtin_fmaf(t.a1, t.d2, t.d1 * t.b2) * t.inv;
}

// The four loss partials at one map position (k_m2 = -2/M), with respect to
// mu_x, mu_y (dmu = mu_x - mu_y), R and P'.  With S = A1 A2 inv,
// inv = 1/(B1 B2), and every term a multiple of D1, D2 or dmu (so all vanish
// when x = y):
//   dS/dmu_x = 2 inv (mu_y T1 - mu_y' T2 + T3)
//   dS/dmu_y = 2 inv (mu_x T1 - mu_x' T2 - T3)
//   dS/dP'   = 2 inv T2,      dS/dR = -S / B2 = -S B1 inv
// where T1 = A2 D1 / B1, T2 = A1 D2 / B2, T3 = S (B1 - B2) dmu.
// Maps (loss = mean of 1 - S over M entries, k = -(2/M) inv):
//   m0 = -(1/M) dS/dmu_x = k (mu_y T1 - mu_y' T2 + T3)
//   m1 = -(1/M) dS/dmu_y = k (mu_x T1 - mu_x' T2 - T3)
//   m2 = -(2/M) dS/dR     = -k S B1   (the chain rule's 2 folded in)
//   m3 = -(1/M) dS/dP'    = k T2
// Every product carries k inv = k_m2 inv^2 =: a once, so with X = a A1,
// Y = a A2: k T2 = X D2 B1, k T1 = Y D1 B2, k T3 = X A2 (B1 - B2) dmu and
// k S B1 = X A2 B1.  A zero k_m2 gives four zero partials.
__device__ __forceinline__ void loss_partials(const SsimTerms& t, float k_m2, float (&m)[4]) {
  const float mxs = t.mxs, mys = t.mys;
  const float a = k_m2 * t.inv * t.inv;
  const float X = a * t.a1, Y = a * t.a2;
  const float xa2 = X * t.a2;
  const float kt2 = X * t.d2 * t.b1;
  const float kt1 = Y * t.d1 * t.b2;
  const float kt3 = xa2 * ((t.b1 - t.b2) * t.dm);
  m[0] = __builtin_fmaf(t.muy, kt1, __builtin_fmaf(-mys, kt2, kt3));
  m[1] = __builtin_fmaf(t.mux, kt1, __builtin_fmaf(-mxs, kt2, -kt3));
  m[2] = -xa2 * t.b1;
  m[3] = kt2;
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
template <int MODE, int T>
__device__ __forceinline__ void load_row(const Params& p, const Seg<MODE>& s, int r,
                                         Raw<MODE>& out) {
  const unsigned off = s.colbyte + (unsigned)r * s.in_row;
  if constexpr (MODE == kBwd) {
#pragma unroll
    for (int k = 0; k < 4; ++k) out.v[k] = ld1(s.in[k], off);
  } else {
    out.v[0] = ld_img<T>(s.in[0], off);
    out.v[1] = ld_img<T>(s.in[1], off);
  }
  out.in = (s.colbyte != kOob) && ((unsigned)r < (unsigned)p.in_h);
}

// Quantities blurred by the forward: y, x - y, (x - y)^2 and x' y' with
// x' = x - 1/2, y' = y - 1/2.  Quantities blurred by the backward: the four
// loss partials at each map entry, formed from the saved blurred quantities.
template <int MODE>
__device__ __forceinline__ void quantities(const Raw<MODE>& r, float k_m2, float (&q)[kQ]) {
  if constexpr (MODE == kBwd) {
    // the loss partials at this map entry; zero outside the map (the
    // adjoint's zero fill)
    float m[4];
    loss_partials(ssim_terms(r.v[0], r.v[1], r.v[2], r.v[3]), k_m2, m);
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = r.in ? m[k] : 0.0f;
  } else {
    (void)k_m2;
    const float d = r.v[0] - r.v[1];
    q[0] = r.v[1];
    q[1] = d;
    q[2] = d * d;
    q[3] = (r.v[0] - kShift) * (r.v[1] - kShift);
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

template <int MODE, bool kVec, int T>
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
      ld_img4<T>(s.img[0], g.base, g.xv);
      ld_img4<T>(s.img[1], g.base, g.yv);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        g.xv[t] = ld_img<T>(s.img[0], g.off[t]);
        g.yv[t] = ld_img<T>(s.img[1], g.off[t]);
      }
    }
  }
}

template <int MODE, bool kVec, bool kNt, int T>
__device__ __forceinline__ void consume(const Params& p, const Seg<MODE>& s,
                                        const Group<MODE, kVec>& g, const float (&o)[kQ][4],
                                        float dl, double& acc) {
  if constexpr (MODE == kRef) {
    // the reference's blurred mean, 16 contiguous bytes of its map row
    (void)dl;
    (void)acc;
    st4<kNt>(s.out[0], g.base, make_float4(o[0][0], o[0][1], o[0][2], o[0][3]));
  } else if constexpr (MODE != kBwd) {
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
      // chain rule: d mu_x/dx = B^T, d P'/dx = y' B^T, d R/dx = 2 (x - y) B^T
      const float xs = g.xv[t] - kShift, ys = g.yv[t] - kShift, d = g.xv[t] - g.yv[t];
      g1[t] = dl * __builtin_fmaf(d, o[2][t], __builtin_fmaf(ys, o[3][t], o[0][t]));
      g2[t] = dl * __builtin_fmaf(-d, o[2][t], __builtin_fmaf(xs, o[3][t], o[1][t]));
    }
    // a gradient the caller does not want has a zero-size descriptor: its
    // stores are dropped without a branch
    if constexpr (kVec) {
      st_img4<T, kNt>(s.out[0], g.base, g1);
      st_img4<T, kNt>(s.out[1], g.base, g2);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        st_img<T, kNt>(s.out[0], g.off[t], g1[t]);
        st_img<T, kNt>(s.out[1], g.off[t], g2[t]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// One batch of kRows rows: column pass into the ring and the LDS tile, then
// the row pass and the consumer.  PH = batch index mod 3 fixes the ring slots
// at compile time.

template <int MODE, bool kVec, bool kNt, int T, int PH>
__device__ __forceinline__ void batch(const Params& p, const Seg<MODE>& s,
                                      float (&tile)[2][kQ][kRows][kTileW],
                                      float (&ring)[kRing][kQ], float (&prev)[kByParts],
                                      Raw<MODE> (&pre)[kRows], int t, int buf, float dl,
                                      double& acc) {
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;

  Group<MODE, kVec> g;
  group_begin<MODE, kVec, T>(p, s, 4 * t + wave, lane, g);

  Raw<MODE> cur[kRows];
#pragma unroll
  for (int m = 0; m < kRows; ++m) cur[m] = pre[m];
  // prefetch the next batch (rows past the segment are harmless: in range
  // they are real pixels, out of range they read as 0)
#pragma unroll
  for (int m = 0; m < kRows; ++m) load_row<MODE, T>(p, s, s.r0 + 10 + 4 * (t + 1) + m, pre[m]);

  // column pass.  The ring holds the backward's partials, and the forward's
  // quantity 3, as values; the forward's quantities 0 .. 2 as differences
  // from the row before (prev: that row's values), blurred by parts.
#pragma unroll
  for (int m = 0; m < kRows; ++m) {
    const int base = 4 * PH + m;  // compile-time after unrolling
    float nq[kQ];
    quantities<MODE>(cur[m], p.k_m2, nq);
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      if (MODE != kBwd && q < kByParts) {
        ring[(base + 10) % kRing][q] = nq[q] - prev[q];
        prev[q] = nq[q];
        tile[buf][q][m][tid] =
            blur11_by_parts(nq[q], [&](int j) { return ring[(base + j) % kRing][q]; });
      } else {
        ring[(base + 10) % kRing][q] = nq[q];
        tile[buf][q][m][tid] = blur11_plain([&](int a) { return ring[(base + a) % kRing][q]; });
      }
    }
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
    if (MODE != kBwd && q < kByParts) blur4<true>(v, o[q]);
    else blur4<false>(v, o[q]);
  }
  consume<MODE, kVec, kNt, T>(p, s, g, o, dl, acc);
}

// Workgroup sum of the map of 1 - S, then the last workgroup to finish
// forms the mean: loss = sum / M.  Every thread of the workgroup calls it.
//
// One 64-bit word carries both the running sum and the completion count:
// each workgroup adds (round(partial * 2^F) << T) + 1 with a single atomic,
// T = the bit length of the grid size (so the count never carries into the
// sum) and F = 62 - T - ceil(log2(2M)) (every partial is at most 2 per map
// entry, so the whole sum stays below bit 62).  The workgroup whose add
// brings the count to the grid size holds the whole sum in the returned
// value: one round trip to memory, and no other value has to be published or
// ordered.  Integer addition is exact and associative, so the loss is the
// same bits on every run; the fixed point's rounding is at most G 2^-(F+1) on
// the sum, about 2^(2T - 62) / loss relative to the loss.  A partial that is
// not finite or not below that bound (NaN or infinite inputs) sets bit 63
// with an atomic OR completed before its add, and the loss is then NaN.
template <int kNW>
__device__ __forceinline__ void finish_loss(const Params& p, double acc, double (&red)[kNW]) {
  const int tid = threadIdx.x;
  const unsigned G = gridDim.x;
  const int wave = tid / kWave, lane = tid % kWave;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  if (tid == 0) {
    double bs = 0.0;
#pragma unroll
    for (int w = 0; w < kNW; ++w) bs += red[w];
    const int T = 32 - __clz((int)G);  // 2^T > G
    int e;
    frexp(2.0 / p.inv_m, &e);           // 2M < 2^e
    const int F = 62 - T - e;
    const double scaled = ldexp(bs, F);
    constexpr unsigned long long kPoison = 1ull << 63;
    if (!(fabs(scaled) < ldexp(1.0, 62 - T))) {  // also true for NaN
      __hip_atomic_fetch_or(&p.ws->acc, kPoison, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
    }
    // rounding may leave a partial of zero slightly negative: it adds 0
    const unsigned long long q =
        scaled > 0.0 && scaled < ldexp(1.0, 62 - T) ? (unsigned long long)__double2ll_rn(scaled)
                                                    : 0ull;
    const unsigned long long add = (q << T) + 1ull;
    const unsigned long long now =
        __hip_atomic_fetch_add(&p.ws->acc, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + add;
    if ((now & ((1ull << T) - 1ull)) == G) {
      const unsigned long long total = (now & ~kPoison) >> T;
      *p.loss = (now & kPoison) ? __builtin_nanf("")
                                : (float)(ldexp((double)total, -F) * p.inv_m);
      __hip_atomic_store(&p.ws->acc, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// This workgroup's share of the grid: one row range of one strip-column, or
// a run of whole strip-columns.  Workgroup ids are first remapped so that
// each XCD (hardware hands consecutive ids to the 8 XCDs in turn) owns one
// contiguous eighth of the work.
struct Share {
  int64_t sc_begin, sc_end;
  int row_begin, row_end;
};

__device__ __forceinline__ int logical_block() {
  const int G = gridDim.x;
  int lb = blockIdx.x;
  if ((G & 7) == 0) lb = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  return lb;
}

__device__ __forceinline__ Share work_share(const Params& p, int rows) {
  const int lb = logical_block();
  Share w;
  if (p.parts > 1) {
    w.sc_begin = lb / p.parts;
    w.sc_end = w.sc_begin + 1;
    const int part = lb - (int)w.sc_begin * p.parts;
    w.row_begin = (int)((int64_t)part * rows / p.parts);
    w.row_end = (int)((int64_t)(part + 1) * rows / p.parts);
  } else {
    w.sc_begin = (int64_t)lb * p.per_block;
    w.sc_end = w.sc_begin + p.per_block < p.cols ? w.sc_begin + p.per_block : p.cols;
    w.row_begin = 0;
    w.row_end = rows;
  }
  return w;
}

template <int MODE, bool kVec, bool kNt, int T>
__device__ __forceinline__ void strip_body(const Params& p) {
  __shared__ float tile[2][kQ][kRows][kTileW];
  __shared__ double red[kWaves];

  const int tid = threadIdx.x;
  // Every workgroup gets the same amount of work, so the grid (one resident
  // wave of workgroups) finishes together.
  const Share w = work_share(p, p.out_h);
  const int64_t sc_begin = w.sc_begin, sc_end = w.sc_end;
  const int row_begin = w.row_begin, row_end = w.row_end;

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
    // the forward reads images of type T; the backward reads fp32 maps
    constexpr unsigned kInElem = (MODE == kBwd) ? 4u : img_bytes<T>();
    constexpr unsigned kEb = img_bytes<T>();
    s.colbyte = (c >= 0 && c < p.in_w) ? (unsigned)c * kInElem : kOob;
    s.in_row = (unsigned)p.in_pitch * kInElem;
    s.r0 = s.row0 - p.off;
    if constexpr (MODE == kBwd) {
      const float* mp = p.maps + plane * 4 * p.map_plane;
#pragma unroll
      for (int k = 0; k < 4; ++k) s.in[k] = make_rsrc(mp + k * p.map_plane, p.map_plane * 4);
      const int64_t pb = plane * p.img_plane * kEb;
      s.img[0] = make_rsrc(byte_ptr(p.x, pb), p.img_plane * kEb);
      s.img[1] = make_rsrc(byte_ptr(p.y, pb), p.img_plane * kEb);
      s.out[0] = make_rsrc(p.gx ? byte_ptr(p.gx, pb) : p.x, p.gx ? p.img_plane * kEb : 0);
      s.out[1] = make_rsrc(p.gy ? byte_ptr(p.gy, pb) : p.y, p.gy ? p.img_plane * kEb : 0);
      s.out_row = (unsigned)p.img_w * kEb;
      s.out_elem = kEb;
    } else {
      s.in[0] = make_rsrc(byte_ptr(p.x, plane * p.in_plane * kEb), p.in_plane * kEb);
      s.in[1] = make_rsrc(byte_ptr(p.y, plane * p.in_plane * kEb), p.in_plane * kEb);
      if constexpr (MODE == kFwdTrain) {
        const float* mp = p.maps + plane * 4 * p.map_plane;
#pragma unroll
        for (int k = 0; k < 4; ++k) s.out[k] = make_rsrc(mp + k * p.map_plane, p.map_plane * 4);
      } else if constexpr (MODE == kRef) {
        s.out[0] = make_rsrc(p.maps + plane * p.map_plane, p.map_plane * 4);
      }
      s.out_row = (unsigned)p.map_pitch * 4u;
      s.out_elem = 4u;
    }
    const int nb = (s.nrows + kRows - 1) / kRows;

    float ring[kRing][kQ];
    float prev[kByParts];
    Raw<MODE> warm[10];
    Raw<MODE> pre[kRows];
#pragma unroll
    for (int k = 0; k < 10; ++k) load_row<MODE, T>(p, s, s.r0 + k, warm[k]);
#pragma unroll
    for (int m = 0; m < kRows; ++m) load_row<MODE, T>(p, s, s.r0 + 10 + m, pre[m]);
    // the first 10 rows of the window; for the quantities blurred by parts,
    // each row's difference from the one before (slot 0's is never read)
#pragma unroll
    for (int k = 0; k < 10; ++k) {
      float nq[kQ];
      quantities<MODE>(warm[k], p.k_m2, nq);
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        if (MODE != kBwd && q < kByParts) {
          ring[k][q] = k > 0 ? nq[q] - prev[q] : 0.0f;
          prev[q] = nq[q];
        } else {
          ring[k][q] = nq[q];
        }
      }
    }

    for (int t = 0;;) {
      if (t >= nb) break;
      batch<MODE, kVec, kNt, T, 0>(p, s, tile, ring, prev, pre, t, buf, dl, acc);
      buf ^= 1;
      if (++t >= nb) break;
      batch<MODE, kVec, kNt, T, 1>(p, s, tile, ring, prev, pre, t, buf, dl, acc);
      buf ^= 1;
      if (++t >= nb) break;
      batch<MODE, kVec, kNt, T, 2>(p, s, tile, ring, prev, pre, t, buf, dl, acc);
      buf ^= 1;
      ++t;
    }
  }

  if constexpr (MODE == kFwdInfer || MODE == kFwdTrain) finish_loss<kWaves>(p, acc, red);
}

}  // namespace ssim_dev
