// ssim_api.hip -- host side of the fused SSIM loss: the C ABI declared in
// ssim_loss_amd.h, argument checks (all before any HIP call), per-device
// launch planning and the launches.  The kernels live in ssim_device.hpp
// (the saved-maps strip kernels and the shared arithmetic), ssim_fused.hpp
// (the recomputing kernels) and ssim_vol.hpp (volumes); ssim_entry.hpp
// declares the entry kernels, instantiated per image type in
// ssim_kernels_{f32,f16,bf16}.hip.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "ssim_entry.hpp"
#include "ssim_loss_amd.h"

namespace {

using namespace ssim_dev;

constexpr int kTypes = 3;  // SSIM_DTYPE_F32, SSIM_DTYPE_F16, SSIM_DTYPE_BF16

const void* const* kernel_table(int dtype) {
  switch (dtype) {
    case SSIM_DTYPE_F16: return ssim_kernel_table_f16();
    case SSIM_DTYPE_BF16: return ssim_kernel_table_bf16();
    default: return ssim_kernel_table_f32();
  }
}

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
  int occ[kTypes][kKinds] = {};  // resident workgroups per CU, per entry kernel
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
      for (int t = 0; t < kTypes; ++t)
        for (int k = 0; k < kKinds; ++k) {
          int n = 0;
          if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel_table(t)[k], kind_threads(k), 0) !=
              hipSuccess)
            return SSIM_ERR_HIP;
          d.occ[t][k] = n > 0 ? n : 1;
        }
      d.status = SSIM_OK;
    }
    d.ready = true;
  }
  *out = &d;
  return d.status;
}

int64_t roundup4(int64_t v) { return (v + 3) & ~(int64_t)3; }

// Scratch of the allocation-free entry point (ssim_loss_and_grad_noalloc):
// the one-launch step's only memory beyond its inputs and outputs is the
// loss accumulator (a Workspace), which here lives in a file-scope device
// array instead of a caller's buffer.  Each GPU holds its own copy for the
// life of the process.  In host code `scratch` names a host-side stand-in,
// not device memory: its device address is taken once per device with
// hipGetSymbolAddress and only that address is used.
constexpr size_t kScratchBytes = 256;
static_assert(sizeof(Workspace) <= kScratchBytes, "the accumulator fits the scratch array");
static __device__ __align__(256) unsigned long long scratch[kScratchBytes / 8];

struct ScratchInfo {
  bool ready = false;
  int status = SSIM_OK;
  void* ptr = nullptr;  // this device's copy of `scratch`
};
ScratchInfo g_scratch[kMaxDevices];

// zero n 64-bit words (a plain kernel, so that a caller capturing the stream
// records a kernel node rather than a memset)
__global__ __launch_bounds__(64) void ssim_zero_words_kernel(unsigned long long* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0ull;
}

// This device's scratch address.  The first call on a device, with that
// device current, resolves it and clears the array on `stream` (ahead of the
// call's own launch on the same stream); later calls reuse the address.  The
// kernels leave the accumulator at zero when they finish, so it stays clear.
int scratch_for_device(void* stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SSIM_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SSIM_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_mu);
  ScratchInfo& s = g_scratch[dev];
  if (!s.ready) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      s.status = SSIM_ERR_HIP;
    } else {
      ssim_zero_words_kernel<<<dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream)>>>(
          static_cast<unsigned long long*>(ptr), (int)(kScratchBytes / 8));
      s.status = hipGetLastError() == hipSuccess ? SSIM_OK : SSIM_ERR_HIP;
      s.ptr = ptr;
    }
    s.ready = true;
  }
  *out = s.ptr;
  return s.status;
}


bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return pa < pb + nb && pb < pa + na;
}

int elem_bytes(int dtype) { return dtype == SSIM_DTYPE_F32 ? 4 : 2; }

// out = *dloss * grad over n fp32 elements, grid-stride; kVec: both arrays
// 16-byte aligned, four elements per load and store, the last n % 4 one at a
// time.  The product is the one the gradient kernels form last.
constexpr int kScaleThreads = 256;
template <bool kVec>
__global__ __launch_bounds__(kScaleThreads) void ssim_grad_scale_kernel(const float* dloss,
                                                                        const float* grad,
                                                                        float* out, int64_t n) {
  const float s = *dloss;
  const int64_t stride = (int64_t)gridDim.x * kScaleThreads;
  const int64_t i0 = (int64_t)blockIdx.x * kScaleThreads + threadIdx.x;
  int64_t done = 0;
  if constexpr (kVec) {
    const int64_t n4 = n >> 2;
    const float4* g4 = reinterpret_cast<const float4*>(grad);
    float4* o4 = reinterpret_cast<float4*>(out);
    for (int64_t k = i0; k < n4; k += stride) {
      const float4 v = g4[k];
      o4[k] = make_float4(s * v.x, s * v.y, s * v.z, s * v.w);
    }
    done = n4 << 2;
  }
  for (int64_t k = done + i0; k < n; k += stride) out[k] = s * grad[k];
}
// an image or gradient pointer must be aligned to its element size
bool misaligned(const void* ptr, int dtype) {
  return ((uintptr_t)ptr % (uintptr_t)elem_bytes(dtype)) != 0;
}

struct Shape {
  int64_t N, C, H, W, Ho, Wo, pitch, planes;
  size_t img_bytes, map_bytes;
};

int check_shape(int64_t N, int64_t C, int64_t H, int64_t W, int padding, int dtype, Shape* s) {
  if (padding != SSIM_PAD_VALID && padding != SSIM_PAD_SAME) return SSIM_ERR_PADDING;
  if (dtype != SSIM_DTYPE_F32 && dtype != SSIM_DTYPE_F16 && dtype != SSIM_DTYPE_BF16)
    return SSIM_ERR_DTYPE;
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
  s->img_bytes = (size_t)(planes * H * W) * elem_bytes(dtype);
  s->map_bytes = (size_t)(planes * Ho * pitch) * 4 * sizeof(float);
  return SSIM_OK;
}

// Grid: one resident wave of workgroups (CUs x occupancy), or fewer when
// the work is small.  With fewer strip-columns than resident workgroups,
// each strip-column is split into `parts` equal row ranges of at least
// kMinRowsPerBlock rows; otherwise each workgroup takes `per_block` whole
// strip-columns.
int plan_grid(const DeviceInfo* d, int dtype, int which, Params& p, int min_rows) {
  int64_t resident = (int64_t)d->cus * d->occ[dtype][which];
  if (resident > kMaxBlocks) resident = kMaxBlocks;
  if (p.cols >= resident) {
    p.parts = 1;
    p.per_block = (int)((p.cols + resident - 1) / resident);
    return (int)((p.cols + p.per_block - 1) / p.per_block);
  }
  int64_t parts = resident / p.cols;
  const int64_t max_parts = (p.out_h + min_rows - 1) / min_rows;
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

int launch(const DeviceInfo* d, int dtype, int which, Params& p, void* stream,
           int min_rows = kMinRowsPerBlock) {
  const int G = plan_grid(d, dtype, which, p, min_rows);
  void* args[] = {&p};
  if (hipLaunchKernel(kernel_table(dtype)[which], dim3(G), dim3(kThreads), args, 0,
                      static_cast<hipStream_t>(stream)) != hipSuccess)
    return SSIM_ERR_HIP;
  return hipGetLastError() == hipSuccess ? SSIM_OK : SSIM_ERR_HIP;
}

int forward_impl(const void* img1, const void* img2, int dtype, int64_t N, int64_t C, int64_t H,
                 int64_t W, int padding, float* loss, float* saved_maps, void* workspace,
                 void* stream) {
  if (!img1 || !img2 || !loss || !workspace) return SSIM_ERR_NULL;
  Shape s;
  int rc = check_shape(N, C, H, W, padding, dtype, &s);
  if (rc != SSIM_OK) return rc;
  if (saved_maps && ((uintptr_t)saved_maps & 15u)) return SSIM_ERR_SHAPE;
  if (misaligned(img1, dtype) || misaligned(img2, dtype)) return SSIM_ERR_SHAPE;
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
  return launch(d, dtype, which, p, stream);
}

int backward_impl(const float* dloss, const void* img1, const void* img2, int dtype, int64_t N,
                  int64_t C, int64_t H, int64_t W, int padding, const float* saved_maps,
                  void* grad_img1, void* grad_img2, void* stream) {
  if (!dloss || !img1 || !img2 || !saved_maps) return SSIM_ERR_NULL;
  Shape s;
  int rc = check_shape(N, C, H, W, padding, dtype, &s);
  if (rc != SSIM_OK) return rc;
  if ((uintptr_t)saved_maps & 15u) return SSIM_ERR_SHAPE;
  if (misaligned(img1, dtype) || misaligned(img2, dtype) || misaligned(grad_img1, dtype) ||
      misaligned(grad_img2, dtype))
    return SSIM_ERR_SHAPE;
  const void* ins[4] = {dloss, img1, img2, saved_maps};
  const size_t inb[4] = {sizeof(float), s.img_bytes, s.img_bytes, s.map_bytes};
  void* outs[2] = {grad_img1, grad_img2};
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

  // 4-wide groups of image elements: 16 bytes (fp32) or 8 bytes (fp16, bf16)
  const uintptr_t al = (uintptr_t)(4 * elem_bytes(dtype));
  const bool vec = (s.W % 4 == 0) && ((uintptr_t)img1 % al == 0) && ((uintptr_t)img2 % al == 0) &&
                   ((uintptr_t)grad_img1 % al == 0) && ((uintptr_t)grad_img2 % al == 0);
  const bool stream_st = 4 * s.img_bytes + s.map_bytes > kStreamBytes;
  const int which = !vec ? kKBwdUnaligned : stream_st ? kKBwdStream : kKBwd;
  return launch(d, dtype, which, p, stream);
}

// The recomputing kernels read only the images: the backward without saved
// maps (loss == NULL) and the one-pass loss and gradients (loss != NULL).
// A share of n gradient rows of one strip-column takes about n/4 + 4 ticks
// and reads n + 20 image rows.  When the work cannot fill the resident grid,
// shorter shares on more workgroups still finish sooner, down to about
// kRecompRowsPerBlock rows each; at least one workgroup per CU runs while
// there are rows for it.
constexpr int kRecompRowsPerBlock = 8;

// ref (optional, with loss): the cached statistics of img2 written by
// ssim_reference_stats; then only grad_img1 is formed.
// use_scratch (with loss, workspace NULL): the accumulator is this device's
// copy of the library's scratch array, looked up after every argument check.
int recompute_impl(const float* dloss, const void* img1, const void* img2, int dtype, int64_t N,
                   int64_t C, int64_t H, int64_t W, int padding, float* loss, void* workspace,
                   void* grad_img1, void* grad_img2, void* stream, const float* ref = nullptr,
                   bool use_scratch = false) {
  if (!dloss || !img1 || !img2) return SSIM_ERR_NULL;
  if (use_scratch && (!loss || workspace)) return SSIM_ERR_NULL;
  if (loss && !workspace && !use_scratch) return SSIM_ERR_NULL;
  Shape s;
  int rc = check_shape(N, C, H, W, padding, dtype, &s);
  if (rc != SSIM_OK) return rc;
  if (misaligned(img1, dtype) || misaligned(img2, dtype) || misaligned(grad_img1, dtype) ||
      misaligned(grad_img2, dtype))
    return SSIM_ERR_SHAPE;
  if (ref && ((uintptr_t)ref & 15u)) return SSIM_ERR_SHAPE;
  const size_t ref_bytes = ref ? s.map_bytes / 4 : 0;  // one fp32 plane of the map layout
  const void* ins[4] = {dloss, img1, img2, ref};
  const size_t inb[4] = {sizeof(float), s.img_bytes, s.img_bytes, ref_bytes};
  const void* outs[4] = {grad_img1, grad_img2, loss, workspace};
  const size_t outb[4] = {s.img_bytes, s.img_bytes, sizeof(float),
                          loss ? sizeof(Workspace) : 0};
  for (int k = 0; k < 4; ++k) {
    for (int l = 0; l < 4; ++l)
      if (overlaps(outs[k], outb[k], ins[l], inb[l])) return SSIM_ERR_ALIAS;
    for (int l = k + 1; l < 4; ++l)
      if (overlaps(outs[k], outb[k], outs[l], outb[l])) return SSIM_ERR_ALIAS;
  }
  if (!loss && !grad_img1 && !grad_img2) return SSIM_OK;

  const DeviceInfo* d = nullptr;
  rc = device_info(&d);
  if (rc != SSIM_OK) return rc;
  if (use_scratch) {
    rc = scratch_for_device(stream, &workspace);
    if (rc != SSIM_OK) return rc;
  }

  Params p;
  memset(&p, 0, sizeof(p));
  p.in_h = (int)s.H;
  p.in_w = (int)s.W;
  p.in_pitch = (int)s.W;
  p.in_plane = s.H * s.W;
  p.out_h = (int)s.H;  // gradient extent
  p.out_w = (int)s.W;
  p.off = padding == SSIM_PAD_VALID ? 0 : 5;    // image -> map
  p.off2 = padding == SSIM_PAD_VALID ? 10 : 5;  // map -> gradient (the adjoint)
  p.map_h = (int)s.Ho;
  p.map_w = (int)s.Wo;
  // the planes side by side, each followed by a gap of at least 10 zero
  // columns (the halo of either padding), a plane pitch of at least 256 (a
  // strip's 256 lanes then touch at most two planes) and a multiple of 4
  // (4-column groups stay inside one plane or one gap)
  int64_t vp = s.W + 10 > 256 ? s.W + 10 : 256;
  vp = (vp + 3) / 4 * 4;
  p.vpitch = (int)vp;
  p.planes = s.planes;
  p.cols = ((s.planes - 1) * vp + s.W + kFOut - 1) / kFOut;
  p.x = img1;
  p.y = img2;
  p.img_plane = s.H * s.W;
  p.img_w = (int)s.W;
  p.dloss = dloss;
  p.gx = grad_img1;
  p.gy = grad_img2;
  const double M = (double)s.planes * (double)s.Ho * (double)s.Wo;
  p.k_m2 = (float)(-2.0 / M);
  p.inv_m = 1.0 / M;
  p.loss = loss;
  p.ws = static_cast<Workspace*>(workspace);

  const uintptr_t al = (uintptr_t)(4 * elem_bytes(dtype));
  const bool vec = (s.W % 4 == 0) && ((uintptr_t)img1 % al == 0) && ((uintptr_t)img2 % al == 0) &&
                   ((uintptr_t)grad_img1 % al == 0) && ((uintptr_t)grad_img2 % al == 0);
  const bool stream_st = 4 * s.img_bytes > kStreamBytes;
  int which = loss ? (!vec ? kKLossGradUnaligned : stream_st ? kKLossGradStream : kKLossGrad)
                   : (!vec ? kKRecompUnaligned : stream_st ? kKRecompStream : kKRecomp);
  // one gradient wanted: the kernels that skip the other's partial and blur
  if (vec && (grad_img1 == nullptr) != (grad_img2 == nullptr)) {
    const bool x = grad_img1 != nullptr;
    which = loss ? (x ? (stream_st ? kKLossGradXStream : kKLossGradX)
                      : (stream_st ? kKLossGradYStream : kKLossGradY))
                 : (x ? (stream_st ? kKRecompXStream : kKRecompX)
                      : (stream_st ? kKRecompYStream : kKRecompY));
  }
  if (ref) {
    which = !vec ? kKLossGradRefUnaligned : stream_st ? kKLossGradRefStream : kKLossGradRef;
    p.maps = const_cast<float*>(ref);
    p.map_pitch = (int)s.pitch;
    p.map_plane = s.Ho * s.pitch;
  }
  // one resident wave of workgroups, each with an equal run of (strip-column,
  // row) pairs; fewer when the rows are few (see kRecompRowsPerBlock)
  const int64_t rows = p.cols * (int64_t)p.out_h;
  int64_t G = (int64_t)d->cus * d->occ[dtype][which];
  if (G > kMaxBlocks) G = kMaxBlocks;
  int64_t want = (rows + kRecompRowsPerBlock - 1) / kRecompRowsPerBlock;
  if (want < d->cus) want = d->cus;
  if (G > want) G = want;
  if (G > rows) G = rows;
  if (G < 1) G = 1;
  // two workgroups per CU: the first dispatched onto a CU takes the larger
  // share (fused_share), by a weight that grows with the share's length --
  // measured best 1.35 at about 54 rows per workgroup (1080p), 1.7 at about
  // 200, 1.9 at 1,700 (8 x 4K)
  p.first_w = 100;
  if (G == 2 * (int64_t)d->cus && d->cus % 8 == 0 && d->occ[dtype][which] == 2) {
    const int64_t per_wg = p.cols * ((int64_t)p.out_h + kWarm) / G;
    p.first_w = per_wg <= 100 ? 135 : per_wg <= 600 ? 170 : 190;
  }

  void* args[] = {&p};
  if (hipLaunchKernel(kernel_table(dtype)[which], dim3((unsigned)G), dim3(kind_threads(which)), args,
                      0, static_cast<hipStream_t>(stream)) != hipSuccess)
    return SSIM_ERR_HIP;
  return hipGetLastError() == hipSuccess ? SSIM_OK : SSIM_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Volumes (NCDHW)

struct Shape3 {
  int64_t N, C, D, H, W, Do, Ho, Wo, vols;
  size_t img_bytes, map_bytes;
};

int check_shape3(int64_t N, int64_t C, int64_t D, int64_t H, int64_t W, int padding, int dtype,
                 Shape3* s) {
  if (padding != SSIM_PAD_VALID && padding != SSIM_PAD_SAME) return SSIM_ERR_PADDING;
  if (dtype != SSIM_DTYPE_F32 && dtype != SSIM_DTYPE_F16 && dtype != SSIM_DTYPE_BF16)
    return SSIM_ERR_DTYPE;
  if (N <= 0 || C <= 0 || D <= 0 || H <= 0 || W <= 0) return SSIM_ERR_SHAPE;
  const int64_t sh = padding == SSIM_PAD_VALID ? 10 : 0;
  const int64_t Do = D - sh, Ho = H - sh, Wo = W - sh;
  if (Do <= 0 || Ho <= 0 || Wo <= 0) return SSIM_ERR_SHAPE;
  // one volume (and its map) holds at most 2^27 elements, so that every
  // byte offset inside it fits 32 bits with room for the out-of-range marker
  const int64_t lim = (int64_t)1 << 27;
  if (W > lim || H > lim / W || D > lim / (H * W)) return SSIM_ERR_OVERFLOW;
  if (N > (int64_t)1 << 40 || C > ((int64_t)1 << 40) / N) return SSIM_ERR_OVERFLOW;
  const int64_t vols = N * C;
  if (vols > ((int64_t)1 << 58) / (D * H * W)) return SSIM_ERR_OVERFLOW;
  s->N = N; s->C = C; s->D = D; s->H = H; s->W = W; s->Do = Do; s->Ho = Ho; s->Wo = Wo;
  s->vols = vols;
  s->img_bytes = (size_t)(vols * D * H * W) * elem_bytes(dtype);
  s->map_bytes = (size_t)(vols * Do * Ho * Wo) * 4 * sizeof(float);
  return SSIM_OK;
}

// One resident wave of workgroups over (tile-column, output slice) work: a
// depth range of one tile-column each, or whole tile-columns.  A depth range
// pays 13 steps before its first output, so ranges are long (at least
// kVMinSlices) while that fills the resident grid; with few tile-columns
// they are shortened, down to kVMinSlicesIdle, until every CU has a
// workgroup: the steps of one range are the latency, and idle CUs cost
// nothing.
constexpr int kVMinSlicesIdle = 4;

int launch_vol(const DeviceInfo* d, int dtype, int which, VolParams& p, void* stream) {
  p.tiles_x = (p.out_w + kVT - 1) / kVT;
  p.tiles_y = (p.out_h + kVTy - 1) / kVTy;
  p.cols = p.cols * p.tiles_x * p.tiles_y;  // volumes * tiles
  int64_t resident = (int64_t)d->cus * d->occ[dtype][which];
  if (resident > kMaxBlocks) resident = kMaxBlocks;
  int64_t G;
  if (p.cols >= resident) {
    p.parts = 1;
    p.per_block = (int)((p.cols + resident - 1) / resident);
    G = (p.cols + p.per_block - 1) / p.per_block;
  } else {
    int64_t parts = resident / p.cols;
    const int64_t max_parts = (p.out_d + kVMinSlices - 1) / kVMinSlices;
    if (parts > max_parts) parts = max_parts;
    int64_t idle = d->cus / p.cols;  // one workgroup per CU
    const int64_t max_idle = (p.out_d + kVMinSlicesIdle - 1) / kVMinSlicesIdle;
    if (idle > max_idle) idle = max_idle;
    if (parts < idle) parts = idle;
    if (parts < 1) parts = 1;
    p.parts = (int)parts;
    p.per_block = 1;
    G = p.cols * parts;
  }
  void* args[] = {&p};
  if (hipLaunchKernel(kernel_table(dtype)[which], dim3((unsigned)G), dim3(kind_threads(which)), args,
                      0, static_cast<hipStream_t>(stream)) != hipSuccess)
    return SSIM_ERR_HIP;
  return hipGetLastError() == hipSuccess ? SSIM_OK : SSIM_ERR_HIP;
}

void fill_vol(VolParams& p, const Shape3& s, int padding) {
  p.D = (int)s.D; p.H = (int)s.H; p.W = (int)s.W;
  p.Do = (int)s.Do; p.Ho = (int)s.Ho; p.Wo = (int)s.Wo;
  p.vol = s.D * s.H * s.W;
  p.map_vol = s.Do * s.Ho * s.Wo;
  p.cols = s.vols;
  const double M = (double)s.vols * (double)p.map_vol;
  p.k_m2 = (float)(-2.0 / M);
  p.inv_m = 1.0 / M;
  (void)padding;
}

int vol_forward_impl(const void* img1, const void* img2, int dtype, int64_t N, int64_t C,
                     int64_t D, int64_t H, int64_t W, int padding, float* loss, float* saved_maps,
                     void* workspace, void* stream) {
  if (!img1 || !img2 || !loss || !workspace) return SSIM_ERR_NULL;
  Shape3 s;
  int rc = check_shape3(N, C, D, H, W, padding, dtype, &s);
  if (rc != SSIM_OK) return rc;
  if (misaligned(img1, dtype) || misaligned(img2, dtype)) return SSIM_ERR_SHAPE;
  if (saved_maps && ((uintptr_t)saved_maps & 15u)) return SSIM_ERR_SHAPE;
  const void* outs[3] = {loss, saved_maps, workspace};
  const size_t outb[3] = {sizeof(float), saved_maps ? s.map_bytes : 0, sizeof(Workspace)};
  for (int k = 0; k < 3; ++k) {
    if (overlaps(outs[k], outb[k], img1, s.img_bytes) || overlaps(outs[k], outb[k], img2, s.img_bytes))
      return SSIM_ERR_ALIAS;
    for (int l = k + 1; l < 3; ++l)
      if (overlaps(outs[k], outb[k], outs[l], outb[l])) return SSIM_ERR_ALIAS;
  }
  const DeviceInfo* d = nullptr;
  rc = device_info(&d);
  if (rc != SSIM_OK) return rc;
  VolParams p;
  memset(&p, 0, sizeof(p));
  fill_vol(p, s, padding);
  p.off = padding == SSIM_PAD_VALID ? 0 : 5;
  p.in_d = (int)s.D; p.in_h = (int)s.H; p.in_w = (int)s.W;
  p.out_d = (int)s.Do; p.out_h = (int)s.Ho; p.out_w = (int)s.Wo;
  p.x = img1;
  p.y = img2;
  p.maps = saved_maps;
  p.loss = loss;
  p.ws = static_cast<Workspace*>(workspace);
  return launch_vol(d, dtype, saved_maps ? kKVolFwdTrain : kKVolFwdInfer, p, stream);
}

int vol_backward_impl(const float* dloss, const void* img1, const void* img2, int dtype,
                      int64_t N, int64_t C, int64_t D, int64_t H, int64_t W, int padding,
                      const float* saved_maps, void* grad_img1, void* grad_img2, void* stream) {
  if (!dloss || !img1 || !img2 || !saved_maps) return SSIM_ERR_NULL;
  Shape3 s;
  int rc = check_shape3(N, C, D, H, W, padding, dtype, &s);
  if (rc != SSIM_OK) return rc;
  if ((uintptr_t)saved_maps & 15u) return SSIM_ERR_SHAPE;
  if (misaligned(img1, dtype) || misaligned(img2, dtype) || misaligned(grad_img1, dtype) ||
      misaligned(grad_img2, dtype))
    return SSIM_ERR_SHAPE;
  const void* ins[4] = {dloss, img1, img2, saved_maps};
  const size_t inb[4] = {sizeof(float), s.img_bytes, s.img_bytes, s.map_bytes};
  void* outs[2] = {grad_img1, grad_img2};
  for (int k = 0; k < 2; ++k)
    for (int l = 0; l < 4; ++l)
      if (overlaps(outs[k], s.img_bytes, ins[l], inb[l])) return SSIM_ERR_ALIAS;
  if (overlaps(grad_img1, s.img_bytes, grad_img2, s.img_bytes)) return SSIM_ERR_ALIAS;
  if (!grad_img1 && !grad_img2) return SSIM_OK;
  const DeviceInfo* d = nullptr;
  rc = device_info(&d);
  if (rc != SSIM_OK) return rc;
  VolParams p;
  memset(&p, 0, sizeof(p));
  fill_vol(p, s, padding);
  p.off = padding == SSIM_PAD_VALID ? 10 : 5;
  p.in_d = (int)s.Do; p.in_h = (int)s.Ho; p.in_w = (int)s.Wo;
  p.out_d = (int)s.D; p.out_h = (int)s.H; p.out_w = (int)s.W;
  p.x = img1;
  p.y = img2;
  p.maps = const_cast<float*>(saved_maps);
  p.dloss = dloss;
  p.gx = grad_img1;
  p.gy = grad_img2;
  return launch_vol(d, dtype, kKVolBwd, p, stream);
}

// The cached reference statistics of img2: B(img2) on the map, one
// fp32 plane per image plane with the saved-maps row pitch.
int ref_stats_impl(const void* img2, int dtype, int64_t N, int64_t C, int64_t H, int64_t W,
                   int padding, float* ref, void* stream) {
  if (!img2 || !ref) return SSIM_ERR_NULL;
  Shape s;
  int rc = check_shape(N, C, H, W, padding, dtype, &s);
  if (rc != SSIM_OK) return rc;
  if (misaligned(img2, dtype) || ((uintptr_t)ref & 15u)) return SSIM_ERR_SHAPE;
  if (overlaps(ref, s.map_bytes / 4, img2, s.img_bytes)) return SSIM_ERR_ALIAS;
  const DeviceInfo* d = nullptr;
  rc = device_info(&d);
  if (rc != SSIM_OK) return rc;
  Params p;
  memset(&p, 0, sizeof(p));
  const int off = padding == SSIM_PAD_VALID ? 0 : 5;
  fill_geometry(p, (int)s.H, (int)s.W, (int)s.W, s.H * s.W, (int)s.Ho, (int)s.Wo, off, s.planes);
  p.x = img2;
  p.y = img2;
  p.img_plane = s.H * s.W;
  p.img_w = (int)s.W;
  p.maps = ref;
  p.map_pitch = (int)s.pitch;
  p.map_plane = s.Ho * s.pitch;
  return launch(d, dtype, kKRefStats, p, stream);
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
    case SSIM_ERR_DTYPE: return "dtype must be SSIM_DTYPE_F32 (0), SSIM_DTYPE_F16 (1) or SSIM_DTYPE_BF16 (2)";
    case SSIM_ERR_SCRATCH: return "the call needs more scratch than the library's fixed device array holds";
    default: return "unknown error code";
  }
}

void ssim_taps(float out[11]) {
  for (int k = 0; k < 11; ++k) out[k] = tap(k);
}

int ssim_map_shape(int64_t H, int64_t W, int padding, int64_t* Ho, int64_t* Wo) {
  if (!Ho || !Wo) return SSIM_ERR_NULL;
  Shape s;
  const int rc = check_shape(1, 1, H, W, padding, SSIM_DTYPE_F32, &s);
  if (rc != SSIM_OK) return rc;
  *Ho = s.Ho;
  *Wo = s.Wo;
  return SSIM_OK;
}

size_t ssim_saved_maps_bytes(int64_t N, int64_t C, int64_t H, int64_t W, int padding) {
  Shape s;
  if (check_shape(N, C, H, W, padding, SSIM_DTYPE_F32, &s) != SSIM_OK) return 0;
  return s.map_bytes;
}

size_t ssim_workspace_bytes(void) { return sizeof(Workspace); }

int ssim_forward(const float* img1, const float* img2, int64_t N, int64_t C, int64_t H,
                 int64_t W, int padding, float* loss, float* saved_maps, void* workspace,
                 void* stream) {
  return forward_impl(img1, img2, SSIM_DTYPE_F32, N, C, H, W, padding, loss, saved_maps,
                      workspace, stream);
}

int ssim_backward(const float* dloss, const float* img1, const float* img2, int64_t N,
                  int64_t C, int64_t H, int64_t W, int padding, const float* saved_maps,
                  float* grad_img1, float* grad_img2, void* stream) {
  return backward_impl(dloss, img1, img2, SSIM_DTYPE_F32, N, C, H, W, padding, saved_maps,
                       grad_img1, grad_img2, stream);
}

int ssim_forward_typed(const void* img1, const void* img2, int dtype, int64_t N, int64_t C,
                       int64_t H, int64_t W, int padding, float* loss, float* saved_maps,
                       void* workspace, void* stream) {
  return forward_impl(img1, img2, dtype, N, C, H, W, padding, loss, saved_maps, workspace, stream);
}

int ssim_backward_typed(const float* dloss, const void* img1, const void* img2, int dtype,
                        int64_t N, int64_t C, int64_t H, int64_t W, int padding,
                        const float* saved_maps, void* grad_img1, void* grad_img2, void* stream) {
  return backward_impl(dloss, img1, img2, dtype, N, C, H, W, padding, saved_maps, grad_img1,
                       grad_img2, stream);
}

int ssim_backward_recompute(const float* dloss, const void* img1, const void* img2, int dtype,
                            int64_t N, int64_t C, int64_t H, int64_t W, int padding,
                            void* grad_img1, void* grad_img2, void* stream) {
  return recompute_impl(dloss, img1, img2, dtype, N, C, H, W, padding, nullptr, nullptr, grad_img1,
                        grad_img2, stream);
}

int ssim_loss_and_grad(const void* img1, const void* img2, int dtype, int64_t N, int64_t C,
                       int64_t H, int64_t W, int padding, const float* dloss, float* loss,
                       void* workspace, void* grad_img1, void* grad_img2, void* stream) {
  if (!loss) return SSIM_ERR_NULL;
  return recompute_impl(dloss, img1, img2, dtype, N, C, H, W, padding, loss, workspace, grad_img1,
                        grad_img2, stream);
}

size_t ssim_noalloc_scratch_bytes(void) { return kScratchBytes; }

int ssim_loss_and_grad_noalloc(const void* img1, const void* img2, int dtype, int64_t N,
                               int64_t C, int64_t H, int64_t W, int padding, const float* dloss,
                               float* loss, void* grad_img1, void* grad_img2, void* stream) {
  if (!loss) return SSIM_ERR_NULL;
  // every shape the step accepts needs one accumulator (a Workspace) of
  // scratch, whatever its size; a larger need would be refused here
  if (sizeof(Workspace) > kScratchBytes) return SSIM_ERR_SCRATCH;
  return recompute_impl(dloss, img1, img2, dtype, N, C, H, W, padding, loss, nullptr, grad_img1,
                        grad_img2, stream, nullptr, true);
}

int ssim_grad_scale(const float* dloss, const float* grad, float* out, int64_t n, void* stream) {
  if (n < 0) return SSIM_ERR_SHAPE;
  if (n == 0) return SSIM_OK;
  if (!dloss || !grad || !out) return SSIM_ERR_NULL;
  if (n > INT64_MAX / 4) return SSIM_ERR_OVERFLOW;
  if (((uintptr_t)grad | (uintptr_t)out | (uintptr_t)dloss) % 4 != 0) return SSIM_ERR_SHAPE;
  const size_t bytes = (size_t)n * 4;
  if ((const void*)out != (const void*)grad && overlaps(out, bytes, grad, bytes))
    return SSIM_ERR_ALIAS;
  // every thread reads *dloss while others write out: it must not lie in out
  if (overlaps(out, bytes, dloss, sizeof(float))) return SSIM_ERR_ALIAS;
  const DeviceInfo* d = nullptr;
  const int rc = device_info(&d);
  if (rc != SSIM_OK) return rc;
  const bool vec = ((uintptr_t)grad | (uintptr_t)out) % 16 == 0;
  const int64_t units = vec ? (n >> 2) + (n & 3) : n;
  int64_t G = (units + kScaleThreads - 1) / kScaleThreads;
  const int64_t cap = (int64_t)d->cus * 8;
  if (G > cap) G = cap;
  if (G < 1) G = 1;
  const hipStream_t st = (hipStream_t)stream;
  if (vec)
    ssim_grad_scale_kernel<true><<<dim3((unsigned)G), dim3(kScaleThreads), 0, st>>>(dloss, grad,
                                                                                     out, n);
  else
    ssim_grad_scale_kernel<false><<<dim3((unsigned)G), dim3(kScaleThreads), 0, st>>>(dloss, grad,
                                                                                      out, n);
  return hipGetLastError() == hipSuccess ? SSIM_OK : SSIM_ERR_HIP;
}

size_t ssim_reference_bytes(int64_t N, int64_t C, int64_t H, int64_t W, int padding) {
  Shape s;
  if (check_shape(N, C, H, W, padding, SSIM_DTYPE_F32, &s) != SSIM_OK) return 0;
  return s.map_bytes / 4;
}

int ssim_reference_stats(const void* img2, int dtype, int64_t N, int64_t C, int64_t H, int64_t W,
                         int padding, float* ref, void* stream) {
  return ref_stats_impl(img2, dtype, N, C, H, W, padding, ref, stream);
}

int ssim_loss_and_grad_ref(const void* img1, const void* img2, const float* ref, int dtype,
                           int64_t N, int64_t C, int64_t H, int64_t W, int padding,
                           const float* dloss, float* loss, void* workspace, void* grad_img1,
                           void* stream) {
  if (!loss || !ref) return SSIM_ERR_NULL;
  return recompute_impl(dloss, img1, img2, dtype, N, C, H, W, padding, loss, workspace, grad_img1,
                        nullptr, stream, ref);
}

int ssim3d_map_shape(int64_t D, int64_t H, int64_t W, int padding, int64_t* Do, int64_t* Ho,
                     int64_t* Wo) {
  if (!Do || !Ho || !Wo) return SSIM_ERR_NULL;
  Shape3 s;
  const int rc = check_shape3(1, 1, D, H, W, padding, SSIM_DTYPE_F32, &s);
  if (rc != SSIM_OK) return rc;
  *Do = s.Do;
  *Ho = s.Ho;
  *Wo = s.Wo;
  return SSIM_OK;
}

size_t ssim3d_saved_maps_bytes(int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                               int padding) {
  Shape3 s;
  if (check_shape3(N, C, D, H, W, padding, SSIM_DTYPE_F32, &s) != SSIM_OK) return 0;
  return s.map_bytes;
}

int ssim3d_forward(const void* img1, const void* img2, int dtype, int64_t N, int64_t C, int64_t D,
                   int64_t H, int64_t W, int padding, float* loss, float* saved_maps,
                   void* workspace, void* stream) {
  return vol_forward_impl(img1, img2, dtype, N, C, D, H, W, padding, loss, saved_maps, workspace,
                          stream);
}

int ssim3d_backward(const float* dloss, const void* img1, const void* img2, int dtype, int64_t N,
                    int64_t C, int64_t D, int64_t H, int64_t W, int padding,
                    const float* saved_maps, void* grad_img1, void* grad_img2, void* stream) {
  return vol_backward_impl(dloss, img1, img2, dtype, N, C, D, H, W, padding, saved_maps,
                           grad_img1, grad_img2, stream);
}

}  // extern "C"
