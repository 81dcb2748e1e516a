/*
 * ssim_loss_amd.h -- C ABI of the fused SSIM loss (forward + backward) for
 * AMD Instinct MI355X (gfx950).
 *
 * The loss is  loss = 1 - mean SSIM  over every map entry of an NCHW batch
 * ("TriSSIM -- A Highly Optimized Triton-based Fused SSIM Library", Usage:
 * the train loss is one minus fused_ssim), where the SSIM map uses the 11x11
 * Gaussian window of the original SSIM paper ("Fully Fused Differentiable
 * SSIM", opening section: separable, symmetric, hard-coded weights; here
 * sigma 1.5, taps normalised to sum 1), C1 = 0.01^2, C2 = 0.03^2 (images in
 * [0,1]: "Fully Fused Differentiable SSIM", Constraints), and either "valid"
 * or zero-filled "same" padding ("Fully Fused Differentiable SSIM", Usage).
 * The backward applies the adjoint of the blur and the chain rule of
 * "TriSSIM", How it works.
 *
 * Conventions shared by every entry point:
 *   - Images, maps, gradients and loss are device pointers (HIP device
 *     memory) owned by the caller.  The library never allocates, frees or
 *     synchronises; all work is enqueued on `stream` (a hipStream_t; NULL is
 *     the default stream) and completes asynchronously.
 *   - Images are contiguous NCHW (fp32 for ssim_forward / ssim_backward,
 *     fp32, fp16 or bf16 for the _typed calls), N*C planes of H rows of W
 *     pixels, each pointer aligned to its element size.  img1 and img2 have
 *     the same shape.  Values are meant to lie in [0,1].
 *   - Outputs are overwritten, never accumulated into.
 *   - Every argument check happens before any HIP call; a failed check
 *     returns a negative code and enqueues nothing.  A launch failure
 *     returns SSIM_ERR_HIP.  Faults inside a kernel surface at the caller's
 *     next synchronisation, as HIP errors.  No C++ exception crosses the ABI.
 *   - Calls are reentrant.  Concurrent calls (on different streams) need
 *     distinct loss, saved_maps and workspace buffers.
 */
#ifndef SSIM_LOSS_AMD_H
#define SSIM_LOSS_AMD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSIM_ABI_VERSION 8

/* padding ("Fully Fused Differentiable SSIM", Usage) */
enum {
  SSIM_PAD_VALID = 0, /* map is (H-10) x (W-10): windows inside the image only */
  SSIM_PAD_SAME = 1   /* map is H x W: window centred, zeros outside the image */
};

/* return codes */
enum {
  SSIM_OK = 0,
  SSIM_ERR_NULL = -1,     /* a required pointer is NULL */
  SSIM_ERR_SHAPE = -2,    /* N, C, H or W <= 0, valid padding with H < 11 or W < 11, an
                             image or gradient pointer not aligned to its element size,
                             or saved_maps not 16-byte aligned */
  SSIM_ERR_PADDING = -3,  /* padding is neither SSIM_PAD_VALID nor SSIM_PAD_SAME */
  SSIM_ERR_OVERFLOW = -4, /* a plane (image, or map with its row pitch) holds more than
                             2^27 elements, a row more than 2^20, or a size overflows */
  SSIM_ERR_ALIAS = -5,    /* an output buffer overlaps an input or another output */
  SSIM_ERR_HIP = -6,      /* a HIP runtime call failed (launch, device query) */
  SSIM_ERR_DEVICE = -7,   /* the current device is not a wave64 gfx950 GPU */
  SSIM_ERR_DTYPE = -8,    /* dtype is not one of SSIM_DTYPE_* */
  SSIM_ERR_SCRATCH = -9   /* the call needs more scratch than the library's fixed device
                             array holds (ssim_loss_and_grad_noalloc) */
};

/* storage type of images and gradients for the _typed entry points; the
 * arithmetic is fp32 in every case and the saved maps are always fp32 */
enum {
  SSIM_DTYPE_F32 = 0,
  SSIM_DTYPE_F16 = 1, /* IEEE binary16 */
  SSIM_DTYPE_BF16 = 2 /* bfloat16 (the top 16 bits of an fp32); gradients rounded to nearest even */
};

/* Version of this ABI (SSIM_ABI_VERSION of the library that was built). */
int ssim_abi_version(void);

/* Static, human-readable text for a return code.  Never NULL. */
const char* ssim_strerror(int code);

/* The 11 one-dimensional Gaussian taps (fp32) the kernels use, copied to
 * `out` (host memory, 11 floats).  g[k] is proportional to
 * exp(-(k-5)^2 / (2 * 1.5^2)), normalised to sum 1, rounded once to fp32;
 * the 2-D window is g g^T.  Host-only; touches no GPU. */
void ssim_taps(float out[11]);

/* Output (map) extent for an H x W image: valid gives (H-10) x (W-10),
 * same gives H x W.  Returns SSIM_OK, or SSIM_ERR_SHAPE / SSIM_ERR_PADDING.
 * Host-only. */
int ssim_map_shape(int64_t H, int64_t W, int padding, int64_t* Ho, int64_t* Wo);

/* Bytes of the saved-maps buffer ssim_forward writes in training mode and
 * ssim_backward reads: four fp32 map planes per image plane, each Ho rows
 * with a row pitch of Wo rounded up to a multiple of 4 floats, i.e.
 * 16 * N*C * Ho * roundup(Wo, 4) bytes.  The buffer must be 16-byte
 * aligned.  Returns 0 for invalid arguments.  Host-only. */
size_t ssim_saved_maps_bytes(int64_t N, int64_t C, int64_t H, int64_t W, int padding);

/* Bytes of the workspace ssim_forward needs (the loss reduction's
 * accumulator: a fixed-point sum and a completion count in one 64-bit word).
 * The caller zero-fills it once, before its first use; every ssim_forward
 * leaves it ready for the next call (the last workgroup resets it).  One
 * workspace must not be used by two ssim_forward calls that may run at the
 * same time.  Host-only. */
size_t ssim_workspace_bytes(void);

/* Forward.  Computes loss = 1 - (1/M) * sum over the N*C*Ho*Wo map entries
 * of SSIM, M = N*C*Ho*Wo, and writes it as one fp32 to `loss` (device).
 *
 *   img1, img2  : fp32 NCHW device images (inputs, not modified)
 *   N, C, H, W  : shape; a plane holds at most 2^27 elements (its map
 *                 too, with Wo rounded up to 4) and a row at most 2^20;
 *                 N*C is unbounded
 *   padding     : SSIM_PAD_VALID or SSIM_PAD_SAME
 *   loss        : device fp32 scalar (output)
 *   saved_maps  : NULL for inference (no gradient will be taken), else a
 *                 device buffer of ssim_saved_maps_bytes(...) bytes that
 *                 receives the forward's state for ssim_backward.  Its
 *                 contents are opaque: only ssim_backward reads them, and
 *                 they change meaning between versions of this ABI.  (In this
 *                 version: at every map entry the four blurred quantities the
 *                 kernels form -- B(y), B(x - y), B((x - y)^2) and
 *                 B((x - 1/2)(y - 1/2)) -- one map plane each; ssim_backward
 *                 forms the loss partials from them.)
 *   workspace   : device buffer of ssim_workspace_bytes() bytes, zeroed
 *                 before its first use
 *   stream      : hipStream_t (NULL = default stream)
 *
 * The reduction is deterministic: the same inputs give the same bits.  A NaN
 * or infinite image value makes the loss NaN (and the workspace is still
 * left ready for the next call); every loss-forming entry point below does
 * the same. */
int ssim_forward(const float* img1, const float* img2, int64_t N, int64_t C, int64_t H,
                 int64_t W, int padding, float* loss, float* saved_maps, void* workspace,
                 void* stream);

/* Backward.  Writes grad_img1 = dloss * d loss / d img1 and
 * grad_img2 = dloss * d loss / d img2 (fp32 NCHW, same shape as the images)
 * by applying the adjoint of the blur to the saved maps and the chain rule
 * ("TriSSIM", How it works).
 *
 *   dloss       : device fp32 scalar, the upstream gradient of the loss
 *   img1, img2  : the images given to ssim_forward (unchanged since)
 *   N..padding  : as given to ssim_forward
 *   saved_maps  : the buffer ssim_forward filled (unchanged since)
 *   grad_img1   : device output, or NULL to skip it
 *   grad_img2   : device output, or NULL to skip it (both NULL: no-op)
 *   stream      : hipStream_t (NULL = default stream) */
int ssim_backward(const float* dloss, const float* img1, const float* img2, int64_t N,
                  int64_t C, int64_t H, int64_t W, int padding, const float* saved_maps,
                  float* grad_img1, float* grad_img2, void* stream);

/* Half-precision image I/O: ssim_forward / ssim_backward for images (and
 * gradients) stored as `dtype` (SSIM_DTYPE_F32, _F16 or _BF16), same shape
 * and layout rules, all arithmetic in fp32 and maps in fp32.  Elements are
 * widened exactly on load; gradients are rounded to nearest even on store.
 * fp32 calls behave exactly as ssim_forward / ssim_backward.  Halving the
 * image and gradient bytes is the point: a training step moves 44 bytes per
 * element instead of 56.  Returns SSIM_ERR_DTYPE for an unknown dtype. */
int ssim_forward_typed(const void* img1, const void* img2, int dtype, int64_t N, int64_t C,
                       int64_t H, int64_t W, int padding, float* loss, float* saved_maps,
                       void* workspace, void* stream);
int ssim_backward_typed(const float* dloss, const void* img1, const void* img2, int dtype,
                        int64_t N, int64_t C, int64_t H, int64_t W, int padding,
                        const float* saved_maps, void* grad_img1, void* grad_img2, void* stream);

/* Backward without saved maps.  Same result as ssim_backward (the adjoint of
 * the blur and the chain rule of "TriSSIM", How it works), but the blurred
 * statistics are formed again from the images instead of being read from a
 * forward's saved maps: pair it with an inference-mode ssim_forward
 * (saved_maps = NULL).  It moves only the images and the gradients through
 * HBM and needs no map buffer, at about twice the arithmetic.
 *
 *   dloss        : device fp32 scalar, the upstream gradient of the loss
 *   img1, img2   : device images of `dtype` (inputs)
 *   dtype, N..padding : as for ssim_forward_typed
 *   grad_img1/2  : device outputs of `dtype`, or NULL to skip (both NULL: no-op);
 *                  with exactly one NULL (and 16-byte aligned images, W a
 *                  multiple of 4) a kernel runs that forms the other gradient
 *                  alone, bit for bit the same, skipping the missing one's
 *                  partial and adjoint blur
 *   stream       : hipStream_t (NULL = default stream) */
int ssim_backward_recompute(const float* dloss, const void* img1, const void* img2, int dtype,
                            int64_t N, int64_t C, int64_t H, int64_t W, int padding,
                            void* grad_img1, void* grad_img2, void* stream);

/* Loss and gradients in one pass: the forward (loss = 1 - mean SSIM, as
 * ssim_forward) and the backward (as ssim_backward, scaled by *dloss) of one
 * training step in a single launch, for callers that know the upstream
 * gradient before the forward -- the weight of the SSIM term in a training
 * loss, or 1.  Reads the images once and writes the gradients; no map
 * buffer.
 *
 *   img1, img2   : device images of `dtype` (inputs)
 *   dtype, N..padding : as for ssim_forward_typed
 *   dloss        : device fp32 scalar, read before any gradient is formed
 *   loss         : device fp32 scalar (output; required)
 *   workspace    : as for ssim_forward (the same rules: zeroed once, not
 *                  shared by calls that may overlap)
 *   grad_img1/2  : device outputs of `dtype`, or NULL to skip; with exactly one
 *                  NULL (and 16-byte aligned images, W a multiple of 4) a
 *                  kernel runs that forms the other gradient alone, bit for
 *                  bit the same
 *   stream       : hipStream_t (NULL = default stream)
 * Deterministic, like ssim_forward; the loss equals ssim_forward's up to the
 * rounding of the summation (the two kernels split the map differently). */
int ssim_loss_and_grad(const void* img1, const void* img2, int dtype, int64_t N, int64_t C,
                       int64_t H, int64_t W, int padding, const float* dloss, float* loss,
                       void* workspace, void* grad_img1, void* grad_img2, void* stream);

/* Allocation-free variant of ssim_loss_and_grad, for callers that cannot
 * allocate device memory or own a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments and
 * result as ssim_loss_and_grad without `workspace`; the loss accumulator
 * lives instead in a device array inside the library,
 * ssim_noalloc_scratch_bytes() bytes on each GPU it runs on, held until the
 * process ends.  Every shape the step accepts needs one accumulator (8 bytes
 * used of that array), so no shape exceeds it; SSIM_ERR_SCRATCH would report
 * a need beyond it.  The call allocates nothing (no hipMalloc, no allocating
 * library routine); the first call on a device, with that device current,
 * looks up the array's address and clears the array with a small kernel on
 * `stream` ahead of its own launch.  Each launch leaves the accumulator at
 * zero when it completes.
 *
 * All calls on one GPU share that GPU's array: two calls that may run at the
 * same time on one GPU (different streams without ordering between them)
 * race on it and may both write a wrong loss.  Calls on one stream, or
 * ordered by events, are safe.
 *
 *   img1, img2   : device images of `dtype` (inputs)
 *   dtype, N..padding : as for ssim_forward_typed
 *   dloss        : device fp32 scalar, read before any gradient is formed
 *   loss         : device fp32 scalar (output; required)
 *   grad_img1/2  : device outputs of `dtype`, or NULL to skip
 *   stream       : hipStream_t (NULL = default stream)
 * Argument checks and codes as for ssim_loss_and_grad, all before any HIP
 * call. */
int ssim_loss_and_grad_noalloc(const void* img1, const void* img2, int dtype, int64_t N,
                               int64_t C, int64_t H, int64_t W, int padding, const float* dloss,
                               float* loss, void* grad_img1, void* grad_img2, void* stream);

/* Bytes of the per-GPU scratch array ssim_loss_and_grad_noalloc uses (256).
 * Host-only. */
size_t ssim_noalloc_scratch_bytes(void);

/* The chain rule's last factor, applied later: out[i] = *dloss * grad[i] for
 * 0 <= i < n, fp32.  "TriSSIM", How it works: the backward multiplies the
 * loss's own gradient by the upstream gradient.  A caller that does not know
 * the upstream gradient at the forward (an autograd step) runs
 * ssim_loss_and_grad there with *dloss = 1 and this call in the backward.
 * The kernels form a gradient as *dloss times an fp32 value, and with
 * *dloss = 1 they store that value exactly, so the result equals
 * ssim_loss_and_grad's with the same *dloss bit for bit (fp32 gradients; a
 * half-precision gradient would be rounded twice).
 *
 *   dloss  : device fp32 scalar, the upstream gradient
 *   grad   : device fp32 array of n elements (input), 4-byte aligned
 *   out    : device fp32 array of n elements (output, overwritten); may be
 *            grad itself (in place), must not otherwise overlap it, and must
 *            not contain dloss
 *   n      : element count; 0 launches nothing
 *   stream : hipStream_t (NULL = default stream)
 * Returns SSIM_ERR_SHAPE for n < 0 or a pointer not 4-byte aligned,
 * SSIM_ERR_NULL for a NULL pointer with n > 0, SSIM_ERR_OVERFLOW when 4 n
 * bytes overflow and SSIM_ERR_ALIAS for a partial overlap of out and grad or
 * for dloss inside out, all before any
 * HIP call; SSIM_ERR_DEVICE on a device that is not gfx950; SSIM_ERR_HIP if
 * the launch fails. */
int ssim_grad_scale(const float* dloss, const float* grad, float* out, int64_t n, void* stream);

/* ---------------------------------------------------------------------------
 * Cached reference statistics.  In a training run the second image is often
 * a fixed reference (the ground-truth view, with only the first image
 * differentiable: "Fully Fused Differentiable SSIM", Constraints).  Of the
 * statistics the kernels blur, B(y) depends on the reference alone; it
 * can be computed once per reference and reused by every step that compares
 * against it.  (The pages' SSIMULACRA2 port caches reference-side work the
 * same way; here it is the one reference-only statistic of the SSIM basis.)
 */

/* Bytes of the cached statistics of an N x C x H x W reference: one fp32
 * plane per image plane over the map, row pitch Wo rounded up to 4, i.e.
 * 4 * N*C * Ho * roundup(Wo, 4) bytes; 16-byte aligned.  0 for invalid
 * arguments.  Host-only. */
size_t ssim_reference_bytes(int64_t N, int64_t C, int64_t H, int64_t W, int padding);

/* Writes B(img2) (the reference's blurred mean) to `ref`
 * (device, ssim_reference_bytes(...) bytes).  img2: device image of
 * `dtype`.  The result is valid for that exact image, shape and padding. */
int ssim_reference_stats(const void* img2, int dtype, int64_t N, int64_t C, int64_t H, int64_t W,
                         int padding, float* ref, void* stream);

/* As ssim_loss_and_grad with grad_img2 = NULL, reading B(img2) from
 * `ref` (ssim_reference_stats of this img2) instead of forming it: loss =
 * 1 - mean SSIM and grad_img1 = *dloss * d loss / d img1 in one launch, one
 * blur fewer in each direction.  img2 is still read (the other statistics mix
 * both images).  grad_img1 may be NULL (loss only). */
int ssim_loss_and_grad_ref(const void* img1, const void* img2, const float* ref, int dtype,
                           int64_t N, int64_t C, int64_t H, int64_t W, int padding,
                           const float* dloss, float* loss, void* workspace, void* grad_img1,
                           void* stream);

/* ---------------------------------------------------------------------------
 * Volumes ("Fully Fused Differentiable SSIM", 3D data): NCDHW volumes, the
 * 11x11x11 window g g g (the same taps on every axis), the same constants,
 * SSIM formula and loss; valid padding shrinks every axis by 10, same keeps
 * it (zero fill).  Each volume (and its map) holds at most 2^27 elements;
 * N*C is unbounded.  Images and gradients are of `dtype`; arithmetic fp32.
 * Every argument check happens before any HIP call, with the 2-D codes.
 */

/* Map extent of a D x H x W volume.  Host-only. */
int ssim3d_map_shape(int64_t D, int64_t H, int64_t W, int padding, int64_t* Do, int64_t* Ho,
                     int64_t* Wo);

/* Bytes of the saved-maps buffer of a training-mode ssim3d_forward: the four
 * loss partials (fp32) at every map voxel, 16 * N*C * Do*Ho*Wo bytes, layout
 * [N*C][4][Do][Ho][Wo]; 16-byte aligned.  0 for invalid arguments. */
size_t ssim3d_saved_maps_bytes(int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                               int padding);

/* Forward: loss = 1 - mean SSIM over the N*C*Do*Ho*Wo map voxels, one fp32 to
 * `loss` (device).  saved_maps: NULL (inference) or a device buffer of
 * ssim3d_saved_maps_bytes(...) bytes that receives the loss partials for
 * ssim3d_backward.  workspace: as for ssim_forward.  Deterministic. */
int ssim3d_forward(const void* img1, const void* img2, int dtype, int64_t N, int64_t C, int64_t D,
                   int64_t H, int64_t W, int padding, float* loss, float* saved_maps,
                   void* workspace, void* stream);

/* Backward: grad_img1/2 = dloss * d loss / d img1/2 (device outputs of
 * `dtype`, either may be NULL) from the partials a training-mode
 * ssim3d_forward saved, by the adjoint of the 3-D blur and the chain rule
 * ("TriSSIM", How it works, on the 3-D window). */
int ssim3d_backward(const float* dloss, const void* img1, const void* img2, int dtype, int64_t N,
                    int64_t C, int64_t D, int64_t H, int64_t W, int padding,
                    const float* saved_maps, void* grad_img1, void* grad_img2, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSIM_LOSS_AMD_H */
