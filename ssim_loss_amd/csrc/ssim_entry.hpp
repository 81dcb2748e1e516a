// ssim_entry.hpp -- the entry kernels, one set per image type, and the table
// the host launches them from.  Each ssim_kernels_<type>.hip instantiates the
// set for one type with SSIM_ENTRY_KERNELS; ssim_api.hip sees the KernelKind
// order and the table accessors only.  Kernels are named for profiles:
// "stream" kernels mark their stores non-temporal; "unaligned" kernels move
// image elements one at a time (W not a multiple of 4, or unaligned
// pointers).

#pragma once

#include "ssim_fused.hpp"
#include "ssim_vol.hpp"

namespace ssim_dev {
// threads per workgroup of each kernel kind: the recomputing kernels run two
// groups of 4 waves (one per stencil stage)
enum KernelKind {
  kKFwdInfer,          // forward, loss only
  kKFwdTrain,          // forward, loss + saved statistics
  kKFwdTrainStream,
  kKBwd,               // backward from the saved statistics
  kKBwdStream,
  kKBwdUnaligned,
  kKRecomp,            // backward recomputing the statistics from the images
  kKRecompStream,
  kKRecompUnaligned,
  kKLossGrad,          // loss and both gradients in one pass
  kKLossGradStream,
  kKLossGradUnaligned,
  kKLossGradRef,       // loss and grad_x in one pass, with cached reference statistics
  kKLossGradRefStream,
  kKLossGradRefUnaligned,
  kKRecompX,           // the recomputing backward and the one-pass step forming
  kKRecompXStream,     // grad_x alone or grad_y alone (the other pointer NULL);
  kKRecompY,           // the unaligned case uses the both-gradient kernels
  kKRecompYStream,
  kKLossGradX,
  kKLossGradXStream,
  kKLossGradY,
  kKLossGradYStream,
  kKRefStats,          // the cached reference statistics of an image
  kKVolFwdInfer,       // volumes: forward, loss only
  kKVolFwdTrain,       // volumes: forward, loss + saved partials
  kKVolBwd,            // volumes: backward from the saved partials
  kKinds
};
__host__ __device__ constexpr int kind_threads(int k) {
  return (k >= kKRecomp && k <= kKLossGradYStream) ? kFThreads
         : k >= kKVolFwdInfer                           ? kVThreads
                                                        : kThreads;
}
// the parameter block each kind takes
__host__ __device__ constexpr bool kind_is_volume(int k) { return k >= kKVolFwdInfer; }
}  // namespace ssim_dev

#define SSIM_KERNEL_(NAME, BODY)                                                           \
  __global__ __launch_bounds__(ssim_dev::kThreads) void NAME(const ssim_dev::Params p) {   \
    BODY(p);                                                                               \
  }
// 8-wave workgroups: two per CU need at most 128 VGPRs (4 waves per SIMD)
#define SSIM_FKERNEL_(NAME, BODY)                                                          \
  __global__ __launch_bounds__(ssim_dev::kFThreads) __attribute__((amdgpu_waves_per_eu(4))) \
  void NAME(const ssim_dev::Params p) {                                                    \
    BODY(p);                                                                               \
  }

// the volume kernels' working set is a 44-register depth window and a few
// LDS reads in flight; without an occupancy target the scheduler hoists
// reads into registers far past that
#define SSIM_VKERNEL_(NAME, WAVES, BODY)                                                   \
  __global__ __launch_bounds__(ssim_dev::kVThreads) __attribute__((amdgpu_waves_per_eu(WAVES))) \
  void NAME(const ssim_dev::VolParams p) {                                                 \
    BODY(p);                                                                               \
  }

#define SSIM_ENTRY_KERNELS(T, NAME, TABLE)                                                  \
  namespace {                                                                              \
  SSIM_KERNEL_(ssim_fwd_infer##NAME##kernel,                                               \
               (ssim_dev::strip_body<ssim_dev::kFwdInfer, false, false, T>))               \
  SSIM_KERNEL_(ssim_fwd_train##NAME##kernel,                                               \
               (ssim_dev::strip_body<ssim_dev::kFwdTrain, false, false, T>))               \
  SSIM_KERNEL_(ssim_fwd_train_stream##NAME##kernel,                                        \
               (ssim_dev::strip_body<ssim_dev::kFwdTrain, false, true, T>))                \
  SSIM_KERNEL_(ssim_bwd##NAME##kernel, (ssim_dev::strip_body<ssim_dev::kBwd, true, false, T>)) \
  SSIM_KERNEL_(ssim_bwd_stream##NAME##kernel,                                              \
               (ssim_dev::strip_body<ssim_dev::kBwd, true, true, T>))                      \
  SSIM_KERNEL_(ssim_bwd_unaligned##NAME##kernel,                                           \
               (ssim_dev::strip_body<ssim_dev::kBwd, false, false, T>))                    \
  SSIM_FKERNEL_(ssim_bwd_recompute##NAME##kernel, (ssim_dev::fused_body<false, true, false, T>)) \
  SSIM_FKERNEL_(ssim_bwd_recompute_stream##NAME##kernel,                                    \
               (ssim_dev::fused_body<false, true, true, T>))                               \
  SSIM_FKERNEL_(ssim_bwd_recompute_unaligned##NAME##kernel,                                 \
               (ssim_dev::fused_body<false, false, false, T>))                             \
  SSIM_FKERNEL_(ssim_loss_grad##NAME##kernel, (ssim_dev::fused_body<true, true, false, T>))  \
  SSIM_FKERNEL_(ssim_loss_grad_stream##NAME##kernel,                                        \
               (ssim_dev::fused_body<true, true, true, T>))                                 \
  SSIM_FKERNEL_(ssim_loss_grad_unaligned##NAME##kernel,                                     \
               (ssim_dev::fused_body<true, false, false, T>))                              \
  SSIM_FKERNEL_(ssim_loss_grad_ref##NAME##kernel,                                          \
                (ssim_dev::fused_body<true, true, false, T, true>))                        \
  SSIM_FKERNEL_(ssim_loss_grad_ref_stream##NAME##kernel,                                   \
                (ssim_dev::fused_body<true, true, true, T, true>))                         \
  SSIM_FKERNEL_(ssim_loss_grad_ref_unaligned##NAME##kernel,                                \
                (ssim_dev::fused_body<true, false, false, T, true>))                       \
  SSIM_FKERNEL_(ssim_bwd_recompute_x##NAME##kernel,                                         \
                (ssim_dev::fused_body<false, true, false, T, false, ssim_dev::kOnlyX>))     \
  SSIM_FKERNEL_(ssim_bwd_recompute_x_stream##NAME##kernel,                                  \
                (ssim_dev::fused_body<false, true, true, T, false, ssim_dev::kOnlyX>))      \
  SSIM_FKERNEL_(ssim_bwd_recompute_y##NAME##kernel,                                         \
                (ssim_dev::fused_body<false, true, false, T, false, ssim_dev::kOnlyY>))     \
  SSIM_FKERNEL_(ssim_bwd_recompute_y_stream##NAME##kernel,                                  \
                (ssim_dev::fused_body<false, true, true, T, false, ssim_dev::kOnlyY>))      \
  SSIM_FKERNEL_(ssim_loss_grad_x##NAME##kernel,                                             \
                (ssim_dev::fused_body<true, true, false, T, false, ssim_dev::kOnlyX>))      \
  SSIM_FKERNEL_(ssim_loss_grad_x_stream##NAME##kernel,                                      \
                (ssim_dev::fused_body<true, true, true, T, false, ssim_dev::kOnlyX>))       \
  SSIM_FKERNEL_(ssim_loss_grad_y##NAME##kernel,                                             \
                (ssim_dev::fused_body<true, true, false, T, false, ssim_dev::kOnlyY>))      \
  SSIM_FKERNEL_(ssim_loss_grad_y_stream##NAME##kernel,                                      \
                (ssim_dev::fused_body<true, true, true, T, false, ssim_dev::kOnlyY>))       \
  SSIM_KERNEL_(ssim_ref_stats##NAME##kernel,                                               \
               (ssim_dev::strip_body<ssim_dev::kRef, false, false, T>))                    \
  SSIM_VKERNEL_(ssim3d_fwd_infer##NAME##kernel, 4,                                         \
                (ssim_dev::vol_body<ssim_dev::kFwdInfer, false, T>))                        \
  SSIM_VKERNEL_(ssim3d_fwd_train##NAME##kernel, 4,                                         \
                (ssim_dev::vol_body<ssim_dev::kFwdTrain, false, T>))                        \
  SSIM_VKERNEL_(ssim3d_bwd##NAME##kernel, 4, (ssim_dev::vol_body<ssim_dev::kBwd, false, T>)) \
  }                                                                                        \
  const void* const* TABLE() {                                                             \
    static const void* const t[ssim_dev::kKinds] = {                                      \
        (const void*)ssim_fwd_infer##NAME##kernel,                                         \
        (const void*)ssim_fwd_train##NAME##kernel,                                         \
        (const void*)ssim_fwd_train_stream##NAME##kernel,                                  \
        (const void*)ssim_bwd##NAME##kernel,                                               \
        (const void*)ssim_bwd_stream##NAME##kernel,                                        \
        (const void*)ssim_bwd_unaligned##NAME##kernel,                                     \
        (const void*)ssim_bwd_recompute##NAME##kernel,                                     \
        (const void*)ssim_bwd_recompute_stream##NAME##kernel,                              \
        (const void*)ssim_bwd_recompute_unaligned##NAME##kernel,                           \
        (const void*)ssim_loss_grad##NAME##kernel,                                         \
        (const void*)ssim_loss_grad_stream##NAME##kernel,                                  \
        (const void*)ssim_loss_grad_unaligned##NAME##kernel,                               \
        (const void*)ssim_loss_grad_ref##NAME##kernel,                                     \
        (const void*)ssim_loss_grad_ref_stream##NAME##kernel,                              \
        (const void*)ssim_loss_grad_ref_unaligned##NAME##kernel,                           \
        (const void*)ssim_bwd_recompute_x##NAME##kernel,                                   \
        (const void*)ssim_bwd_recompute_x_stream##NAME##kernel,                            \
        (const void*)ssim_bwd_recompute_y##NAME##kernel,                                   \
        (const void*)ssim_bwd_recompute_y_stream##NAME##kernel,                            \
        (const void*)ssim_loss_grad_x##NAME##kernel,                                       \
        (const void*)ssim_loss_grad_x_stream##NAME##kernel,                                \
        (const void*)ssim_loss_grad_y##NAME##kernel,                                       \
        (const void*)ssim_loss_grad_y_stream##NAME##kernel,                                \
        (const void*)ssim_ref_stats##NAME##kernel,                                         \
        (const void*)ssim3d_fwd_infer##NAME##kernel,                                       \
        (const void*)ssim3d_fwd_train##NAME##kernel,                                       \
        (const void*)ssim3d_bwd##NAME##kernel};                                            \
    return t;                                                                              \
  }

// Kernel tables exported by the per-type translation units.
const void* const* ssim_kernel_table_f32();
const void* const* ssim_kernel_table_f16();
const void* const* ssim_kernel_table_bf16();
