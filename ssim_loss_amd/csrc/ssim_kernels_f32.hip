// Entry kernels of the fused SSIM loss for fp32 images and gradients (the
// arithmetic is fp32 throughout; see ssim_device.hpp and ssim_fused.hpp).
#include "ssim_entry.hpp"

SSIM_ENTRY_KERNELS(ssim_dev::kImgF32, _, ssim_kernel_table_f32)
