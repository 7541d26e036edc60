// The 16-head decode layout of attn_mfma_kernel (attn_kernel.h).  This file
// is compiled with -mllvm -amdgpu-mfma-vgpr-form=1: its matrix instructions
// accumulate in VGPRs, so the output accumulators and the logits share one
// register file and nothing is copied between VGPRs and AGPRs in the tile
// loop.
#include "attn_kernel.h"

namespace csa2 {

int launch_attn_decode(const AttnP& p, unsigned grid, int kv_dtype, hipStream_t st) {
    if (kv_dtype == DT_BF16)
        hipLaunchKernelGGL((attn_mfma_kernel<DT_BF16, 16>), dim3(grid), dim3(kThreads), 0, st, p);
    else if (kv_dtype == DT_E4M3)
        hipLaunchKernelGGL((attn_mfma_kernel<DT_E4M3, 16>), dim3(grid), dim3(kThreads), 0, st, p);
    else
        hipLaunchKernelGGL((attn_mfma_kernel<DT_FP4, 16>), dim3(grid), dim3(kThreads), 0, st, p);
    return static_cast<int>(hipGetLastError());
}

}  // namespace csa2
