// Forward exact attention at head dimension 256: the launches (the kernel
// and its method are in fa_fwd_kernel.h).
//
// Compiled with LLVM's "amdgpu-mfma-vgpr-form" option: where a d = 256 wave
// has the SIMD's whole register file (64-key tiles: fp32 inputs), MFMA
// results kept in VGPRs where they fit (57 AGPRs instead of 162) made the
// launch about 7% faster (0.39 against 0.42 ms at B=4, H=8, N=4096, causal,
// when bf16 inputs took that design too), with bitwise the same results; the
// 32-key kernels (bf16 inputs) use no AGPRs either way. The d = 64 / 128 forward and the backward kernels are as fast
// or faster without it, hence the separate file.
#include "fa_fwd_kernel.h"

namespace fa {

hipError_t launch_forward_wide_bf16(const FwdArgs& a) {
  return a.masked() ? launch_typed<256, true, uint16_t, uint16_t>(a)
                    : launch_typed<256, false, uint16_t, uint16_t>(a);
}

hipError_t launch_forward_wide_sparse(const FwdArgs& a) {
  return launch_typed<256, true, uint16_t, uint16_t, true>(a);
}

hipError_t launch_forward_wide_f32(const FwdArgs& a) {
  return a.masked() ? launch_typed<256, true, float, float>(a)
                    : launch_typed<256, false, float, float>(a);
}

}  // namespace fa
