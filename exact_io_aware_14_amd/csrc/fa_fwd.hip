// Forward exact attention: the launches at d = 64 and 128 (the kernel and
// its method are in fa_fwd_kernel.h; d = 256 launches in fa_fwd_w.hip).
#include "fa_fwd_kernel.h"

namespace fa {
namespace {

template <typename TIn, typename TOut>
hipError_t launch_dtype(const FwdArgs& a) {
  if (a.bmask != nullptr) {  // block-sparse: bf16 only, always the masked kernel
    if (a.d == 64) return launch_typed<64, true, uint16_t, uint16_t, true>(a);
    if (a.d == 128) return launch_typed<128, true, uint16_t, uint16_t, true>(a);
    return launch_forward_wide_sparse(a);
  }
  if (a.d == 64) {
    return a.masked() ? launch_typed<64, true, TIn, TOut>(a) : launch_typed<64, false, TIn, TOut>(a);
  }
  if (a.d == 256) {
    return sizeof(TIn) == 2 ? launch_forward_wide_bf16(a) : launch_forward_wide_f32(a);
  }
  return a.masked() ? launch_typed<128, true, TIn, TOut>(a) : launch_typed<128, false, TIn, TOut>(a);
}

}  // namespace

hipError_t launch_forward_bf16(const FwdArgs& a) { return launch_dtype<uint16_t, uint16_t>(a); }
hipError_t launch_forward_f32(const FwdArgs& a) {
  if (a.bmask != nullptr) return hipErrorInvalidValue;  // block-sparse masks take bf16
  return launch_dtype<float, float>(a);
}

long long forward_grid_size(int B, int H, int N) {
  return (long long)B * H * ((N + kBR - 1) / kBR);
}

}  // namespace fa
