// attn_bwd256.hip - the attention backward kernels at d = 256 (see
// attn_bwd.hip for what they compute). A translation unit of their own: the
// other head dims are built with the MFMA accumulators forced into VGPRs,
// and at d = 256 the key-side kernel's two 128-register accumulators must
// live in AGPRs (one wave a SIMD, 512 registers).
#include "attn_bwd_kernels.h"

namespace mi_attn {

hipError_t launch_bwd_d256(const BwdArgs& a, bool causal, bool f16) {
  if (f16) return causal ? launch_bwd<_Float16, 256, true, 4>(a) : launch_bwd<_Float16, 256, false, 4>(a);
  return causal ? launch_bwd<__bf16, 256, true, 4>(a) : launch_bwd<__bf16, 256, false, 4>(a);
}

}  // namespace mi_attn
