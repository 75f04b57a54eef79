// fa_bwd256.hip -- the attention backward at head dimension 256 (the head
// dimension "FlashAttention-2 on Ascend NPU" (2048ai.net) names among its
// tiling parameters).  The kernels of fa_bwd_kernels.h instantiated at
// D = 256: one workgroup of four waves per CU, the dK^T/dV^T (or dQ^T)
// accumulators of a wave's 32 rows x 256 columns in its 256 AGPRs.  Built
// without the VGPR form of the MFMA instructions, which would put those
// accumulators in the 256 VGPRs beside everything else.
#include "fa_bwd_kernels.h"

namespace fa {
namespace bwd {

hipError_t launch_bwd256(const BwdParams& p, int dtype, int causal, hipStream_t stream) {
    if (dtype == 0) return causal ? run<256, 0, true>(p, stream) : run<256, 0, false>(p, stream);
    return causal ? run<256, 1, true>(p, stream) : run<256, 1, false>(p, stream);
}

}  // namespace bwd
}  // namespace fa
