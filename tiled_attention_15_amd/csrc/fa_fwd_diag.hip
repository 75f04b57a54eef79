// fa_fwd_diag.hip -- the diagnostic (test-only) instances of the fused
// forward: the kernel of fa_fwd_kernel.h with its DIAG switch on (reversed
// workgroup order on request, per-wave tile counts, fp32 copy of O).  The
// arithmetic of every step is that of the product instances.
#include "fa_fwd_kernel.h"

namespace fa {

template <int D, int DT, bool CAUSAL>
static hipError_t launch_diag_kernel(const FwdParams& p, int64_t grid, bool split, hipStream_t stream) {
    if (split)
        hipLaunchKernelGGL((fa_fwd_kernel<D, DT, CAUSAL, false, true, true>), dim3((unsigned)grid), dim3(512), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((fa_fwd_kernel<D, DT, CAUSAL, false, false, true>), dim3((unsigned)grid), dim3(512), 0,
                           stream, p);
    return hipGetLastError();
}

template <int D, int DT>
static hipError_t launch_diag_c(const FwdParams& p, bool causal, int64_t grid, bool split, hipStream_t s) {
    return causal ? launch_diag_kernel<D, DT, true>(p, grid, split, s) : launch_diag_kernel<D, DT, false>(p, grid, split, s);
}

hipError_t launch_fwd_diag(const FwdParams& p, int D, int dtype, bool causal, int64_t grid, bool split,
                           hipStream_t stream) {
    if (D == 64) return dtype == 0 ? launch_diag_c<64, 0>(p, causal, grid, split, stream)
                                   : launch_diag_c<64, 1>(p, causal, grid, split, stream);
    return dtype == 0 ? launch_diag_c<128, 0>(p, causal, grid, split, stream)
                      : launch_diag_c<128, 1>(p, causal, grid, split, stream);
}

}  // namespace fa
