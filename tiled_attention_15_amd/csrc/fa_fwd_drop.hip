// fa_fwd_drop.hip -- launchers of the dropout instances of the fused
// attention forward (the kernel template is in fa_fwd_kernel.h): one
// instance per head dimension, dtype, causal flag, mask and key split, with
// the Philox4x32-10 keep decisions drawn in the softmax phase.
#include "fa_fwd_kernel.h"

namespace fa {

template <int D, int DT, bool CAUSAL>
static hipError_t launch_drop_kernel(const FwdParams& p, int64_t grid, bool split, hipStream_t stream) {
    const dim3 g((unsigned)grid), b(512);
    if constexpr (D == 256) {
        // the head-dimension split; no key-split instance
        if (p.mask != nullptr)
            hipLaunchKernelGGL((fa_fwd_kernel<D, DT, CAUSAL, true, false, false, true>), g, b, 0, stream, p);
        else
            hipLaunchKernelGGL((fa_fwd_kernel<D, DT, CAUSAL, false, false, false, true>), g, b, 0, stream, p);
    } else {
        if (p.mask != nullptr && split)
            hipLaunchKernelGGL((fa_fwd_kernel<D, DT, CAUSAL, true, true, false, true>), g, b, 0, stream, p);
        else if (p.mask != nullptr)
            hipLaunchKernelGGL((fa_fwd_kernel<D, DT, CAUSAL, true, false, false, true>), g, b, 0, stream, p);
        else if (split)
            hipLaunchKernelGGL((fa_fwd_kernel<D, DT, CAUSAL, false, true, false, true>), g, b, 0, stream, p);
        else
            hipLaunchKernelGGL((fa_fwd_kernel<D, DT, CAUSAL, false, false, false, true>), g, b, 0, stream, p);
    }
    return hipGetLastError();
}

template <int D, int DT>
static hipError_t launch_c(const FwdParams& p, bool causal, int64_t grid, bool split, hipStream_t s) {
    return causal ? launch_drop_kernel<D, DT, true>(p, grid, split, s)
                  : launch_drop_kernel<D, DT, false>(p, grid, split, s);
}

hipError_t launch_fwd_drop(const FwdParams& p, int D, int dtype, bool causal, int64_t grid, bool split,
                           hipStream_t stream) {
    if (D == 256) return dtype == 0 ? launch_c<256, 0>(p, causal, grid, false, stream)
                                    : launch_c<256, 1>(p, causal, grid, false, stream);
    if (D == 64) return dtype == 0 ? launch_c<64, 0>(p, causal, grid, split, stream)
                                   : launch_c<64, 1>(p, causal, grid, split, stream);
    return dtype == 0 ? launch_c<128, 0>(p, causal, grid, split, stream)
                      : launch_c<128, 1>(p, causal, grid, split, stream);
}

}  // namespace fa
