// fa_fwd_kernel.hip -- launchers of the fused attention forward (the kernel
// template is in fa_fwd_kernel.h): one instance per head dimension, dtype,
// causal flag, mask and key split.
#include "fa_fwd_kernel.h"

namespace fa {

template <int D, int DT, bool CAUSAL>
static hipError_t launch_kernel(const FwdParams& p, int64_t grid, bool split, hipStream_t stream) {
    if (p.mask != nullptr && split)
        hipLaunchKernelGGL((fa_fwd_kernel<D, DT, CAUSAL, true, true>), dim3((unsigned)grid), dim3(512), 0, stream, p);
    else if (p.mask != nullptr)
        hipLaunchKernelGGL((fa_fwd_kernel<D, DT, CAUSAL, true, false>), dim3((unsigned)grid), dim3(512), 0, stream, p);
    else if (split)
        hipLaunchKernelGGL((fa_fwd_kernel<D, DT, CAUSAL, false, true>), dim3((unsigned)grid), dim3(512), 0, stream, p);
    else
        hipLaunchKernelGGL((fa_fwd_kernel<D, DT, CAUSAL, false, false>), dim3((unsigned)grid), dim3(512), 0, stream, p);
    return hipGetLastError();
}

template <int D, int DT>
static hipError_t launch_c(const FwdParams& p, bool causal, int64_t grid, bool split, hipStream_t s) {
    return causal ? launch_kernel<D, DT, true>(p, grid, split, s) : launch_kernel<D, DT, false>(p, grid, split, s);
}

template <int DT, bool CAUSAL>
static hipError_t launch_d256c(const FwdParams& p, int64_t grid, hipStream_t stream) {
    if (p.mask != nullptr)
        hipLaunchKernelGGL((fa_fwd_kernel<256, DT, CAUSAL, true, false>), dim3((unsigned)grid), dim3(512), 0, stream, p);
    else
        hipLaunchKernelGGL((fa_fwd_kernel<256, DT, CAUSAL, false, false>), dim3((unsigned)grid), dim3(512), 0, stream, p);
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_d256(const FwdParams& p, bool causal, int64_t grid, hipStream_t stream) {
    return causal ? launch_d256c<DT, true>(p, grid, stream) : launch_d256c<DT, false>(p, grid, stream);
}

hipError_t launch_fwd(const FwdParams& p, int D, int dtype, bool causal, int64_t grid, bool split,
                      hipStream_t stream) {
    if (D == 256) return dtype == 0 ? launch_d256<0>(p, causal, grid, stream) : launch_d256<1>(p, causal, grid, stream);
    if (D == 64) return dtype == 0 ? launch_c<64, 0>(p, causal, grid, split, stream)
                                   : launch_c<64, 1>(p, causal, grid, split, stream);
    return dtype == 0 ? launch_c<128, 0>(p, causal, grid, split, stream)
                      : launch_c<128, 1>(p, causal, grid, split, stream);
}

}  // namespace fa
