// fa_clock.hip -- shader-clock stamps for measuring the clock a run delivers.
//
// One thread per workgroup records the id of the XCD it runs on, the
// shader-clock counter and the fixed 100 MHz real-time counter.  Two launches
// on the stream a timed region runs on, one before and one after it, give
// each XCD's average shader clock over the region:
//   (shader ticks after - before) / (real-time ticks after - before) * 100 MHz.
// Launch with a few hundred workgroups so that every XCD holds some.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa.h"

namespace fa {

__global__ void clock_stamp_kernel(uint64_t* out) {
    if (threadIdx.x == 0) {
        uint32_t xcc;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
        const uint64_t t = __builtin_amdgcn_s_memtime();
        const uint64_t r = __builtin_amdgcn_s_memrealtime();
        uint64_t* o = out + 4 * (uint64_t)blockIdx.x;
        o[0] = xcc & 0xF;
        o[1] = t;
        o[2] = r;
        o[3] = 0;
    }
}

}  // namespace fa

extern "C" int fa_clock_stamps(uint64_t* out, int groups, void* stream) {
    if (out == nullptr) return FA_ERR_NULL;
    if (groups < 1 || groups > 65536) return FA_ERR_SHAPE;
    if ((uintptr_t)out & 15) return FA_ERR_ALIGN;
    hipLaunchKernelGGL(fa::clock_stamp_kernel, dim3((unsigned)groups), dim3(64), 0, (hipStream_t)stream, out);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}
