// fa_launch.h -- internal interface between the host API and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

constexpr int kBlockQ = 256;           // query rows per workgroup (B_r): 8 waves x 32
constexpr int kBlockKV = 64;            // keys per K/V tile (B_c)

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;        // may be null
    int S;             // sequence length
    int BH;            // batch * heads
    int nqb;           // query blocks per head: ceil(S / kBlockQ)
    float scale_log2e; // scale * log2(e), fp32
};

// Enqueue the forward kernel; returns hipGetLastError() after the launch.
hipError_t launch_fwd(const FwdParams& p, int D, int dtype, bool causal, int64_t grid,
                      hipStream_t stream);

}  // namespace fa
