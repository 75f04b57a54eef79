// fa_naive.h -- internal interface of the unfused comparison path.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {
namespace naive {

struct NaiveParams {
    const void* q;     // [BH, Sq, D] contiguous
    const void* k;     // [BH, Sk, D]
    const void* v;     // [BH, Sk, D]
    void* o;           // [BH, Sq, D]
    float* lse;        // [BH, Sq] or null
    float* s;          // workspace: scores, [BH, Sq, Skp] fp32
    uint16_t* p;       // workspace: probabilities, [BH, Sq, Skp] of the input dtype
    uint16_t* vt;      // workspace: V^T, [BH, D, Skp]
    int Sq, Sk, Skp;   // Skp = Sk rounded up to a multiple of 64
    int causal;
    float scale;
};

hipError_t launch_naive(const NaiveParams& p, int BH, int D, int dtype, hipStream_t stream);

}  // namespace naive
}  // namespace fa
