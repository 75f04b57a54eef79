// fa_ext.h -- internal interface of the forward with an explicit boolean mask
// and dropout.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {
namespace ext {

struct ExtParams {
    const void* q;          // [BH, Sq, D] contiguous
    const void* k;          // [BH, Sk, D]
    const void* v;          // [BH, Sk, D]
    void* o;                // [BH, Sq, D]
    float* lse;             // [BH, Sq] or null
    const uint8_t* mask;    // nonzero = keep; null = no mask
    int64_t m_sb, m_sh, m_ss;  // mask strides in bytes (batch, head, row); multiples of 4
    int Sq, Sk, H, BH, nqb;
    float scale_log2e;
    uint32_t drop_t;        // keep iff the 16-bit draw >= drop_t (0 = no dropout)
    float keep_scale;       // 65536 / (65536 - drop_t)
    uint32_t seed_lo, seed_hi, offset;
};

constexpr int kQueryBlock = 128;   // queries per workgroup (32 per wave)
constexpr int kKeyTile = 64;       // keys per K/V tile

hipError_t launch_ext(const ExtParams& p, int D, int dtype, int causal, hipStream_t stream);

}  // namespace ext
}  // namespace fa
