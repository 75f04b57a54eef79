// fa_ext.h -- internal interface of the forward with an explicit boolean mask
// and dropout.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {
namespace ext {

struct ExtParams {
    const void* q;          // [B, H, Sq, D] with the element strides below (head dimension contiguous)
    const void* k;          // [B, H, Sk, D]
    const void* v;          // [B, H, Sk, D]
    void* o;                // [B, H, Sq, D]
    float* lse;             // [B*H, Sq] contiguous, or null
    int64_t q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh;   // batch and head strides
    int q_ss, k_ss, v_ss, o_ss;                                 // row strides
    const uint8_t* mask;    // nonzero = keep; null = no mask
    int64_t m_sb, m_sh, m_ss;  // mask strides in bytes (batch, head, row); multiples of 4
    int Sq, Sk, H, BH, nqb;
    int diag;               // causal: key j visible to query i iff j <= i + diag (in [-Sq, Sk])
    float scale_log2e;
    uint32_t drop_t;        // keep iff the 16-bit draw >= drop_t (0 = no dropout)
    float keep_scale;       // 65536 / (65536 - drop_t)
    uint32_t seed_lo, seed_hi, offset;
};

constexpr int kQueryBlock = 128;   // queries per workgroup (32 per wave)
// keys per K/V tile: 64, or 32 at D = 256 (the staged tile and its LDS
// double buffer stay at 32 KiB and 64 KiB)
constexpr int key_tile(int D) { return D == 256 ? 32 : 64; }

hipError_t launch_ext(const ExtParams& p, int D, int dtype, int causal, hipStream_t stream);

}  // namespace ext
}  // namespace fa
