// fa_bwd.h -- internal interface of the attention backward kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {
namespace bwd {

// Layout of one [B, H, S, D] tensor: element strides of batch, head and row
// (the head dimension contiguous).
struct Lay {
    int64_t sb, sh;
    int ss;
};

struct BwdParams {
    const void* q;      // [B, H, Sq, D] (layout Lq), input dtype
    const void* k;      // [B, H, Sk, D]
    const void* v;      // [B, H, Sk, D]
    const void* o;      // [B, H, Sq, D]  forward output
    const void* dout;   // [B, H, Sq, D]  gradient of the output
    const float* lse;   // [BH, Sq]     forward row log-sum-exp (natural log)
    void* dq;           // [B, H, Sq, D]
    void* dk;           // [B, H, Sk, D]
    void* dv;           // [B, H, Sk, D]
    Lay Lq, Lk, Lv, Lo, Ldo, Ldq, Ldk, Ldv;   // layouts of q, k, v, o, dout, dq, dk, dv
    float* dvec;        // workspace [BH, Sq]: rowsum(dout * o)
    const uint8_t* mask;    // nonzero = keep, null = no mask
    int64_t m_sb, m_sh, m_ss;  // mask strides in bytes (batch, head, row)
    uint32_t drop_t;        // dropout: keep iff the 16-bit Philox draw >= drop_t (0 = none)
    float keep_scale;       // 65536 / (65536 - drop_t)
    uint32_t seed_lo, seed_hi, offset;
    int H;
    int Sq, Sk, BH;
    int diag;           // causal: key j visible to query i iff j <= i + diag (in [-Sq, Sk])
    int nkb;            // key blocks of the dK/dV kernel per head
    int nqb;            // query blocks of the dQ kernel per head
    float scale;        // softmax scale
    float scale_log2e;  // scale * log2(e)
};

constexpr int kKeyBlock = 128;   // keys per dK/dV workgroup (32 per wave)
constexpr int kQueryTile = 32;   // queries per step of the dK/dV kernel
constexpr int kQueryBlock = 128; // queries per dQ workgroup (32 per wave)
constexpr int kKeyTile = 64;     // keys per step of the dQ kernel

// Enqueue the backward on `stream`: row dot products, the dK/dV kernel, then
// the dQ kernel.
hipError_t launch_bwd(const BwdParams& p, int D, int dtype, int causal, hipStream_t stream);
// The same at D = 256 (fa_bwd256.hip).
hipError_t launch_bwd256(const BwdParams& p, int dtype, int causal, hipStream_t stream);

}  // namespace bwd
}  // namespace fa
