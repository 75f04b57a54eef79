// fa_launch.h -- internal interface between the host API and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

constexpr int kBlockQ = 256;           // query rows per workgroup (B_r): 8 waves x 32
constexpr int kBlockQSplit = 128;      // B_r of the key-split instance (both wave groups on 128 rows)
constexpr int kBlockKV = 64;            // keys per K/V tile (B_c)

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;        // [B, H, Sq] fp32, contiguous; may be null
    int Sq;            // query rows per head
    int Sk;            // key / value rows per head
    int H;             // heads (bh = b * H + h)
    int BH;            // batch * heads
    int nqb;           // query blocks per head: ceil(Sq / kBlockQ)
    int diag;          // causal instances: key j visible to query i iff j <= i + diag (in [-Sq, Sk])
    float scale_log2e; // scale * log2(e), fp32
    // Element strides of batch, head and row (the head dimension is contiguous).
    int64_t q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh;
    int q_ss, k_ss, v_ss, o_ss;
    // Optional boolean mask: element (b, h, i, j) at byte
    // b*m_sb + h*m_sh + i*m_ss + j, nonzero keeps the score.  Strides are
    // multiples of 4 and one head's rows span less than 2^31 bytes.
    const uint8_t* mask;   // null = no mask
    int64_t m_sb, m_sh;
    int m_ss;
    // Dropout (the DROP instances): score (bh, i, j) is kept iff half j%2 of
    // word (j%8)/2 of Philox4x32-10 at counter (j/8, i, bh, offset), key
    // (seed_lo, seed_hi), is >= drop_t (1..65535); kept probabilities are
    // scaled by keep_scale = 65536 / (65536 - drop_t).
    uint32_t drop_t;
    float keep_scale;
    uint32_t seed_lo, seed_hi, offset;
    // Diagnostic instances only (ignored by the others).
    int diag_flags;        // kDiagReverseOrder: workgroups take their blocks in reverse order
    float* o32;            // null, or fp32 O [B*H, Sq, D] contiguous
    uint32_t* tiles;       // null, or [grid][8]: tiles each wave ran its softmax on
};

constexpr int kDiagReverseOrder = 1;

// Enqueue the forward kernel (the masked instance when p.mask is set; the
// key-split instance when split, p.nqb counted in
// kBlockQSplit-row blocks); returns hipGetLastError() after the launch.
hipError_t launch_fwd(const FwdParams& p, int D, int dtype, bool causal, int64_t grid, bool split,
                      hipStream_t stream);
// The dropout instances (p.drop_t > 0; with the mask when p.mask is set) of
// the same kernel (fa_fwd_drop.hip).
hipError_t launch_fwd_drop(const FwdParams& p, int D, int dtype, bool causal, int64_t grid, bool split,
                           hipStream_t stream);
// The diagnostic instance (D = 64 or 128, no mask) of the same kernel.
hipError_t launch_fwd_diag(const FwdParams& p, int D, int dtype, bool causal, int64_t grid, bool split,
                           hipStream_t stream);

// Compute units of the current device, read once per device and cached
// (falls back to 256, MI355X's count, when no device can be queried).
int compute_units();

}  // namespace fa
