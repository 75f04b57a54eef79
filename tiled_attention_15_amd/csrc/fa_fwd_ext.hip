// fa_fwd_ext.hip -- fused attention forward with an explicit boolean mask and
// keep-and-rescale dropout, for gfx950 (MI355X).
//
// Mask and dropout are applied inside the attention kernel, on the score tile
// in registers, so neither a mask pass nor a dropout pass over an S x S
// matrix touches device memory ("FlashAttention-2 on Ascend NPU: how
// ops-transformer reaches 3x" (2048ai.net), section 3.4, and section 6.3).
// Semantics:
//   * a nonzero mask byte keeps the score, a zero byte hides it (as the
//     page's kernel treats a true entry); combined with the causal rule;
//   * dropout keeps each probability with probability 1 - t/65536 and scales
//     the kept ones by 65536 / (65536 - t); the row normaliser (and the lse)
//     is that of the undropped softmax.  The keep decision of score (bh, i, j)
//     compares half j%2 of word (j%8)/2 of Philox4x32-10 (Salmon et al.,
//     "Parallel random numbers: as easy as 1, 2, 3", SC 2011) at counter
//     (j/8, i, bh, offset) and key (seed low, seed high) with t, so any
//     implementation of the generator reproduces the pattern.
//
// Layout (the helpers and operand conventions are in fa_tile.h): a workgroup
// of 4 waves owns 128 query rows, 32 per wave, with Q resident in registers
// as the B operand of S^T = K Q^T (keys on MFMA rows, queries on columns, so
// a lane holds one query and 32 keys of a 64-key tile).  Tiles of K and V (64
// keys, 32 at D = 256) stream through LDS, double-buffered and staged through
// registers.  Q, K, V and O take batch, head and row strides (head dimension
// contiguous); this kernel also serves the plain forward at D = 256.  Per
// tile: mask bytes (one dword per four keys) are loaded before the MFMAs, the
// online softmax runs in fp32 on the accumulators, the dropout decisions are
// drawn, and O^T += V^T P^T takes P straight from the accumulators with V^T
// read by transposing LDS reads.  This kernel is the general path for masks
// and dropout; the plain forward (fa_fwd_kernel.hip) is the tuned one.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_ext.h"
#include "fa_tile.h"

namespace fa {
namespace ext {

using namespace tile;

template <int D, int DT, bool CAUSAL, bool MASK, bool DROP>
__global__ __launch_bounds__(256) void fwd_ext(ExtParams p) {
    constexpr int DC = D / 16, DB = D / 32;
    constexpr int KT = key_tile(D);
    constexpr int RB = KT / 32;                        // 32-key row blocks of S^T per tile
    constexpr int ST = KT / 16;                        // 16-key k-steps of P V per tile
    constexpr int TILE = KT * D * 2;
    constexpr int CPT = KT * D / 8 / 256;
    static_assert(CPT >= 1, "tile must split over the threads");

    __shared__ __attribute__((aligned(16))) char smem[4 * TILE];
    lds_t* const sm = (lds_t*)smem;

    const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, g = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    int bh, qb;
    block_order(blockIdx.x, p.nqb, p.BH, CAUSAL, bh, qb);
    const int Sq = p.Sq, Sk = p.Sk, diag = p.diag;   // causal: key j visible to query i iff j <= i + diag
    const int q0 = qb * kQueryBlock, qw0 = q0 + 32 * w;
    const int qi = qw0 + lq;

    // One buffer per tensor and head, its record count the head's extent:
    // rows past the sequence read as zero and stores to them are dropped.
    const int b_ = bh / p.H, h_ = bh - b_ * p.H;
    auto head = [&](const void* base, int64_t sb, int64_t sh, int ss, int rows) {
        return rsrc((const char*)base + ((int64_t)b_ * sb + (int64_t)h_ * sh) * 2,
                    (uint64_t)(((int64_t)(rows - 1) * ss + D) * 2));
    };
    const __amdgpu_buffer_rsrc_t rq = head(p.q, p.q_sb, p.q_sh, p.q_ss, Sq);
    auto head_words = [&](const void* base, int64_t sb, int64_t sh, int ss, int rows) {
        return rsrc_words((const char*)base + ((int64_t)b_ * sb + (int64_t)h_ * sh) * 2,
                          (uint64_t)(((int64_t)(rows - 1) * ss + D) * 2));
    };
    const i32x4 rk = head_words(p.k, p.k_sb, p.k_sh, p.k_ss, Sk);
    const i32x4 rv = head_words(p.v, p.v_sb, p.v_sh, p.v_ss, Sk);

    // Mask rows of this head: a buffer over [first row, last row + Sk)
    // rounded up to whole dwords; offsets beyond it read as zero (hidden).
    __amdgpu_buffer_rsrc_t rm = rq;
    if constexpr (MASK) {
        const uint8_t* mb = p.mask + (int64_t)b_ * p.m_sb + (int64_t)h_ * p.m_sh;
        rm = rsrc(mb, (uint64_t)(((int64_t)(Sq - 1) * p.m_ss + Sk + 3) & ~(int64_t)3));
    }

    i32x4 qf[DC];
#pragma unroll
    for (int c = 0; c < DC; ++c)
        qf[c] = __builtin_amdgcn_raw_buffer_load_b128(rq, (qi * p.q_ss + 16 * c + 8 * g) * 2, 0, 0);

    int nkt = (Sk + KT - 1) / KT;
    if (CAUSAL) nkt = min(nkt, max(0, (min(Sq, q0 + kQueryBlock) + diag + KT - 1) / KT));

    // K and V tiles go straight from global memory into the LDS buffers; a
    // step waits for its successor's loads just before the closing barrier.
    // The compiler does not see these loads, so with a mask they are issued
    // after the tile's mask bytes (compiler-visible loads) have been used:
    // its wait for those would otherwise also wait for the tile loads.
    const uint32_t lds0 = (uint32_t)(uintptr_t)sm;
    auto issue = [&](int t, int buf) {
        const uint32_t base = lds0 + (uint32_t)(buf * 2 * TILE);
        tile_dma<D, CPT>(rk, t * KT, p.k_ss, base, w, lane);
        tile_dma<D, CPT>(rv, t * KT, p.v_ss, base + TILE, w, lane);
    };
    // mask bytes of keys t*KT + 32rb + 8a + 4g .. +3 for this lane's query
    uint32_t mk[RB][4];
    auto load_mask = [&](int t) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int a = 0; a < 4; ++a)
                mk[rb][a] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
                    rm, (uint32_t)((int64_t)qi * p.m_ss + t * KT + 32 * rb + 8 * a + 4 * g), 0, 0);
    };

    const TrLane tl = tr_lane(lane);
    const float c2 = p.scale_log2e;
    f32x16 oa[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) oa[b] = zero16();
    float m_run = -INFINITY;   // running max, base-2 units
    float l_run = 0.0f;        // this lane's share of the running sum

    if (nkt > 0) {
        issue(0, 0);
        if constexpr (MASK) load_mask(0);
    }
    wait_vmcnt<0>();
    __syncthreads();

    for (int t = 0; t < nkt; ++t) {
        const int buf = t & 1;
        if constexpr (!MASK)
            if (t + 1 < nkt) issue(t + 1, buf ^ 1);
        const lds_t* tk = sm + buf * 2 * TILE;
        const lds_t* tv = tk + TILE;
        const int kt0 = t * KT;

        // S^T = K Q^T: KT keys x this wave's 32 queries
        f32x16 s[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[rb] = zero16();
#pragma unroll
        for (int c = 0; c < DC; ++c)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                s[rb] = mma<DT>(row_frag<D>(tk, 32 * rb + lq, 2 * c + g), qf[c], s[rb]);

        const bool need_mask = MASK || (kt0 + KT > Sk) || (CAUSAL && kt0 + KT - 1 > qw0 + diag);
        if (need_mask) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kj = kt0 + 32 * rb + 8 * (r >> 2) + 4 * g + (r & 3);
                    bool vis = kj < Sk && (!CAUSAL || kj <= qi + diag);
                    if constexpr (MASK) vis = vis && ((mk[rb][r >> 2] >> (8 * (r & 3))) & 0xffu) != 0;
                    if (!vis) s[rb][r] = -INFINITY;
                }
        }
        if constexpr (MASK) {
            if (t + 1 < nkt) {
                issue(t + 1, buf ^ 1);
                load_mask(t + 1);
            }
        }

        // online softmax (base 2, scale*log2(e) folded into one FMA)
        float mx = s[0][0];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[rb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * c2;
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        const float mb = (m_new == -INFINITY) ? 0.0f : m_new;
        m_run = m_new;
        float lsum = 0.0f;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rb][r], c2, -mb));
                s[rb][r] = e;
                lsum += e;
            }
        l_run = l_run * alpha + lsum;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) oa[b][i] *= alpha;
        }

        if constexpr (DROP) {
            // keys kt0 + 32rb + 8a + 0..7 share one Philox block; this lane
            // uses words 2g and 2g+1 (keys 8a + 4g + 0..3)
            uint32_t kw[RB][4][2];
            keep_words<RB>(kw, kt0, qi, bh, p.offset, p.seed_lo, p.seed_hi, g);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const uint32_t w0 = kw[rb][a][0], w1 = kw[rb][a][1];
                    const uint32_t r16[4] = {w0 & 0xffffu, w0 >> 16, w1 & 0xffffu, w1 >> 16};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (r16[e] < p.drop_t) s[rb][4 * a + e] = 0.0f;
                }
        }

        // O^T += V^T P^T
#pragma unroll
        for (int st = 0; st < ST; ++st) {
            const i32x4 pa = acc_frag<DT>(s[st >> 1], st & 1);
#pragma unroll
            for (int b = 0; b < DB; ++b) oa[b] = mma<DT>(tr_frag<D>(tv, st, b, tl), pa, oa[b]);
        }

        wait_vmcnt<0>();
        __syncthreads();
    }

    // O = O^T / l (times the dropout rescale): register r of block b holds
    // head-dimension index 32b + 8(r/4) + 4g + r%4 of query qi.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.0f ? p.keep_scale / l_tot : 0.0f;
    const __amdgpu_buffer_rsrc_t wo = head(p.o, p.o_sb, p.o_sh, p.o_ss, Sq);
#pragma unroll
    for (int b = 0; b < DB; ++b) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            i32x2 v2;
            v2[0] = pack2<DT>(oa[b][4 * a] * inv, oa[b][4 * a + 1] * inv);
            v2[1] = pack2<DT>(oa[b][4 * a + 2] * inv, oa[b][4 * a + 3] * inv);
            __builtin_amdgcn_raw_buffer_store_b64(v2, wo, (uint32_t)((qi * p.o_ss + 32 * b + 8 * a + 4 * g) * 2), 0, 0);
        }
    }
    if (p.lse != nullptr && g == 0 && qi < Sq) {
        const float lse2 = l_tot > 0.0f ? m_run + log2f(l_tot) : -INFINITY;
        p.lse[(int64_t)bh * Sq + qi] = lse2 * 0.69314718055994530942f;
    }
}

template <int D, int DT, bool CAUSAL>
static hipError_t run(const ExtParams& p, hipStream_t st) {
    const dim3 grid((unsigned)(p.BH * p.nqb)), block(256);
    const bool mask = p.mask != nullptr, drop = p.drop_t != 0;
    if (mask && drop) hipLaunchKernelGGL((fwd_ext<D, DT, CAUSAL, true, true>), grid, block, 0, st, p);
    else if (mask) hipLaunchKernelGGL((fwd_ext<D, DT, CAUSAL, true, false>), grid, block, 0, st, p);
    else if (drop) hipLaunchKernelGGL((fwd_ext<D, DT, CAUSAL, false, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((fwd_ext<D, DT, CAUSAL, false, false>), grid, block, 0, st, p);
    return hipGetLastError();
}

hipError_t launch_ext(const ExtParams& p, int D, int dtype, int causal, hipStream_t stream) {
    if (D == 256) {
        if (dtype == 0) return causal ? run<256, 0, true>(p, stream) : run<256, 0, false>(p, stream);
        return causal ? run<256, 1, true>(p, stream) : run<256, 1, false>(p, stream);
    }
    if (D == 64) {
        if (dtype == 0) return causal ? run<64, 0, true>(p, stream) : run<64, 0, false>(p, stream);
        return causal ? run<64, 1, true>(p, stream) : run<64, 1, false>(p, stream);
    }
    if (dtype == 0) return causal ? run<128, 0, true>(p, stream) : run<128, 0, false>(p, stream);
    return causal ? run<128, 1, true>(p, stream) : run<128, 1, false>(p, stream);
}

}  // namespace ext
}  // namespace fa
