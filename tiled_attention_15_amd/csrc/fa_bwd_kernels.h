// fa_bwd_kernels.h -- the attention backward kernels (templates), shared by
// fa_bwd.hip (head dimensions 64 and 128, built with the VGPR form of the
// MFMA instructions) and fa_bwd256.hip (head dimension 256: one wave per
// SIMD, the dK/dV or dQ accumulators in AGPRs).  The mathematics and the
// kernel structure are described at the top of fa_bwd.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_bwd.h"
#include "fa_tile.h"

namespace fa {
namespace bwd {

using namespace tile;

// Start of head bh of a tensor with layout L (byte pointer), and the bytes one
// head spans over `rows` rows (the last row's end).
__device__ __forceinline__ const char* head_of(const void* base, const Lay& L, int bh, int H) {
    const int b = bh / H, h = bh - b * H;
    return (const char*)base + ((int64_t)b * L.sb + (int64_t)h * L.sh) * 2;
}
template <int D>
__device__ __forceinline__ uint64_t head_bytes(const Lay& L, int rows) {
    return (uint64_t)(((int64_t)(rows - 1) * L.ss + D) * 2);
}

// ---------------------------------------------------------------------------
// D_i = sum_d dO_id O_id in fp32.
template <int D, int DT>
__global__ __launch_bounds__(256) void bwd_pre(BwdParams p) {
    constexpr int TPR = D / 8;            // threads per row (8 values each)
    constexpr int RPB = 256 / TPR;        // rows per workgroup
    const int64_t rows = (int64_t)p.BH * p.Sq;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
    const int c = threadIdx.x % TPR;
    float acc = 0.0f;
    if (row < rows) {
        const int bh = (int)(row / p.Sq), qi = (int)(row - (int64_t)bh * p.Sq);
        const i32x4 a = *(const i32x4*)(head_of(p.o, p.Lo, bh, p.H) + ((int64_t)qi * p.Lo.ss + 8 * c) * 2);
        const i32x4 b = *(const i32x4*)(head_of(p.dout, p.Ldo, bh, p.H) + ((int64_t)qi * p.Ldo.ss + 8 * c) * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc += half_f32<DT>(a[i], 0) * half_f32<DT>(b[i], 0) + half_f32<DT>(a[i], 1) * half_f32<DT>(b[i], 1);
    }
#pragma unroll
    for (int o = TPR / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (row < rows && c == 0) p.dvec[row] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV of one 128-key block.  Sized for two workgroups per CU at D <= 128
// (two waves per SIMD, <= 256 registers per lane; one with a mask or dropout,
// and at D = 256, where the accumulators fill the 256 AGPRs): the key block
// sits in LDS (K fragments are read from there at each use) while V's
// fragments and the dK^T, dV^T accumulators stay in registers; 32-query tiles
// of Q and dO go straight from global memory into LDS.
template <int D, int DT, bool CAUSAL, bool MASK = false, bool DROP = false>
__global__ __launch_bounds__(256, D > 128 ? 1 : 2) void bwd_dkdv(BwdParams p) {
    constexpr int DC = D / 16;                         // k-steps over the head dimension
    constexpr int DB = D / 32;                         // 32-column blocks of the head dimension
    constexpr int QT = kQueryTile;
    constexpr int TILE = QT * D * 2;                   // bytes of one Q or dO tile
    constexpr int TN = QT * D / 8 / 256;               // direct loads per thread per tile
    constexpr int KBLK = kKeyBlock * D * 2;            // bytes of the key block
    constexpr int KN = kKeyBlock * D / 8 / 256;        // direct loads per thread for it
    static_assert(TN >= 1 && KN >= 1, "tile must split over the threads");

    __shared__ __attribute__((aligned(16))) char smem[KBLK + 4 * TILE];
    // one score accumulator at a time: at D = 256 (accumulators fill the
    // AGPRs) and with a mask or dropout
    constexpr bool SEQ = D > 128 || MASK || DROP;
    // lse and D_i of a tile (with SEQ loaded straight into LDS by one wave,
    // 64 entries of which the first QT are the tile's)
    __shared__ __attribute__((aligned(16))) float lse_s[2][SEQ ? 64 : QT];
    __shared__ __attribute__((aligned(16))) float dv_s[2][SEQ ? 64 : QT];
    // mask bytes of a tile, [query][key of the block] (with a mask), and the
    // keep bits of a tile, [query][8-key group] one bit per key (with dropout)
    __shared__ __attribute__((aligned(16))) uint8_t msk_s[2][MASK ? QT * kKeyBlock : 16];
    __shared__ __attribute__((aligned(16))) uint8_t keep_s[2][DROP ? QT * kKeyBlock / 8 : 16];
    lds_t* const sm = (lds_t*)smem;

    const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, g = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    int bh, kb;
    block_order(blockIdx.x, p.nkb, p.BH, false, bh, kb);
    const int Sq = p.Sq, Sk = p.Sk, diag = p.diag;   // causal: key j visible to query i iff j <= i + diag
    const int k0 = kb * kKeyBlock, kw0 = k0 + 32 * w;

    const i32x4 rq = rsrc_words(head_of(p.q, p.Lq, bh, p.H), head_bytes<D>(p.Lq, Sq));
    const i32x4 rdo = rsrc_words(head_of(p.dout, p.Ldo, bh, p.H), head_bytes<D>(p.Ldo, Sq));
    const i32x4 rk = rsrc_words(head_of(p.k, p.Lk, bh, p.H), head_bytes<D>(p.Lk, Sk));
    const __amdgpu_buffer_rsrc_t rv = rsrc(head_of(p.v, p.Lv, bh, p.H), head_bytes<D>(p.Lv, Sk));
    const __amdgpu_buffer_rsrc_t rl = rsrc(p.lse + (int64_t)bh * Sq, (uint64_t)Sq * 4);
    const __amdgpu_buffer_rsrc_t rdv = rsrc(p.dvec + (int64_t)bh * Sq, (uint64_t)Sq * 4);

    const uint32_t lds0 = (uint32_t)(uintptr_t)sm;
    const lds_t* kblk = sm;
    // the key block (keys past Sk read as zero)
    tile_dma<D, KN>(rk, k0, p.Lk.ss, lds0, w, lane);
    // V of this wave's 32 keys as B operands (key = column lq, 8 values of
    // the head dimension per k-step)
    i32x4 vf[DC];
#pragma unroll
    for (int c = 0; c < DC; ++c)
        vf[c] = __builtin_amdgcn_raw_buffer_load_b128(rv, ((kw0 + lq) * p.Lv.ss + 16 * c + 8 * g) * 2, 0, 0);

    const int nqt = (Sq + QT - 1) / QT;
    int t0 = 0;
    if (CAUSAL) t0 = max(0, k0 - diag) / QT;

    // Mask rows of this head: a buffer over [first row, last row + Sk)
    // rounded up to whole dwords; offsets beyond it read as zero (hidden).
    i32x4 rm = rq;
    if constexpr (MASK) {
        const int b_ = bh / p.H, h_ = bh - b_ * p.H;
        rm = rsrc_words(p.mask + (int64_t)b_ * p.m_sb + (int64_t)h_ * p.m_sh,
                        (uint64_t)(((int64_t)(Sq - 1) * p.m_ss + Sk + 3) & ~(int64_t)3));
    }
    const uint32_t msk0 = (uint32_t)(uintptr_t)(lds_t*)&msk_s[0][0];
    const TileDma<D, TN> dmq(p.Lq.ss, w, lane), dmo(p.Ldo.ss, w, lane);
    // mask loads: instruction i of wave w covers rows 8i + 2w + lane/32 of
    // the tile, dword lane%32 of each row's 128 key bytes
    const uint32_t mlo = (uint32_t)((lane >> 5) * p.m_ss + 4 * (lane & 31));
    auto issue = [&](int t, int buf) {
        const uint32_t base = lds0 + (uint32_t)(KBLK + buf * 2 * TILE);
        if constexpr (SEQ) {
            dmq.issue(rq, t * QT, base, w);
            dmo.issue(rdo, t * QT, base + TILE, w);
        } else {
            tile_dma<D, TN>(rq, t * QT, p.Lq.ss, base, w, lane);
            tile_dma<D, TN>(rdo, t * QT, p.Ldo.ss, base + TILE, w, lane);
        }
        if constexpr (MASK) {
            static_assert(QT * kKeyBlock / 4 / 256 * 8 == QT && kKeyBlock == 128, "mask tile split");
#pragma unroll
            for (int i = 0; i < QT * kKeyBlock / 4 / 256; ++i) {
                int u = (int)(uint32_t)((int64_t)(t * QT + 8 * i + 2 * w) * p.m_ss + k0);
                asm volatile("" : "+s"(u));
                lds_dma4(rm, mlo + (uint32_t)u, msk0 + (uint32_t)(buf * QT * kKeyBlock + (4 * i + w) * 256));
            }
        }
    };
    // keep bits of a tile: each thread draws two Philox4x32-10 blocks, one
    // per (query, 8-key group), and stores their 8 keep bits as one byte
    auto make_keep = [&](int t, int buf) {
        // thread index kept opaque: the counters and the tile-invariant
        // part of the rounds are recomputed, not held across the loop
        int tid_ = tid;
        asm volatile("" : "+v"(tid_));
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int id = 2 * tid_ + u, ql = id >> 4, grp = id & 15;
            uint32_t c[4] = {(uint32_t)((k0 >> 3) + grp), (uint32_t)(t * QT + ql), (uint32_t)bh, p.offset};
            philox4x32_10(c, p.seed_lo, p.seed_hi);
            uint32_t bits = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t r16 = (c[e >> 1] >> (16 * (e & 1))) & 0xffffu;
                bits |= (r16 >= p.drop_t ? 1u : 0u) << e;
            }
            keep_s[buf][id] = (uint8_t)bits;
        }
    };
    // lse (times log2 e) and D_i of a tile: threads 0..QT-1 and QT..2QT-1
    float sl = 0.0f;
    const i32x4 rl_w = rsrc_words(p.lse + (int64_t)bh * Sq, (uint64_t)Sq * 4);
    const i32x4 rdv_w = rsrc_words(p.dvec + (int64_t)bh * Sq, (uint64_t)Sq * 4);
    auto fetch_stats = [&](int t, int buf) {
        if constexpr (SEQ) {
            if (w == 0) {
                lds_dma4(rl_w, (uint32_t)((t * QT + lane) * 4), (uint32_t)(uintptr_t)(lds_t*)&lse_s[buf][0]);
                lds_dma4(rdv_w, (uint32_t)((t * QT + lane) * 4), (uint32_t)(uintptr_t)(lds_t*)&dv_s[buf][0]);
            }
            return;
        }
        if (tid < QT)
            sl = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, (t * QT + tid) * 4, 0, 0));
        else if (tid < 2 * QT)
            sl = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rdv, (t * QT + tid - QT) * 4, 0, 0));
    };
    auto store_stats = [&](int buf) {
        if constexpr (SEQ) return;
        if (tid < QT)
            lse_s[buf][tid] = sl * LOG2E;
        else if (tid < 2 * QT)
            dv_s[buf][tid - QT] = sl;
    };

    const TrLane tl = tr_lane(lane);
    // per-lane LDS read offsets: tables at D = 256, XOR masks (fewer
    // registers, one VALU per read) at two waves per SIMD
    using FO = typename std::conditional<(D > 128), FragOff<D>, FragXor<D>>::type;
    const FO fo(lane, tl);
    const float c2 = p.scale_log2e;
    const int key = kw0 + lq;
    f32x16 dva[DB], dka[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) {
        dva[b] = zero16();
        dka[b] = zero16();
    }

    if (t0 < nqt) {
        issue(t0, 0);
        fetch_stats(t0, 0);
        if constexpr (DROP) make_keep(t0, 0);
    }
    wait_vmcnt<0>();
    if (t0 < nqt) store_stats(0);
    __syncthreads();

    for (int t = t0; t < nqt; ++t) {
        const int buf = (t - t0) & 1;
        if (t + 1 < nqt) {
            issue(t + 1, buf ^ 1);
            fetch_stats(t + 1, buf ^ 1);
            if constexpr (DROP && !SEQ) make_keep(t + 1, buf ^ 1);
        }
        const lds_t* tq = sm + KBLK + buf * 2 * TILE;
        const lds_t* tdo = tq + TILE;
        const int q0 = t * QT;

        if constexpr (SEQ) {
            // sequence ends and the causal diagonal only on the tiles they
            // cross; the mask bytes on every tile
            const bool need_bounds = (q0 + QT > Sq) || (kw0 + 32 > Sk) || (CAUSAL && kw0 + 31 > q0 + diag);
            const int kl = 32 * w + lq;                    // key within the block
            // One score accumulator at a time (the dK^T, dV^T accumulators
            // fill the AGPRs): S, then P and dV^T += dO^T (P Z c), then dP
            // and dS = P (Z c dP - D_i), then dK^T += Q^T dS.  LDS reads use
            // the per-lane offset tables; the tile base is kept opaque so the
            // base + offset sums are formed here, not held for both buffers.
            uint32_t tqa = (uint32_t)(uintptr_t)tq, kba = (uint32_t)(uintptr_t)(kblk + 32 * w * 2 * D);
            asm volatile("" : "+s"(tqa), "+s"(kba));
            const lds_t* tq_ = (const lds_t*)(uintptr_t)tqa;
            const lds_t* tdo_ = tq_ + TILE;
            const lds_t* kw_ = (const lds_t*)(uintptr_t)kba;
            f32x16 s = zero16();
#pragma unroll
            for (int c = 0; c < DC; ++c) s = mma<DT>(fo.row(tq_, 0, c), fo.row(kw_, 0, c), s);
            // LDS operands AH MFMAs ahead (two waves per SIMD at D <= 128)
            constexpr int MFMA = 0x008, DSR = 0x100, AH = 2;
            if constexpr (D <= 128) {
                __builtin_amdgcn_sched_group_barrier(DSR, 2 * AH, 0);
#pragma unroll
                for (int m = 0; m < DC - AH; ++m) {
                    __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(DSR, 2, 0);
                }
                __builtin_amdgcn_sched_group_barrier(MFMA, AH, 0);
            }
            uint32_t zb = 0;                           // keep decision of register r at bit r
            // this lane's mask byte and keep byte of query row 4g; rows
            // 8a + e further are constant offsets
            const uint8_t* mrow = &msk_s[buf][4 * g * kKeyBlock + kl];
            const uint8_t* krow = &keep_s[buf][4 * g * (kKeyBlock / 8) + (kl >> 3)];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int qr = 8 * a + 4 * g;
                const f32x4 l4 = *(const f32x4*)&lse_s[buf][qr] * LOG2E;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * a + e;
                    float x = s[r] * c2 - l4[e];
                    if (need_bounds) {
                        const int qi = q0 + qr + e;
                        const bool vis = qi < Sq && key < Sk && (!CAUSAL || key <= qi + diag);
                        x = vis ? x : -__builtin_inff();
                    }
                    if constexpr (MASK) x = mrow[(8 * a + e) * kKeyBlock] != 0 ? x : -__builtin_inff();
                    if constexpr (DROP) zb |= ((krow[(8 * a + e) * (kKeyBlock / 8)] >> (kl & 7)) & 1u) << r;
                    s[r] = __builtin_amdgcn_exp2f(x);
                }
            }
            auto zc = [&](int r) { return ((zb >> r) & 1u) ? p.keep_scale : 0.0f; };
#pragma unroll
            for (int st = 0; st < QT / 16; ++st) {
                i32x4 pa;
                if constexpr (DROP) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = 8 * st + 2 * i;
                        pa[i] = pack2<DT>(s[r] * zc(r), s[r + 1] * zc(r + 1));
                    }
                } else {
                    pa = acc_frag<DT>(s, st);
                }
#pragma unroll
                for (int b = 0; b < DB; ++b) dva[b] = mma<DT>(fo.tr(tdo_, st, b), pa, dva[b]);
            }
            f32x16 dp = zero16();
#pragma unroll
            for (int c = 0; c < DC; ++c) dp = mma<DT>(fo.row(tdo_, 0, c), vf[c], dp);
            if constexpr (D <= 128) {
                constexpr int N = DB * (QT / 16);
                __builtin_amdgcn_sched_group_barrier(DSR, 2 * AH, 1);
#pragma unroll
                for (int m = 0; m < N - AH; ++m) {
                    __builtin_amdgcn_sched_group_barrier(MFMA, 1, 1);
                    __builtin_amdgcn_sched_group_barrier(DSR, 2, 1);
                }
                __builtin_amdgcn_sched_group_barrier(MFMA, AH, 1);
                __builtin_amdgcn_sched_group_barrier(DSR, AH, 2);
#pragma unroll
                for (int m = 0; m < DC - AH; ++m) {
                    __builtin_amdgcn_sched_group_barrier(MFMA, 1, 2);
                    __builtin_amdgcn_sched_group_barrier(DSR, 1, 2);
                }
                __builtin_amdgcn_sched_group_barrier(MFMA, AH, 2);
            }
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int qr = 8 * a + 4 * g;
                const f32x4 d4 = *(const f32x4*)&dv_s[buf][qr];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * a + e;
                    if constexpr (DROP) dp[r] = s[r] * (zc(r) * dp[r] - d4[e]);
                    else dp[r] = s[r] * (dp[r] - d4[e]);
                }
            }
#pragma unroll
            for (int st = 0; st < QT / 16; ++st) {
                const i32x4 da = acc_frag<DT>(dp, st);
#pragma unroll
                for (int b = 0; b < DB; ++b) dka[b] = mma<DT>(fo.tr(tq_, st, b), da, dka[b]);
            }
            if constexpr (D <= 128) {
                constexpr int N = DB * (QT / 16);
                __builtin_amdgcn_sched_group_barrier(DSR, 2 * AH, 3);
#pragma unroll
                for (int m = 0; m < N - AH; ++m) {
                    __builtin_amdgcn_sched_group_barrier(MFMA, 1, 3);
                    __builtin_amdgcn_sched_group_barrier(DSR, 2, 3);
                }
                __builtin_amdgcn_sched_group_barrier(MFMA, AH, 3);
            }
        } else {
            // S = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys
            f32x16 s = zero16(), dp = zero16();
#pragma unroll
            for (int c = 0; c < DC; ++c)
                s = mma<DT>(row_frag<D>(tq, lq, 2 * c + g), row_frag<D>(kblk, 32 * w + lq, 2 * c + g), s);
#pragma unroll
            for (int c = 0; c < DC; ++c)
                dp = mma<DT>(row_frag<D>(tdo, lq, 2 * c + g), vf[c], dp);
            if constexpr (!MASK && !DROP && D <= 128) {
                // LDS operands two MFMAs ahead: two reads per MFMA of S, one of dP
                constexpr int MFMA = 0x008, DSR = 0x100, AH = 2;
                __builtin_amdgcn_sched_group_barrier(DSR, 2 * AH, 0);
#pragma unroll
                for (int m = 0; m < DC - AH; ++m) {
                    __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(DSR, 2, 0);
                }
#pragma unroll
                for (int m = DC - AH; m < 2 * DC - AH; ++m) {
                    __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(DSR, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(MFMA, AH, 0);
            }

            // P = exp2(s * scale*log2e - lse*log2e), dS = P (Z c dP - D_i) and
            // P Z c for dV, with Z c the dropout keep factor
            const bool need_mask = MASK || (q0 + QT > Sq) || (kw0 + 32 > Sk) || (CAUSAL && kw0 + 31 > q0 + diag);
            const int kl = 32 * w + lq;                    // key within the block
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int qr = 8 * a + 4 * g;
                const f32x4 l4 = *(const f32x4*)&lse_s[buf][qr];
                const f32x4 d4 = *(const f32x4*)&dv_s[buf][qr];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * a + e;
                    float pv = __builtin_amdgcn_exp2f(s[r] * c2 - l4[e]);
                    if (need_mask) {
                        const int qi = q0 + qr + e;
                        bool vis = qi < Sq && key < Sk && (!CAUSAL || key <= qi + diag);
                        if constexpr (MASK) vis = vis && msk_s[buf][(qr + e) * kKeyBlock + kl] != 0;
                        pv = vis ? pv : 0.0f;
                    }
                    if constexpr (DROP) {
                        const float z = ((keep_s[buf][(qr + e) * (kKeyBlock / 8) + (kl >> 3)] >> (kl & 7)) & 1)
                                            ? p.keep_scale : 0.0f;
                        s[r] = pv * z;
                        dp[r] = pv * (z * dp[r] - d4[e]);
                    } else {
                        s[r] = pv;
                        dp[r] = pv * (dp[r] - d4[e]);
                    }
                }
            }

            // dV^T += dO^T P, dK^T += Q^T dS  (rows: head dimension, columns: keys)
#pragma unroll
            for (int st = 0; st < QT / 16; ++st) {
                const i32x4 pa = acc_frag<DT>(s, st);
                const i32x4 da = acc_frag<DT>(dp, st);
#pragma unroll
                for (int b = 0; b < DB; ++b) {
                    dva[b] = mma<DT>(tr_frag<D>(tdo, st, b, tl), pa, dva[b]);
                    dka[b] = mma<DT>(tr_frag<D>(tq, st, b, tl), da, dka[b]);
                }
            }
            if constexpr (!MASK && !DROP && D <= 128) {
                // transposing reads (two per operand) four MFMAs ahead
                constexpr int MFMA = 0x008, DSR = 0x100, N = 2 * DB * (QT / 16), AH = 4;
                __builtin_amdgcn_sched_group_barrier(DSR, 2 * AH, 1);
#pragma unroll
                for (int m = 0; m < N - AH; ++m) {
                    __builtin_amdgcn_sched_group_barrier(MFMA, 1, 1);
                    __builtin_amdgcn_sched_group_barrier(DSR, 2, 1);
                }
                __builtin_amdgcn_sched_group_barrier(MFMA, AH, 1);
            }
        }

        if constexpr (DROP && SEQ) {
            // the next tile's keep bits once this tile's scores are dead
            __builtin_amdgcn_sched_barrier(0);
            if (t + 1 < nqt) make_keep(t + 1, buf ^ 1);
        }
        wait_vmcnt<0>();
        if (t + 1 < nqt) store_stats(buf ^ 1);
        __syncthreads();
    }

    // dK^T (times scale) and dV^T: register r of block b holds head-dimension
    // index 32b + 8(r/4) + 4g + r%4 of key `key`: four consecutive values per
    // 8-byte store; stores past Sk are dropped by the buffer range.
    const __amdgpu_buffer_rsrc_t wk = rsrc(head_of(p.dk, p.Ldk, bh, p.H), head_bytes<D>(p.Ldk, Sk));
    const __amdgpu_buffer_rsrc_t wv = rsrc(head_of(p.dv, p.Ldv, bh, p.H), head_bytes<D>(p.Ldv, Sk));
    const float sc = p.scale;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const uint32_t offk = (uint32_t)((key * p.Ldk.ss + 32 * b + 8 * a + 4 * g) * 2);
            const uint32_t offv = (uint32_t)((key * p.Ldv.ss + 32 * b + 8 * a + 4 * g) * 2);
            i32x2 kv, vv;
            kv[0] = pack2<DT>(dka[b][4 * a] * sc, dka[b][4 * a + 1] * sc);
            kv[1] = pack2<DT>(dka[b][4 * a + 2] * sc, dka[b][4 * a + 3] * sc);
            vv[0] = pack2<DT>(dva[b][4 * a], dva[b][4 * a + 1]);
            vv[1] = pack2<DT>(dva[b][4 * a + 2], dva[b][4 * a + 3]);
            __builtin_amdgcn_raw_buffer_store_b64(kv, wk, offk, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b64(vv, wv, offv, 0, 0);
        }
    }
}

// ---------------------------------------------------------------------------
// dK, dV of one 256-key block at D = 128 without mask or dropout: eight
// waves in two groups of four (group g owns keys 128g .. 128g + 127 of the
// block, 32 per wave; waves w and w + 4 share a SIMD) that alternate, as the
// forward does, between a matrix phase and an elementwise phase:
//   matrix phase of tile t:  dV^T += dO_{t-1}^T P_{t-1}, dK^T += Q_{t-1}^T dS_{t-1}
//                            (the previous tile's probabilities), then
//                            S_t = Q_t K^T and dP_t = dO_t V^T;
//   elementwise phase of t:  P_t = exp2(S_t scale log2 e - lse log2 e) (0 where
//                            hidden), dS_t = P_t (dP_t - D_i), both packed.
// While one wave of a SIMD runs its matrix phase the other runs its
// elementwise phase; a workgroup barrier separates the phases.  Group 0 runs
// the matrix phase of tile t in half-step 2(t - t0), group 1 one half-step
// later, so the 32-query tiles of Q and dO (and their lse and D_i) are shared
// by both groups through a ring of three LDS stages: tiles t - 1 and t are
// read during half-steps 2(t - t0) and 2(t - t0) + 1, and group 1 loads tile
// t + 1 straight into the third stage at the start of its elementwise phase
// in half-step 2(t - t0), waiting for it before the barrier that ends
// half-step 2(t - t0) + 1.  The key block sits in LDS (K fragments read at
// each use), V of a wave's 32 keys in registers, as in bwd_dkdv.
template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(512) void bwd_dkdv_pp(BwdParams p) {
    constexpr int DC = D / 16;
    constexpr int DB = D / 32;
    constexpr int QT = kQueryTile;
    constexpr int KBP = 256;                           // keys per workgroup
    constexpr int TILE = QT * D * 2;                   // bytes of one Q or dO tile
    constexpr int TN = QT * D / 8 / 256;               // direct loads per thread of a group per tile
    constexpr int KHALF = 128 * D * 2;                 // bytes of a group's 128 keys
    constexpr int KN = 128 * D / 8 / 256;
    constexpr int NST = 3;
    static_assert(TN >= 1 && KN >= 1, "tile must split over the threads");
    static_assert(D <= 128, "two waves per SIMD");
    __shared__ __attribute__((aligned(16))) char smem[2 * KHALF + NST * 2 * TILE];
    __shared__ __attribute__((aligned(16))) float lse_s[NST][64];
    __shared__ __attribute__((aligned(16))) float dv_s[NST][64];
    lds_t* const sm = (lds_t*)smem;

    const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, g = lane >> 5;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wid >> 2, w4 = wid & 3;
    int bh, kb;
    block_order(blockIdx.x, p.nkb, p.BH, false, bh, kb);
    const int Sq = p.Sq, Sk = p.Sk, diag = p.diag;
    const int k0 = kb * KBP, kw0 = k0 + 128 * grp + 32 * w4;

    const i32x4 rq = rsrc_words(head_of(p.q, p.Lq, bh, p.H), head_bytes<D>(p.Lq, Sq));
    const i32x4 rdo = rsrc_words(head_of(p.dout, p.Ldo, bh, p.H), head_bytes<D>(p.Ldo, Sq));
    const i32x4 rk = rsrc_words(head_of(p.k, p.Lk, bh, p.H), head_bytes<D>(p.Lk, Sk));
    const __amdgpu_buffer_rsrc_t rv = rsrc(head_of(p.v, p.Lv, bh, p.H), head_bytes<D>(p.Lv, Sk));
    const i32x4 rl_w = rsrc_words(p.lse + (int64_t)bh * Sq, (uint64_t)Sq * 4);
    const i32x4 rdv_w = rsrc_words(p.dvec + (int64_t)bh * Sq, (uint64_t)Sq * 4);

    const uint32_t lds0 = (uint32_t)(uintptr_t)sm;
    const lds_t* kblk = sm + KHALF * grp;              // this group's 128 keys
    // each group loads its own 128 keys (keys past Sk read as zero)
    tile_dma<D, KN>(rk, k0 + 128 * grp, p.Lk.ss, lds0 + (uint32_t)(KHALF * grp), w4, lane);
    i32x4 vf[DC];
#pragma unroll
    for (int c = 0; c < DC; ++c)
        vf[c] = __builtin_amdgcn_raw_buffer_load_b128(rv, ((kw0 + lq) * p.Lv.ss + 16 * c + 8 * g) * 2, 0, 0);

    const int nqt = (Sq + QT - 1) / QT;
    int t0 = 0;
    if (CAUSAL) t0 = min(nqt, max(0, k0 - diag) / QT);

    // tile t's Q, dO, lse and D_i into stage t % 3 (group 1's waves)
    auto issue = [&](int t) {
        const int st = t % NST;
        const uint32_t base = lds0 + (uint32_t)(2 * KHALF + st * 2 * TILE);
        tile_dma<D, TN>(rq, t * QT, p.Lq.ss, base, w4, lane);
        tile_dma<D, TN>(rdo, t * QT, p.Ldo.ss, base + TILE, w4, lane);
        if (w4 == 0) {
            lds_dma4(rl_w, (uint32_t)((t * QT + lane) * 4), (uint32_t)(uintptr_t)(lds_t*)&lse_s[st][0]);
            lds_dma4(rdv_w, (uint32_t)((t * QT + lane) * 4), (uint32_t)(uintptr_t)(lds_t*)&dv_s[st][0]);
        }
    };

    const TrLane tl = tr_lane(lane);
    const FragXor<D> fo(lane, tl);
    const float c2 = p.scale_log2e;
    const int key = kw0 + lq;
    f32x16 dva[DB], dka[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) {
        dva[b] = zero16();
        dka[b] = zero16();
    }
    f32x16 s = zero16(), dp = zero16();
    i32x4 pa[QT / 16], da[QT / 16];

    constexpr int MFMA = 0x008, DSR = 0x100;
    // matrix phase: products of tile tp = t - 1 (if any) with the packed
    // P, dS, then S and dP of tile t (if any)
    auto mphase = [&](int tp, int t) {
        __builtin_amdgcn_s_setprio(1);
        if (tp >= t0) {
            // stage bases kept opaque: base + offset sums are formed per
            // phase, not held for all three stages
            uint32_t ta = (uint32_t)(uintptr_t)(sm + 2 * KHALF + (tp % NST) * 2 * TILE);
            asm volatile("" : "+s"(ta));
            const lds_t* tq = (const lds_t*)(uintptr_t)ta;
            const lds_t* tdo = tq + TILE;
#pragma unroll
            for (int st = 0; st < QT / 16; ++st) {
#pragma unroll
                for (int b = 0; b < DB; ++b) {
                    dva[b] = mma<DT>(fo.tr(tdo, st, b), pa[st], dva[b]);
                    dka[b] = mma<DT>(fo.tr(tq, st, b), da[st], dka[b]);
                }
            }
            constexpr int N = 2 * DB * (QT / 16), AH = 4;
            __builtin_amdgcn_sched_group_barrier(DSR, 2 * AH, 1);
#pragma unroll
            for (int m = 0; m < N - AH; ++m) {
                __builtin_amdgcn_sched_group_barrier(MFMA, 1, 1);
                __builtin_amdgcn_sched_group_barrier(DSR, 2, 1);
            }
            __builtin_amdgcn_sched_group_barrier(MFMA, AH, 1);
        }
        if (t < nqt) {
            uint32_t ta = (uint32_t)(uintptr_t)(sm + 2 * KHALF + (t % NST) * 2 * TILE);
            uint32_t ka = (uint32_t)(uintptr_t)(kblk + 32 * w4 * 2 * D);
            asm volatile("" : "+s"(ta), "+s"(ka));
            const lds_t* tq = (const lds_t*)(uintptr_t)ta;
            const lds_t* tdo = tq + TILE;
            const lds_t* kw = (const lds_t*)(uintptr_t)ka;
            s = zero16();
            dp = zero16();
            // the S and dP chains interleaved (independent accumulators back
            // to back), three LDS reads per pair two pairs ahead
#pragma unroll
            for (int c = 0; c < DC; ++c) {
                s = mma<DT>(fo.row(tq, 0, c), fo.row(kw, 0, c), s);
                dp = mma<DT>(fo.row(tdo, 0, c), vf[c], dp);
            }
            constexpr int AH = 2;
            __builtin_amdgcn_sched_group_barrier(DSR, 3 * AH, 0);
#pragma unroll
            for (int m = 0; m < DC - AH; ++m) {
                __builtin_amdgcn_sched_group_barrier(MFMA, 2, 0);
                __builtin_amdgcn_sched_group_barrier(DSR, 3, 0);
            }
            __builtin_amdgcn_sched_group_barrier(MFMA, 2 * AH, 0);
        }
        __builtin_amdgcn_s_setprio(0);
    };
    // elementwise phase of tile t
    auto ephase = [&](int t) {
        const int st = t % NST, q0 = t * QT;
        const bool need_mask = (q0 + QT > Sq) || (kw0 + 32 > Sk) || (CAUSAL && kw0 + 31 > q0 + diag);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int qr = 8 * a + 4 * g;
            const f32x4 l4 = *(const f32x4*)&lse_s[st][qr] * LOG2E;
            const f32x4 d4 = *(const f32x4*)&dv_s[st][qr];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * a + e;
                float x = s[r] * c2 - l4[e];
                if (need_mask) {
                    const int qi = q0 + qr + e;
                    const bool vis = qi < Sq && key < Sk && (!CAUSAL || key <= qi + diag);
                    x = vis ? x : -__builtin_inff();
                }
                const float pv = __builtin_amdgcn_exp2f(x);
                s[r] = pv;
                dp[r] = pv * (dp[r] - d4[e]);
            }
        }
#pragma unroll
        for (int h = 0; h < QT / 16; ++h) {
            pa[h] = acc_frag<DT>(s, h);
            da[h] = acc_frag<DT>(dp, h);
        }
    };
    auto barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    auto publish = [&]() {                             // this wave's loads done, then the barrier
        wait_vmcnt<0>();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };

    // Prologue: tile t0 (group 1) and the key block (both).  Then step t
    // (t0 <= t <= nqt) is two half-steps: group 0 runs the matrix phase
    // (tiles t - 1, t) and then the elementwise phase of tile t; group 1 first
    // requests tile t + 1 and runs the elementwise phase of tile t - 1, then
    // the matrix phase (tiles t - 1, t).  Each group runs its own loop with
    // the same barriers; the first and last steps are peeled off.
    if (grp == 1 && t0 < nqt) issue(t0);
    publish();
    if (t0 < nqt) {
        if (grp == 0) {
            mphase(t0 - 1, t0);
            barrier();
            ephase(t0);
            publish();
            for (int t = t0 + 1; t < nqt; ++t) {
                mphase(t - 1, t);
                barrier();
                ephase(t);
                publish();
            }
            mphase(nqt - 1, nqt);
            barrier();
            publish();
        } else {
            if (t0 + 1 < nqt) issue(t0 + 1);
            barrier();
            mphase(t0 - 1, t0);
            publish();
            for (int t = t0 + 1; t < nqt; ++t) {
                if (t + 1 < nqt) issue(t + 1);
                ephase(t - 1);
                barrier();
                mphase(t - 1, t);
                publish();
            }
            ephase(nqt - 1);
            barrier();
            mphase(nqt - 1, nqt);
            publish();
        }
    }

    // dK^T (times scale) and dV^T: as in bwd_dkdv
    const __amdgpu_buffer_rsrc_t wk = rsrc(head_of(p.dk, p.Ldk, bh, p.H), head_bytes<D>(p.Ldk, Sk));
    const __amdgpu_buffer_rsrc_t wv = rsrc(head_of(p.dv, p.Ldv, bh, p.H), head_bytes<D>(p.Ldv, Sk));
    const float sc = p.scale;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const uint32_t offk = (uint32_t)((key * p.Ldk.ss + 32 * b + 8 * a + 4 * g) * 2);
            const uint32_t offv = (uint32_t)((key * p.Ldv.ss + 32 * b + 8 * a + 4 * g) * 2);
            i32x2 kv, vv;
            kv[0] = pack2<DT>(dka[b][4 * a] * sc, dka[b][4 * a + 1] * sc);
            kv[1] = pack2<DT>(dka[b][4 * a + 2] * sc, dka[b][4 * a + 3] * sc);
            vv[0] = pack2<DT>(dva[b][4 * a], dva[b][4 * a + 1]);
            vv[1] = pack2<DT>(dva[b][4 * a + 2], dva[b][4 * a + 3]);
            __builtin_amdgcn_raw_buffer_store_b64(kv, wk, offk, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b64(vv, wv, offv, 0, 0);
        }
    }
}

// ---------------------------------------------------------------------------
// dQ of one 128-query block.
template <int D, int DT, bool CAUSAL, bool MASK = false, bool DROP = false>
__global__ __launch_bounds__(256, D > 128 ? 1 : 2) void bwd_dq(BwdParams p) {
    constexpr int DC = D / 16, DB = D / 32;
    constexpr int KT = kKeyTile;
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

    const __amdgpu_buffer_rsrc_t rq = rsrc(head_of(p.q, p.Lq, bh, p.H), head_bytes<D>(p.Lq, Sq));
    const __amdgpu_buffer_rsrc_t rdo = rsrc(head_of(p.dout, p.Ldo, bh, p.H), head_bytes<D>(p.Ldo, Sq));
    const i32x4 rk = rsrc_words(head_of(p.k, p.Lk, bh, p.H), head_bytes<D>(p.Lk, Sk));
    const i32x4 rv = rsrc_words(head_of(p.v, p.Lv, bh, p.H), head_bytes<D>(p.Lv, Sk));
    const __amdgpu_buffer_rsrc_t rl = rsrc(p.lse + (int64_t)bh * Sq, (uint64_t)Sq * 4);
    const __amdgpu_buffer_rsrc_t rdv = rsrc(p.dvec + (int64_t)bh * Sq, (uint64_t)Sq * 4);

    // Q and dO of this wave's 32 queries as B operands (query = column lq).
    i32x4 qf[DC], df[DC];
#pragma unroll
    for (int c = 0; c < DC; ++c) {
        qf[c] = __builtin_amdgcn_raw_buffer_load_b128(rq, (qi * p.Lq.ss + 16 * c + 8 * g) * 2, 0, 0);
        df[c] = __builtin_amdgcn_raw_buffer_load_b128(rdo, (qi * p.Ldo.ss + 16 * c + 8 * g) * 2, 0, 0);
    }
    const float lse2 = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, qi * 4, 0, 0)) * LOG2E;
    const float dvl = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rdv, qi * 4, 0, 0));

    // Mask rows of this head (offsets beyond the buffer read as zero: hidden).
    __amdgpu_buffer_rsrc_t rm = rl;
    if constexpr (MASK) {
        const int b_ = bh / p.H, h_ = bh - b_ * p.H;
        rm = rsrc(p.mask + (int64_t)b_ * p.m_sb + (int64_t)h_ * p.m_sh,
                  (uint64_t)(((int64_t)(Sq - 1) * p.m_ss + Sk + 3) & ~(int64_t)3));
    }
    // mask bytes of keys t*KT + 32rb + 8a + 4g .. +3 for this lane's query
    uint32_t mk[2][4];
    auto load_mask = [&](int t) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int a = 0; a < 4; ++a)
                mk[rb][a] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
                    rm, (uint32_t)((int64_t)qi * p.m_ss + t * KT + 32 * rb + 8 * a + 4 * g), 0, 0);
    };

    int nkt = (Sk + KT - 1) / KT;
    if (CAUSAL) nkt = min(nkt, max(0, (min(Sq, q0 + kQueryBlock) + diag + KT - 1) / KT));

    // K and V tiles go straight from global memory into the LDS buffers
    // (no staging registers); a step waits for its successor's loads just
    // before the closing barrier.
    // (one per-lane offset per swizzle class and tensor: the offsets of every
    // load held in registers across the loop spilled in the masked and
    // dropout variants)
    const uint32_t lds0 = (uint32_t)(uintptr_t)sm;
    const TileDma<D, CPT> dmk(p.Lk.ss, w, lane), dmv(p.Lv.ss, w, lane);
    auto issue = [&](int t, int buf) {
        const uint32_t base = lds0 + (uint32_t)(buf * 2 * TILE);
        dmk.issue(rk, t * KT, base, w);
        dmv.issue(rv, t * KT, base + TILE, w);
    };

    const TrLane tl = tr_lane(lane);
    const float c2 = p.scale_log2e;
    f32x16 dqa[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) dqa[b] = zero16();

    if (nkt > 0) {
        issue(0, 0);
        if constexpr (MASK) load_mask(0);
    }
    wait_vmcnt<0>();
    __syncthreads();

    for (int t = 0; t < nkt; ++t) {
        const int buf = t & 1;
        // with a mask the next tile's loads wait until this tile's mask bytes
        // (loads the compiler waits for) have been used
        if constexpr (!MASK)
            if (t + 1 < nkt) issue(t + 1, buf ^ 1);
        const lds_t* tk = sm + buf * 2 * TILE;
        const lds_t* tv = tk + TILE;
        const int kt0 = t * KT;

        // S^T = K Q^T and dP^T = V dO^T: 64 keys (rows) x this wave's 32 queries
        f32x16 s[2], dp[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            s[rb] = zero16();
            dp[rb] = zero16();
        }
#pragma unroll
        for (int c = 0; c < DC; ++c) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                s[rb] = mma<DT>(row_frag<D>(tk, 32 * rb + lq, 2 * c + g), qf[c], s[rb]);
                dp[rb] = mma<DT>(row_frag<D>(tv, 32 * rb + lq, 2 * c + g), df[c], dp[rb]);
            }
        }
        if constexpr (!MASK && !DROP && D <= 128) {
            // LDS operands four MFMAs ahead
            constexpr int MFMA = 0x008, DSR = 0x100, N = 4 * DC, AH = 4;
            __builtin_amdgcn_sched_group_barrier(DSR, AH, 0);
#pragma unroll
            for (int m = 0; m < N - AH; ++m) {
                __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
                __builtin_amdgcn_sched_group_barrier(DSR, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(MFMA, AH, 0);
        }

        // sequence ends and the causal diagonal only on the tiles they
        // cross; the mask bytes on every tile
        const bool need_bounds = (kt0 + KT > Sk) || (qw0 + 32 > Sq) || (CAUSAL && kt0 + KT - 1 > qw0 + diag);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = s[rb][r] * c2 - lse2;
                if (need_bounds) {
                    const int kj = kt0 + 32 * rb + 8 * (r >> 2) + 4 * g + (r & 3);
                    const bool vis = qi < Sq && kj < Sk && (!CAUSAL || kj <= qi + diag);
                    x = vis ? x : -__builtin_inff();
                }
                if constexpr (MASK) x = ((mk[rb][r >> 2] >> (8 * (r & 3))) & 0xffu) != 0 ? x : -__builtin_inff();
                s[rb][r] = __builtin_amdgcn_exp2f(x);
            }
        }
        if constexpr (MASK) {
            if (t + 1 < nkt) {
                issue(t + 1, buf ^ 1);
                load_mask(t + 1);
            }
        }
        // dS^T = P (Z c dP - D_i): keys kt0 + 32rb + 8a + 0..7 share one
        // Philox block; this lane uses words 2g and 2g+1 (keys 8a + 4g + 0..3)
        uint32_t kw[2][4][2];
        if constexpr (DROP) keep_words<2>(kw, kt0, qi, bh, p.offset, p.seed_lo, p.seed_hi, g);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                float z[4] = {1.0f, 1.0f, 1.0f, 1.0f};
                if constexpr (DROP) {
                    const uint32_t w0 = kw[rb][a][0];
                    const uint32_t w1 = kw[rb][a][1];
                    const uint32_t r16[4] = {w0 & 0xffffu, w0 >> 16, w1 & 0xffffu, w1 >> 16};
#pragma unroll
                    for (int e = 0; e < 4; ++e) z[e] = r16[e] >= p.drop_t ? p.keep_scale : 0.0f;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * a + e;
                    dp[rb][r] = s[rb][r] * (z[e] * dp[rb][r] - dvl);
                }
            }
        }

        // dQ^T += K^T dS^T  (rows: head dimension, columns: queries)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const i32x4 da = acc_frag<DT>(dp[st >> 1], st & 1);
#pragma unroll
            for (int b = 0; b < DB; ++b) dqa[b] = mma<DT>(tr_frag<D>(tk, st, b, tl), da, dqa[b]);
        }
        if constexpr (!MASK && !DROP && D <= 128) {
            // transposing reads (two per operand) four MFMAs ahead
            constexpr int MFMA = 0x008, DSR = 0x100, N = 4 * DB, AH = 4;
            __builtin_amdgcn_sched_group_barrier(DSR, 2 * AH, 1);
#pragma unroll
            for (int m = 0; m < N - AH; ++m) {
                __builtin_amdgcn_sched_group_barrier(MFMA, 1, 1);
                __builtin_amdgcn_sched_group_barrier(DSR, 2, 1);
            }
            __builtin_amdgcn_sched_group_barrier(MFMA, AH, 1);
        }

        wait_vmcnt<0>();
        __syncthreads();
    }

    const __amdgpu_buffer_rsrc_t wq = rsrc(head_of(p.dq, p.Ldq, bh, p.H), head_bytes<D>(p.Ldq, Sq));
    const float sc = p.scale;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            i32x2 v2;
            v2[0] = pack2<DT>(dqa[b][4 * a] * sc, dqa[b][4 * a + 1] * sc);
            v2[1] = pack2<DT>(dqa[b][4 * a + 2] * sc, dqa[b][4 * a + 3] * sc);
            __builtin_amdgcn_raw_buffer_store_b64(v2, wq, (uint32_t)((qi * p.Ldq.ss + 32 * b + 8 * a + 4 * g) * 2), 0, 0);
        }
    }
}

// ---------------------------------------------------------------------------
template <int D, int DT, bool CAUSAL, bool MASK, bool DROP>
static void run_masked(const BwdParams& p, hipStream_t st) {
    hipLaunchKernelGGL((bwd_dkdv<D, DT, CAUSAL, MASK, DROP>), dim3((unsigned)(p.BH * p.nkb)), dim3(256), 0, st, p);
    hipLaunchKernelGGL((bwd_dq<D, DT, CAUSAL, MASK, DROP>), dim3((unsigned)(p.BH * p.nqb)), dim3(256), 0, st, p);
}

template <int D, int DT, bool CAUSAL>
static hipError_t run(const BwdParams& p, hipStream_t st) {
    const int64_t rows = (int64_t)p.BH * p.Sq;
    constexpr int RPB = 256 / (D / 8);
    if (rows > 0)
        hipLaunchKernelGGL((bwd_pre<D, DT>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st, p);
    if (p.mask != nullptr || p.drop_t != 0) {
        if (p.mask != nullptr && p.drop_t != 0) run_masked<D, DT, CAUSAL, true, true>(p, st);
        else if (p.mask != nullptr) run_masked<D, DT, CAUSAL, true, false>(p, st);
        else run_masked<D, DT, CAUSAL, false, true>(p, st);
        return hipGetLastError();
    }
    if (p.Sk > 0) {
        if constexpr (D == 128) {
            BwdParams q = p;
            q.nkb = (p.Sk + 255) / 256;
            hipLaunchKernelGGL((bwd_dkdv_pp<D, DT, CAUSAL>), dim3((unsigned)(q.BH * q.nkb)), dim3(512), 0, st, q);
        } else {
            hipLaunchKernelGGL((bwd_dkdv<D, DT, CAUSAL>), dim3((unsigned)(p.BH * p.nkb)), dim3(256), 0, st, p);
        }
    }
    if (rows > 0)
        hipLaunchKernelGGL((bwd_dq<D, DT, CAUSAL>), dim3((unsigned)(p.BH * p.nqb)), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace bwd
}  // namespace fa
