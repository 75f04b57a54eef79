// fa_fwd_kernel.hip -- fused attention forward for gfx950 (MI355X).
//
// One workgroup owns a block of B_r = 32 * NW query rows of one (batch, head);
// each of its NW wavefronts owns 32 rows.  K/V tiles of B_c = 64 keys stream
// through double-buffered LDS.  Per tile and wave:
//   S^T = K_tile . Q_w^T    on the matrix cores (v_mfma_f32_32x32x16_{f16,bf16}),
//   online softmax on S     (fp32, base-2 exponentials, scale*log2(e) folded in),
//   O^T += V_tile^T . P^T   on the matrix cores, P taken straight from registers.
// Only O (and the row log-sum-exp) is written to device memory.
//
// The method (tiling of Q into row blocks with K/V column blocks visited in
// an inner loop, the running max m and running sum l with the old partial
// sum rescaled by exp(m_old - m_new), and the fusion of both products and the
// softmax into one kernel) is that of "FlashAttention-2 on Ascend NPU: how
// ops-transformer reaches 3x" (2048ai.net), sections 2.1-2.3.  The causal
// tile skip follows "catlass FlashAttention tuning for a 13B service"
// (gsyq.cn), section "Causal Mask implementation", mode 2.  The pages'
// kernels were written for Ascend's Cube/Vector units and unified buffer;
// none of their code is used here.  The gfx950 layout decisions are:
//
// * Orientation.  The score tile is computed transposed (keys on MFMA rows,
//   queries on MFMA columns).  In the 32x32 accumulator a lane then holds
//   one query column and 16 keys, so row max / row sum are in-lane reductions
//   plus a single exchange between lane l and lane l^32 (v_permlane32_swap).
// * Key permutation.  Row r of the K operand is loaded from key
//   pi(r) = 16*((r/4)%2) + 4*(r/8) + r%4, which makes accumulator register i
//   of lane-half g hold key 16*g + i.  Then the probabilities a lane holds are
//   already in the B-operand layout of the second product (k index 8*g + e
//   of chunk c <-> key 16*g + 8*c + e): no LDS round trip for P.
// * V operand.  The second product needs V with keys along the MFMA k index,
//   i.e. transposed with respect to its [S, D] layout.  ds_read_b64_tr_b16
//   does the transpose in the LDS read: in each 16-lane group, output lane n,
//   element j comes from element n%4 of the 8 bytes addressed by lane 4j+n/4.
// * Output permutation.  MFMA row r of the second product is fed with d
//   column 4*phi(r/4) + r%4, phi(rc) = 4*(rc%2) + rc/2, so that accumulator
//   register i of lane-half g holds d = 16*g + i: each lane writes 32
//   contiguous bytes per 32-column block.
// * Lazy rescaling.  The running max used for the exponentials is only
//   raised when some row's new max exceeds it by more than 2^8 (base-2
//   units); otherwise probabilities up to 2^8 are accumulated against the
//   stale max.  The result is the same in exact arithmetic and skips most
//   O rescales.
// * Edges.  All global traffic uses buffer instructions with the head's
//   extent as the record count: reads past the sequence end return zero and
//   writes past it are dropped, so ragged S needs no branches on loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_launch.h"

namespace fa {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int BC = 64;            // keys per K/V tile
constexpr float RESCALE_THRESHOLD = 8.0f;  // log2 units of allowed max staleness
constexpr uint32_t BUF_FLAGS = 0x00020000u;  // gfx9 buffer descriptor word 3

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)BUF_FLAGS);
}

template <int DT>
__device__ __forceinline__ f32x16 mfma32(i32x4 a, i32x4 b, f32x16 c) {
    if constexpr (DT == 0) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
}

// Two fp32 -> one dword of two 16-bit values, round to nearest even.
template <int DT>
__device__ __forceinline__ int pack2(float x, float y) {
    if constexpr (DT == 0) {
        f16x2 h = __builtin_convertvector((f32x2){x, y}, f16x2);
        return __builtin_bit_cast(int, h);
    } else {
        bf16x2 h = __builtin_convertvector((f32x2){x, y}, bf16x2);
        return __builtin_bit_cast(int, h);
    }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of the partner lane (l ^ 32) combined with our own: returns both halves.
__device__ __forceinline__ float xmax32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xsum32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS swizzles.  K rows are read 16 bytes per lane by 32 rows at once (the
// rows pi(0..31)); XOR-ing the 16-byte chunk index with kswz(row) spreads a
// 16-lane (or 8-lane) group over distinct banks.  V rows are read 8 bytes per
// lane, 64 contiguous bytes per row; XOR-ing the 64-byte segment with the
// row's low bits spreads four consecutive rows over distinct segments.
template <int D>
__device__ __forceinline__ int kswz(int row) {
    row &= 31;
    if constexpr (D == 128) {
        return (row & 3) | (((row >> 4) & 1) << 2) | (((row >> 2) & 1) << 3);
    } else {
        return ((row & 3) | (((row >> 4) & 1) << 2)) ^ ((row >> 2) & 1);
    }
}
template <int D>
__device__ __forceinline__ int vseg_swz(int row) {
    return (D == 128) ? (row & 3) : (row & 1);
}
// byte offset inside a K tile of 16-byte chunk `ch` of row `row`
template <int D>
__device__ __forceinline__ int k_lds_off(int row, int ch) {
    return row * (D * 2) + ((ch ^ kswz<D>(row)) << 4);
}
// byte offset inside a V tile of the 8-byte piece d4 (4 columns) of row `row`
template <int D>
__device__ __forceinline__ int v_lds_off(int row, int d4) {
    int seg = d4 >> 3, in = d4 & 7;
    return row * (D * 2) + ((seg ^ vseg_swz<D>(row)) << 6) + (in << 3);
}

// Workgroup -> (batch*head, query block).  Causal: longest query blocks
// first (their work grows with the block index).  When the head count is a
// multiple of 8, the heads are split over the 8 XCDs (workgroup ids are
// handed to XCDs round-robin), so all blocks of a head share one L2.
__device__ __forceinline__ void schedule(int wg, int nqb, int BH, bool causal, int& bh, int& qb) {
    int slot;
    if ((BH & 7) == 0) {
        const int xcd = wg & 7, k = wg >> 3, hpx = BH >> 3;
        bh = xcd * hpx + k % hpx;
        slot = k / hpx;
    } else {
        bh = wg % BH;
        slot = wg / BH;
    }
    qb = causal ? (nqb - 1 - slot) : slot;
}

template <int D, int DT, bool CAUSAL, int NW>
__global__ __launch_bounds__(NW * 64) void fa_fwd_kernel(FwdParams p) {
    constexpr int NT = NW * 64;           // threads
    constexpr int BR = NW * 32;           // query rows per workgroup
    constexpr int DC = D / 16;            // 16-wide d chunks (k steps of S^T)
    constexpr int DB = D / 32;            // 32-wide d blocks (output tiles)
    constexpr int TILE_BYTES = BC * D * 2;
    constexpr int CHUNKS = TILE_BYTES / 16;          // 16-byte chunks per tile
    constexpr int CPT = CHUNKS / NT;                 // chunks per thread per tensor
    static_assert(CHUNKS % NT == 0, "tile must split evenly over threads");

    __shared__ __attribute__((aligned(16))) char smem[2 * 2 * TILE_BYTES];  // [buf][K,V]

    const int tid = threadIdx.x;
    const int wid = tid >> 6;
    const int lane = tid & 63;
    const int lq = lane & 31;             // query column within the wave
    const int g = lane >> 5;              // lane half

    int bh, qb;
    schedule(blockIdx.x, p.nqb, p.BH, CAUSAL, bh, qb);
    const int S = p.S;
    const int q0 = qb * BR;
    const int qw0 = q0 + wid * 32;        // first query row of this wave
    const int64_t head = (int64_t)bh * S * D;
    const uint32_t head_bytes = (uint32_t)S * D * 2;

    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char*)p.q + head * 2, head_bytes);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc((const char*)p.k + head * 2, head_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc((const char*)p.v + head * 2, head_bytes);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc((char*)p.o + head * 2, head_bytes);

    // Number of K/V tiles this workgroup visits.  Causal: tiles whose first
    // key lies beyond the block's last row are skipped.
    const int nkv = (S + BC - 1) / BC;
    int nt = nkv;
    if (CAUSAL) {
        const int last = min(S, q0 + BR);
        nt = min(nkv, (last + BC - 1) / BC);
    }
    // Tiles this wave needs (causal: up to its own last row).
    int nt_w = (qw0 < S) ? nt : 0;
    if (CAUSAL && qw0 < S) nt_w = min(nt, (min(S, qw0 + 32) + BC - 1) / BC);

    // ---- Q fragments: B operand of S^T, lane (lq, g): d = 16c + 8g + [0,8)
    i32x4 qf[DC];
#pragma unroll
    for (int c = 0; c < DC; ++c)
        qf[c] = __builtin_amdgcn_raw_buffer_load_b128(rq, ((qw0 + lq) * D + 16 * c + 8 * g) * 2, 0, 0);

    // ---- per-thread K/V staging registers and their LDS destinations
    i32x4 kst[CPT], vst[CPT];
    auto gload = [&](int t) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int x = tid + i * NT;          // chunk id within tile
            const int row = x / (D / 8), ch = x % (D / 8);
            const uint32_t off = ((uint32_t)(t * BC + row) * D + ch * 8) * 2;
            kst[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
            vst[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
        }
    };
    auto lstore = [&](int buf) {
        char* kb = smem + buf * 2 * TILE_BYTES;
        char* vb = kb + TILE_BYTES;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int x = tid + i * NT;
            const int row = x / (D / 8), ch = x % (D / 8);
            *(i32x4*)(kb + k_lds_off<D>(row, ch)) = kst[i];
            // a 16-byte V chunk is two 8-byte pieces (d4 = 2ch, 2ch+1), same segment
            *(i32x4*)(vb + v_lds_off<D>(row, 2 * ch)) = vst[i];
        }
    };

    // ---- accumulators and running statistics
    f32x16 oacc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[b][i] = 0.0f;
    float m_run = -INFINITY;   // running max of scale*log2e*s (base-2 units)
    float l_run = 0.0f;        // this lane's partial row sum (keys of its half)
    const float c2 = p.scale_log2e;

    // K operand row for this lane: pi(lq)
    const int krow = 16 * ((lq >> 2) & 1) + 4 * (lq >> 3) + (lq & 3);
    // V transposed-read addressing for this lane (see header comment)
    const int vkey = 16 * g + ((lane & 15) >> 2);                           // + 32kb + 8c + 4rr
    const int vphi = 4 * (lane & 1) + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);  // + 8db

    if (nt > 0) {
        gload(0);
        lstore(0);
    }
    __syncthreads();

    for (int t = 0; t < nt; ++t) {
        const int buf = t & 1;
        if (t + 1 < nt) gload(t + 1);
        if (t < nt_w) {
            const char* kb = smem + buf * 2 * TILE_BYTES;
            const char* vb = kb + TILE_BYTES;
            // ---- S^T = K Q^T for the 64 keys of this tile (two 32-key blocks)
            f32x16 s[2];
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kb2][i] = 0.0f;
#pragma unroll
                for (int c = 0; c < DC; ++c) {
                    const i32x4 a = *(const i32x4*)(kb + k_lds_off<D>(32 * kb2 + krow, 2 * c + g));
                    s[kb2] = mfma32<DT>(a, qf[c], s[kb2]);
                }
            }
            // ---- mask: causal keys beyond the row, and keys past the end
            const int key0 = t * BC + 16 * g;  // key of s[kb2][i] is key0 + 32*kb2 + i
            const int qrow = qw0 + lq;
            const bool need_mask = (t * BC + BC > S) || (CAUSAL && t * BC + BC - 1 > qw0);
            if (need_mask) {
                const int lim = CAUSAL ? min(qrow, S - 1) : S - 1;  // last visible key
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (key0 + 32 * kb2 + i > lim) s[kb2][i] = -INFINITY;
            }
            // ---- online softmax (base 2)
            float mx = s[0][0];
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb2][i]);
            mx = xmax32(mx) * c2;  // c2 > 0, so max commutes with the scaling
            const bool grow = mx > m_run + RESCALE_THRESHOLD;
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
                const float m_new = fmaxf(m_run, mx);
                const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int b = 0; b < DB; ++b)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[b][i] *= alpha;
            }
            const float mb = (m_run == -INFINITY) ? 0.0f : m_run;
            float lsum = 0.0f;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float e = fast_exp2(__builtin_fmaf(s[kb2][i], c2, -mb));
                    s[kb2][i] = e;
                    lsum += e;
                }
            l_run += lsum;
            // ---- P as B operand: chunk (kb2, c) holds keys 32kb2 + 16g + 8c + [0,8)
            i32x4 pf[4];
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    i32x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        w[e] = pack2<DT>(s[kb2][8 * c + 2 * e], s[kb2][8 * c + 2 * e + 1]);
                    pf[2 * kb2 + c] = w;
                }
            // ---- O^T += V^T P^T
#pragma unroll
            for (int b = 0; b < DB; ++b) {
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) {
                    const int kb2 = kc >> 1, c = kc & 1;
                    const int key = 32 * kb2 + 8 * c + vkey;
                    const int d4 = 8 * b + vphi;
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4*)(vb + v_lds_off<D>(key, d4)));
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4*)(vb + v_lds_off<D>(key + 4, d4)));
                    i32x4 a;
                    a[0] = __builtin_bit_cast(int, (short __attribute__((ext_vector_type(2)))){lo[0], lo[1]});
                    a[1] = __builtin_bit_cast(int, (short __attribute__((ext_vector_type(2)))){lo[2], lo[3]});
                    a[2] = __builtin_bit_cast(int, (short __attribute__((ext_vector_type(2)))){hi[0], hi[1]});
                    a[3] = __builtin_bit_cast(int, (short __attribute__((ext_vector_type(2)))){hi[2], hi[3]});
                    oacc[b] = mfma32<DT>(a, pf[kc], oacc[b]);
                }
            }
        }
        if (t + 1 < nt) lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O /= l, round to dtype, store; lse = (m + log2 l) ln 2
    const float l_tot = xsum32(l_run);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const int qrow = qw0 + lq;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
        i32x4 w0, w1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            w0[e] = pack2<DT>(oacc[b][2 * e] * inv, oacc[b][2 * e + 1] * inv);
            w1[e] = pack2<DT>(oacc[b][8 + 2 * e] * inv, oacc[b][8 + 2 * e + 1] * inv);
        }
        const uint32_t off = ((uint32_t)qrow * D + 32 * b + 16 * g) * 2;
        __builtin_amdgcn_raw_buffer_store_b128(w0, ro, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(w1, ro, off + 16, 0, 0);
    }
    if (p.lse != nullptr && g == 0 && qrow < S) {
        const float lse2 = (l_tot > 0.0f) ? (m_run == -INFINITY ? 0.0f : m_run) + log2f(l_tot) : -INFINITY;
        p.lse[(int64_t)bh * S + qrow] = lse2 * 0.69314718055994530942f;
    }
}

template <int D, int DT, bool CAUSAL, int NW>
static hipError_t launch_instance(const FwdParams& p, int64_t grid, hipStream_t stream) {
    hipLaunchKernelGGL((fa_fwd_kernel<D, DT, CAUSAL, NW>), dim3((unsigned)grid), dim3(NW * 64), 0,
                       stream, p);
    return hipGetLastError();
}

template <int D, int DT>
static hipError_t launch_c(const FwdParams& p, bool causal, int64_t grid, hipStream_t s) {
    return causal ? launch_instance<D, DT, true, FA_WAVES>(p, grid, s)
                  : launch_instance<D, DT, false, FA_WAVES>(p, grid, s);
}

hipError_t launch_fwd(const FwdParams& p, int D, int dtype, bool causal, int64_t grid,
                      hipStream_t stream) {
    if (D == 64) return dtype == 0 ? launch_c<64, 0>(p, causal, grid, stream)
                                   : launch_c<64, 1>(p, causal, grid, stream);
    return dtype == 0 ? launch_c<128, 0>(p, causal, grid, stream)
                      : launch_c<128, 1>(p, causal, grid, stream);
}

}  // namespace fa
