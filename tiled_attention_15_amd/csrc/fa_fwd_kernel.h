// fa_fwd_kernel.h -- fused attention forward for gfx950 (MI355X): the kernel
// template (instantiated by fa_fwd_kernel.hip and fa_fwd_diag.hip).
//
// One workgroup owns a block of B_r = 256 query rows of one (batch, head);
// each of its 8 wavefronts owns 32 rows.  K/V tiles of B_c = 64 keys stream
// through LDS.  Per tile and wave:
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
// * Key split (the SPLIT instances): for grids too small to fill the chip,
//   both wave groups own the same 128 query rows and take the even and odd
//   K/V tiles respectively; the two partial (O, running max, running sum)
//   are merged through LDS at the end, the same rescale-and-add as the
//   online softmax's own update.
// * Optional boolean mask (the MASK instances): each lane reads the mask
//   bytes of its query row and its 32 keys of a tile one step ahead and sets
//   the hidden scores to -inf before the online softmax, as the causal rule
//   does on diagonal tiles ("FlashAttention-2 on Ascend NPU: how
//   ops-transformer reaches 3x" (2048ai.net), section 3.4: the mask acts on
//   the score tile on chip).
// * Optional dropout (the DROP instances): in its softmax phase each lane
//   draws the Philox4x32-10 blocks of its own 32 keys (a lane's 16
//   consecutive keys of a 32-key block are two whole 8-key blocks of the
//   generator's counter, so no lane needs another's words) and clears the
//   dropped probabilities in the packed P; O's divisor and the lse stay
//   those of the undropped softmax and the kept weights are scaled by
//   65536 / (65536 - t) at the end ("FlashAttention-2 on Ascend NPU: how
//   ops-transformer reaches 3x" (2048ai.net), sections 3.4 and 6.3: dropout
//   fused into the kernel, on chip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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

// acc + x.lo + x.hi for a dword of two 16-bit values (a dot product with
// (1, 1): the products are exact, the sum accumulates in fp32).
template <int DT>
__device__ __forceinline__ float dot2_ones(int x, float acc) {
    if constexpr (DT == 0) {
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), one, acc, false);
    } else {
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), one, acc, false);
    }
}

// Dropout on a dword of two packed 16-bit probabilities pw: half h is kept
// iff half h of the random word r is >= t, with t - 1 in both halves of
// tm1x2.  The saturating difference r - (t - 1) is nonzero exactly for the
// kept halves, its minimum with 1 is then 1 or 0, and the 16-bit product
// keeps the probability's bits or clears them: three packed 16-bit integer
// instructions per pair (the compiler renders the same expression as
// compares, selects and a permute, five).  `ones` holds 1 in both halves.
__device__ __forceinline__ int drop_pair(int pw, uint32_t r, uint32_t tm1x2, uint32_t ones) {
    int out;
    asm("v_pk_sub_u16 %0, %1, %2 clamp\n\t"
        "v_pk_min_u16 %0, %0, %3\n\t"
        "v_pk_mul_lo_u16 %0, %4, %0"
        : "=&v"(out)
        : "v"(r), "s"(tm1x2), "s"(ones), "v"(pw));
    return out;
}

// The first two steps of drop_pair alone: 1 in each 16-bit half whose random
// half is >= t, 0 elsewhere (a keep multiplier, applied by keep_apply).
__device__ __forceinline__ uint32_t keep_mult(uint32_t r, uint32_t tm1x2, uint32_t ones) {
    uint32_t out;
    asm("v_pk_sub_u16 %0, %1, %2 clamp\n\t"
        "v_pk_min_u16 %0, %0, %3"
        : "=&v"(out)
        : "v"(r), "s"(tm1x2), "s"(ones));
    return out;
}
// The last step of drop_pair: the packed probabilities times their multipliers.
__device__ __forceinline__ int keep_apply(int pw, uint32_t km) {
    int out;
    asm("v_pk_mul_lo_u16 %0, %1, %2" : "=v"(out) : "v"(pw), "v"(km));
    return out;
}

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
// lane, 64 contiguous bytes from each of four consecutive rows per 32 lanes
// (256 bytes: all 64 banks once); XOR-ing the 64-byte segment with row bits
// puts the four rows on four distinct quarters of the banks: the row's two
// low bits at D >= 128 (rows of 256 bytes or more), bit 1 at D = 64 (rows of
// 128 bytes, whose bit 0 already selects the upper half of the banks).
template <int D>
__device__ __forceinline__ int kswz(int row) {
    row &= 31;
    if constexpr (D >= 128) {
        return (row & 3) | (((row >> 4) & 1) << 2) | (((row >> 2) & 1) << 3);
    } else {
        return ((row & 3) | (((row >> 4) & 1) << 2)) ^ ((row >> 2) & 1);
    }
}
template <int D>
__device__ __forceinline__ int vseg_swz(int row) {
    return (D >= 128) ? (row & 3) : ((row >> 1) & 1);
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

// ---------------------------------------------------------------------------
// Ping-pong schedule.  The eight wavefronts form two groups of four (waves w
// and w + 4 share a SIMD) that alternate between a matrix phase (P_{t-1} V_{t-1}
// and K_t Q^T on the matrix cores, operands from LDS) and a softmax phase
// (mask, max, exp2, sum, packing of P_t, all VALU).  While one wave of a SIMD
// runs its matrix phase the other runs its softmax phase, so the matrix core
// and the vector ALU work at the same time instead of in turn.  A workgroup
// barrier separates the phases; the matrix phase raises the wave's issue
// priority.
//
// K/V tiles stream into a ring of four LDS slots with direct global->LDS
// buffer loads issued two steps ahead: the loads of tile t+2 are issued
// during step t into the slot that held tile t-2 (whose last reads ended with
// step t-1), and each wave waits for its own loads of tile t+1 at the end of
// step t.  Group 1 loads the K tiles and group 0 the V tiles, each at the
// start of its softmax phase, so no matrix phase queues behind load
// instructions.  The loads are written as inline assembly so that the
// compiler, which cannot tell the slots apart, does not make every
// transposing LDS read wait for all of them; M0, which they set, is used by
// nothing else in this kernel.
// ---------------------------------------------------------------------------

// One 16-byte-per-lane direct load into LDS: lane l's 16 bytes at voffset go
// to LDS address lds_addr + 16*l.  lds_addr must be wave-uniform.
__device__ __forceinline__ void lds_dma16(i32x4 rsrc, uint32_t voffset, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voffset), "s"(rsrc), "s"(lds_addr) : "memory", "m0");
}

// s_waitcnt vmcnt(n) alone (gfx9 encoding: vmcnt split over bits 3:0 and
// 15:14; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Buffer descriptor as four dwords (for inline assembly).
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffff));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = (int)BUF_FLAGS;
    return r;
}

// DIAG instances (test-only, no mask): the same kernel that additionally
// honours p.diag_flags (reversed workgroup order), counts the K/V tiles each
// wave runs its softmax on into p.tiles, and stores O in fp32 to p.o32
// beside the usual store, so the kernel's own error can be measured before
// the rounding of O to 16 bits.
template <int D, int DT, bool CAUSAL, bool MASK, bool SPLIT, bool DIAG = false, bool DROP = false>
__global__ __launch_bounds__(512) void fa_fwd_kernel(FwdParams p) {
    static_assert(!DIAG || (!MASK && !DROP && D != 256), "diagnostic instances: no mask or dropout, D <= 128");
    constexpr int NW = 8;
    constexpr int NT = 512;
    // D = 256: waves w and w ^ 1 of one group share 32 query rows; each
    // computes the scores and probabilities of its own 32 keys of a tile and
    // holds half of O's columns (the pair exchanges row maxima and packed
    // probabilities through LDS).
    constexpr bool DSPLIT = D == 256;
    static_assert(!DSPLIT || !SPLIT, "D = 256 is split by head dimension, not by keys");
    constexpr int BR = (SPLIT || DSPLIT) ? 128 : 256;
    constexpr int DC = D / 16;
    constexpr int DB = D / 32;
    constexpr int DO = DSPLIT ? DB / 2 : DB;          // 32-column O blocks this wave holds
    constexpr int TILE_BYTES = BC * D * 2;
    constexpr int SLOT_BYTES = 2 * TILE_BYTES;      // K tile then V tile
    constexpr int NSLOT = DSPLIT ? 2 : (SPLIT && D == 64) ? 8 : 4;
    constexpr int CHUNKS = TILE_BYTES / 16;
    constexpr int LPT = CHUNKS / NT;                // 16-byte loads per thread per tensor
    static_assert(CHUNKS % NT == 0, "tile must split evenly over threads");

    // D = 256: after the ring, each wave's row maxima (64 floats; at the end
    // its two partial sums) and packed probabilities (2 x 64 x 16 bytes) for
    // its pair mate
    constexpr int XMAX_BYTES = DSPLIT ? 8 * 2 * 64 * 4 : 0;   // also the pair's final sums
    constexpr int XP_BYTES = DSPLIT ? 8 * 2 * 64 * 16 : 0;
    __shared__ __attribute__((aligned(16))) char smem[NSLOT * SLOT_BYTES + XMAX_BYTES + XP_BYTES];

    const int tid = threadIdx.x;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lq = lane & 31;
    const int g = lane >> 5;
    const int grp = wid >> 2;

    int bh, qb;
    const int wg_id = (DIAG && (p.diag_flags & kDiagReverseOrder)) ? (int)(gridDim.x - 1 - blockIdx.x)
                                                                     : (int)blockIdx.x;
    schedule(wg_id, p.nqb, p.BH, CAUSAL, bh, qb);
    const int Sq = p.Sq, Sk = p.Sk;
    // Causal diagonal: key j is visible to query i iff j <= i + diag
    // (Sk - Sq unless the caller placed it elsewhere: the last query row then
    // sees the last key).
    const int diag = p.diag;
    const int q0 = qb * BR;
    // key split: both groups share the rows; D = 256: a pair per 32 rows
    const int qw0 = q0 + (SPLIT ? (wid & 3) : DSPLIT ? (wid >> 1) : wid) * 32;
    const int dob = DSPLIT ? (wid & 1) * DO : 0;                       // first O block of this wave
    const int b_ = bh / p.H, h_ = bh - b_ * p.H;

    // One buffer descriptor per tensor and head; its record count is the
    // head's extent (last row's end), so rows past the sequence read as zero
    // and stores to them are dropped.
    auto head_rsrc = [&](const void* base, int64_t sb, int64_t sh, int ss, int rows) {
        const char* hb = (const char*)base + ((int64_t)b_ * sb + (int64_t)h_ * sh) * 2;
        return make_rsrc(hb, (uint32_t)(((int64_t)(rows - 1) * ss + D) * 2));
    };
    const __amdgpu_buffer_rsrc_t rq = head_rsrc(p.q, p.q_sb, p.q_sh, p.q_ss, Sq);
    const __amdgpu_buffer_rsrc_t ro = head_rsrc(p.o, p.o_sb, p.o_sh, p.o_ss, Sq);
    const i32x4 rk = rsrc_words((const char*)p.k + ((int64_t)b_ * p.k_sb + (int64_t)h_ * p.k_sh) * 2,
                                (uint32_t)(((int64_t)(Sk - 1) * p.k_ss + D) * 2));
    const i32x4 rv = rsrc_words((const char*)p.v + ((int64_t)b_ * p.v_sb + (int64_t)h_ * p.v_sh) * 2,
                                (uint32_t)(((int64_t)(Sk - 1) * p.v_ss + D) * 2));

    // Mask rows of this head: one buffer over [first row, last row + Sk)
    // rounded up to whole dwords, so reads past it (rows beyond the sequence,
    // keys beyond the last dword) return zero, i.e. hidden.  A lane reads the
    // bytes of its query row and its 32 keys of a tile: mk[4*kb2 + j] holds
    // keys 32*kb2 + 16*g + 4*j .. +3, byte e of it key 32*kb2 + 16*g + 4*j + e,
    // the keys of accumulator registers 4*j + e of s[kb2].
    __amdgpu_buffer_rsrc_t rm = rq;
    uint32_t mk[8];
    if constexpr (MASK) {
        const uint8_t* mbase = p.mask + (int64_t)b_ * p.m_sb + (int64_t)h_ * p.m_sh;
        rm = make_rsrc(mbase, (uint32_t)(((int64_t)(Sq - 1) * p.m_ss + Sk + 3) & ~(int64_t)3));
    }
    // Separate dword loads (an empty asm statement between them keeps the
    // compiler from fusing a lane's four adjacent dwords into one 16-byte
    // load): each dword is range-checked on its own, so a row's last keys
    // read correctly up to the buffer's end.
    auto load_mask = [&](int t) {
        // rows past the sequence read from beyond the buffer (2^31 exceeds
        // its record count): zero, without 32-bit wraparound of the offset
        const int qrow = qw0 + lq;
        const uint32_t row = qrow < Sq ? (uint32_t)qrow * (uint32_t)p.m_ss + (uint32_t)(t * BC + 16 * g)
                                       : 0x80000000u;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                mk[4 * kb2 + j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rm, row + 32 * kb2 + 4 * j, 0, 0);
                asm volatile("" ::: "memory");
            }
    };

    // Every wave visits all nt tiles of its workgroup: a wave whose rows end
    // before a diagonal tile finds it fully masked (probabilities exactly 0),
    // and the phase barriers would make it wait for that tile anyway.  A
    // block none of whose rows sees a key still runs one (fully masked) tile.
    const int nkv = (Sk + BC - 1) / BC;
    int nt = nkv;
    if (CAUSAL) nt = max(1, min(nkv, (min(Sq, q0 + BR) + diag + BC - 1) / BC));

    // Direct-to-LDS loads.  Group 1 loads every K tile and group 0 every V
    // tile, each at the start of its softmax phase, so no wave's matrix phase
    // queues behind load instructions.  Instruction i of wave w (w within its
    // group) fills LDS chunks (i*4 + w)*64 + lane of the tile; each lane
    // fetches the global chunk that the swizzled layout puts there.
    const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)smem);
    const int kv_ss = grp != 0 ? p.k_ss : p.v_ss;     // row stride of the tensor this wave loads
    uint32_t src[2 * LPT];
#pragma unroll
    for (int i = 0; i < 2 * LPT; ++i) {
        const int c = (i * 4 + (wid & 3)) * 64 + lane;
        const int row = c / (D / 8), cl = c % (D / 8);
        if (grp != 0) {
            src[i] = (uint32_t)(row * kv_ss + ((cl ^ kswz<D>(row)) << 3)) * 2;
        } else {
            const int gc = (((cl >> 2) ^ vseg_swz<D>(row)) << 2) | (cl & 3);
            src[i] = (uint32_t)(row * kv_ss + (gc << 3)) * 2;
        }
    }
    const i32x4 rkv = grp != 0 ? rk : rv;
    const uint32_t part = grp != 0 ? 0u : (uint32_t)TILE_BYTES;
    const uint32_t tile_stride = (uint32_t)BC * kv_ss * 2;     // bytes between K/V tiles
    auto issue_tile = [&](int t) {
        const uint32_t tb = (uint32_t)t * tile_stride;
        const uint32_t sb = lds0 + (uint32_t)(t & (NSLOT - 1)) * SLOT_BYTES + part;
#pragma unroll
        for (int i = 0; i < 2 * LPT; ++i)
            lds_dma16(rkv, src[i] + tb, sb + (uint32_t)(i * 4 + (wid & 3)) * 1024);
    };

    i32x4 qf[DC];
#pragma unroll
    for (int c = 0; c < DC; ++c)
        qf[c] = __builtin_amdgcn_raw_buffer_load_b128(rq, ((qw0 + lq) * p.q_ss + 16 * c + 8 * g) * 2, 0, 0);

    f32x16 oacc[DO];
#pragma unroll
    for (int b = 0; b < DO; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[b][i] = 0.0f;
    f32x16 s[2];
    i32x4 pf[4];
    // Dropout without a mask or key split: the keep multipliers of a tile are
    // drawn in the matrix phase that computes its scores (where the vector
    // unit has slack) instead of in its softmax phase.
    constexpr bool KEEP_EARLY = DROP && !SPLIT && !DSPLIT && !MASK;
    uint32_t km[4][4];
    float m_run = -INFINITY;
    float l_run = 0.0f;     // running sum of the probabilities (fp32): the lse
    float r_run = 0.0f;     // running sum of the probabilities as rounded for P V: O's divisor
    const float c2 = p.scale_log2e;
    const int krow = 16 * ((lq >> 2) & 1) + 4 * (lq >> 3) + (lq & 3);
    const int vkey = 16 * g + ((lane & 15) >> 2);
    const int vphi = 4 * (lane & 1) + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);

    // LDS read addresses.  With the swizzles above, every address this lane
    // reads is (lane base + slot base) XOR (a small per-read constant in bits
    // that neither base touches) plus a per-read immediate, so a step costs a
    // handful of XORs instead of dozens of precomputed address registers.
    const int ks = kswz<D>(krow);
    const int kbase_l = krow * (2 * D) + ((g ^ (ks & 1)) << 4) + ((ks >> 1) << 5);
    const int vbase_l = vkey * (2 * D) + (vseg_swz<D>(vkey) << 6) + (vphi << 3);

    // Matrix phase pieces: O += P V (V tile of tile t), S = K Q^T (K tile of t).
    auto pv = [&](int t) {
        const int vb = (t & (NSLOT - 1)) * SLOT_BYTES + TILE_BYTES + vbase_l;
        // kc outer, b inner: consecutive MFMAs accumulate into different O
        // blocks, so none waits for the previous one's result.
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
            for (int b = 0; b < DO; ++b) {
                const int kb2 = kc >> 1, c = kc & 1;
                const int off = (vb ^ ((b + dob) << 6)) + (32 * kb2 + 8 * c) * (2 * D);
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4*)(smem + off));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4*)(smem + off + 4 * (2 * D)));
                i32x4 a;
                a[0] = __builtin_bit_cast(int, (short __attribute__((ext_vector_type(2)))){lo[0], lo[1]});
                a[1] = __builtin_bit_cast(int, (short __attribute__((ext_vector_type(2)))){lo[2], lo[3]});
                a[2] = __builtin_bit_cast(int, (short __attribute__((ext_vector_type(2)))){hi[0], hi[1]});
                a[3] = __builtin_bit_cast(int, (short __attribute__((ext_vector_type(2)))){hi[2], hi[3]});
                oacc[b] = mfma32<DT>(a, pf[kc], oacc[b]);
            }
        }
    };
    auto qk = [&](int t) {
        const int kb = (t & (NSLOT - 1)) * SLOT_BYTES + kbase_l;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kb2][i] = 0.0f;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            const int kc_off = kb ^ (c << 5);
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
                const i32x4 a = *(const i32x4*)(smem + kc_off + kb2 * 32 * (2 * D));
                s[kb2] = mfma32<DT>(a, qf[c], s[kb2]);
            }
        }
    };

    // Explicit mask of the scores of tile t (the words load_mask(t) read).
    // It runs before the phase issues its tile loads, and an asm statement
    // holding the results keeps it there: the compiler, which does not see those loads,
    // waits for every outstanding load before it reads the mask words, and
    // the loads in flight at that point are ones this step needs anyway.
    // The next tile's mask words are requested right after the tile loads.
    auto mask_scores = [&]() {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (((mk[4 * kb2 + (i >> 2)] >> (8 * (i & 3))) & 0xffu) == 0) s[kb2][i] = -INFINITY;
        // the masked scores as operands of a volatile asm statement: they are
        // complete before the (volatile asm) tile loads that follow
        asm volatile("" : "+v"(s[0]), "+v"(s[1]));
    };

    // Diagnostic count of the tiles this wave runs its softmax on.
    int ntiles = 0;
    auto store_tiles = [&]() {
        if constexpr (DIAG)
            if (p.tiles != nullptr && lane == 0) p.tiles[((int64_t)bh * p.nqb + qb) * 8 + wid] = (uint32_t)ntiles;
    };

    // Softmax phase of step t: mask, running max, exponentials, P_t packed.
    auto swork = [&](int t) {
        if constexpr (DIAG) ++ntiles;
        const int key0 = t * BC + 16 * g;
        const int qrow = qw0 + lq;
        const bool need_mask = (t * BC + BC > Sk) || (CAUSAL && t * BC + BC - 1 > qw0 + diag);
        if (need_mask) {
            const int lim = CAUSAL ? min(qrow + diag, Sk - 1) : Sk - 1;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (key0 + 32 * kb2 + i > lim) s[kb2][i] = -INFINITY;
        }
        float mx = s[0][0];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb2][i]);
        mx = xmax32(mx) * c2;
        const bool grow = mx > m_run + RESCALE_THRESHOLD;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
            r_run *= alpha;
#pragma unroll
            for (int b = 0; b < DO; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[b][i] *= alpha;
        }
        const float mb = (m_run == -INFINITY) ? 0.0f : m_run;
        // all exponent arguments first, in place, then all exponentials:
        // independent instructions back to back instead of 32 dependent
        // (argument, exponential) pairs through one temporary register
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kb2][i] = __builtin_fmaf(s[kb2][i], c2, -mb);
        asm volatile("" : "+v"(s[0]), "+v"(s[1]));
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kb2][i] = fast_exp2(s[kb2][i]);
        float lsum = 0.0f;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int i = 0; i < 16; ++i) lsum += s[kb2][i];
        l_run += lsum;
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
        // The same probabilities as the second product sees them (rounded
        // to 16 bits), summed exactly by dot products with (1, 1).  O is
        // divided by this sum, so the weights it applies to V are the
        // rounded probabilities normalised by their own total: a row
        // dominated by one key returns that key's V row up to fp32 rounding,
        // where dividing by the unrounded sum would leave the probability's
        // 16-bit rounding (up to 2^-9 relative in bf16) on the output.
        float rsum = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) rsum = dot2_ones<DT>(pf[c][e], rsum);
        r_run += rsum;
        if constexpr (KEEP_EARLY) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) pf[j][e] = keep_apply(pf[j][e], km[j][e]);
        } else if constexpr (DROP) {
            // keys t*BC + 32*kb2 + 16*g + 8*u + 0..7 (registers 8u..8u+7 of
            // s[kb2], i.e. pf[2*kb2 + u]) form the Philox block at counter
            // (8t + 4kb2 + 2g + u, query, bh, offset); word e decides the
            // keys 2e (low half) and 2e + 1 (high half) of the eight, the
            // halves of pf[2*kb2 + u][e]
            const uint32_t tm1 = p.drop_t - 1u;
            const uint32_t tm1x2 = tm1 | (tm1 << 16);
            const uint32_t c0 = (uint32_t)(8 * t + 2 * g);
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    uint32_t c[4] = {c0 + 4 * kb2 + u, (uint32_t)qrow, (uint32_t)bh, p.offset};
                    tile::philox4x32_10(c, p.seed_lo, p.seed_hi);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        pf[2 * kb2 + u][e] = drop_pair(pf[2 * kb2 + u][e], c[e], tm1x2, 0x00010001u);
                }
        }
    };

    // Instruction order of a matrix phase (P V then K Q^T: 32 MFMAs, 2*16
    // transposing V reads then 16 K reads): LDS reads run a few MFMAs ahead
    // of their use, so the matrix core does not wait on LDS latency.
    auto mphase_schedule = [&]() {
        constexpr int MFMA = 0x008, DSR = 0x100;
        constexpr int PV_N = 4 * DO, QK_N = 2 * DC;         // MFMAs of each product
        constexpr int AHEAD = 4;                            // MFMAs of lookahead
        __builtin_amdgcn_sched_group_barrier(DSR, 2 * AHEAD, 0);
#pragma unroll
        for (int m = 0; m < PV_N - AHEAD; ++m) {
            __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(DSR, 2, 0);
        }
#pragma unroll
        for (int m = 0; m < AHEAD; ++m) {
            __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(DSR, 1, 0);
        }
#pragma unroll
        for (int m = 0; m < QK_N - AHEAD; ++m) {
            __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(DSR, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(MFMA, AHEAD, 0);
    };
    // keys t*BC + 32*kb2 + 16*g + 8*u + 0..7 form the Philox block at
    // counter (8t + 4kb2 + 2g + u, query, bh, offset), as in swork
    auto make_keep = [&](int t) {
        if constexpr (KEEP_EARLY) {
            const uint32_t tm1 = p.drop_t - 1u;
            const uint32_t tm1x2 = tm1 | (tm1 << 16);
            const uint32_t c0 = (uint32_t)(8 * t + 2 * g);
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    uint32_t c[4] = {c0 + 4 * kb2 + u, (uint32_t)(qw0 + lq), (uint32_t)bh, p.offset};
                    tile::philox4x32_10(c, p.seed_lo, p.seed_hi);
#pragma unroll
                    for (int e = 0; e < 4; ++e) km[2 * kb2 + u][e] = keep_mult(c[e], tm1x2, 0x00010001u);
                }
        }
    };
    // matrix phase: O += P_tp V_tp, then S = K_t Q^T
    auto mphase2 = [&](int tp, int t) {
        __builtin_amdgcn_s_setprio(1);
        pv(tp);
        qk(t);
        mphase_schedule();
        make_keep(t);
        __builtin_amdgcn_s_setprio(0);
    };
    auto mphase = [&](int t) { mphase2(t - 1, t); };

    // Phase boundaries.  The one in the middle of a step only keeps the two
    // groups in alternation (no data passes through LDS across it).  The one
    // ending step t first waits for this wave's loads of tile t+1 (loads
    // complete in issue order, so at most those of tile t+2 stay in flight),
    // which together with the barrier publishes tile t+1 to every wave.
    auto mid_barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // mask_after: this wave issued the mask words of its next softmax phase
    // after its loads of tile t + 2, so those 8 loads may stay in flight too.
    auto end_barrier = [&](int t, bool mask_after) {
        if (t + 2 < nt) {
            if (MASK && mask_after) wait_vmcnt<2 * LPT + 8>();
            else wait_vmcnt<2 * LPT>();
        } else {
            wait_vmcnt<0>();
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };

    if constexpr (SPLIT) {
    // Key range split inside the workgroup (for grids smaller than the chip):
    // both groups own the same 128 query rows; group 0 takes the even K/V
    // tiles and group 1 the odd ones, with the same ping-pong, and their
    // partial (O, m, l) are merged through LDS at the end.  Step s handles
    // tiles 2s (group 0) and 2s + 1 (group 1); with an odd tile count group 1's
    // last tile lies past the block's keys and is fully masked (it is loaded,
    // so its values are finite and its probabilities exactly 0).  The ring has
    // eight slots; the loads of step s + 2 are issued during step s.
    const int ns = (nt + 1) >> 1;
    if constexpr (D == 128) {
    // At D = 128 the four-slot ring holds the split with loads one step
    // ahead: in step s group 1 loads K of tiles 2s + 2 and 2s + 3 (into the K
    // halves last read in step s - 1) and group 0, before its matrix phase,
    // V of tiles 2s and 2s + 1 (into the V halves last read in step s - 1).
    // Every load of step s is consumed in step s + 1, so each step ends with
    // all of them complete.
    auto end_split = [&]() {
        wait_vmcnt<0>();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };
    // With a mask each group reads the mask words of its own next tile
    // right after its tile loads and applies them at the start of its
    // softmax phase (every step ends with all loads complete).
    if constexpr (MASK) load_mask(grp);
    if (grp != 0) {
        issue_tile(0);
        issue_tile(1);
    }
    end_split();
    if (grp == 0) {
        issue_tile(0);
        issue_tile(1);
        qk(0);
        mid_barrier();
        if constexpr (MASK) {
            mask_scores();
            if (ns > 1) load_mask(2);
        }
        swork(0);
        end_split();
        for (int st = 1; st < ns; ++st) {
            issue_tile(2 * st);
            issue_tile(2 * st + 1);
            mphase2(2 * st - 2, 2 * st);
            mid_barrier();
            if constexpr (MASK) {
                mask_scores();
                if (st + 1 < ns) load_mask(2 * st + 2);
            }
            swork(2 * st);
            end_split();
        }
        pv(2 * ns - 2);
        mid_barrier();
    } else {
        if (ns > 1) {
            issue_tile(2);
            issue_tile(3);
        }
        mid_barrier();
        qk(1);
        end_split();
        for (int st = 1; st < ns; ++st) {
            if constexpr (MASK) mask_scores();
            if (st + 1 < ns) {
                issue_tile(2 * st + 2);
                issue_tile(2 * st + 3);
            }
            if constexpr (MASK) load_mask(2 * st + 1);
            swork(2 * st - 1);
            mid_barrier();
            mphase2(2 * st - 1, 2 * st + 1);
            end_split();
        }
        if constexpr (MASK) mask_scores();
        swork(2 * ns - 1);
        mid_barrier();
        pv(2 * ns - 1);
    }
    } else {
    auto issue_pair = [&](int st) { issue_tile(2 * st); issue_tile(2 * st + 1); };
    // mask_after: this wave requested mask words after this step's tile loads
    auto end_split = [&](int st, bool mask_after) {
        if (st + 2 < ns) {
            if (MASK && mask_after) wait_vmcnt<4 * LPT + 8>();
            else wait_vmcnt<4 * LPT>();
        } else {
            wait_vmcnt<0>();
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };
    if constexpr (MASK) load_mask(grp);
    issue_pair(0);
    if (ns > 1) issue_pair(1);
    end_split(-1, false);
    if (grp == 0) {
        qk(0);
        mid_barrier();
        if constexpr (MASK) mask_scores();
        if (ns > 2) issue_pair(2);
        if constexpr (MASK) if (ns > 1) load_mask(2);
        swork(0);
        end_split(0, true);
        for (int st = 1; st < ns; ++st) {
            mphase2(2 * st - 2, 2 * st);
            mid_barrier();
            if constexpr (MASK) mask_scores();
            if (st + 2 < ns) issue_pair(st + 2);
            if constexpr (MASK) if (st + 1 < ns) load_mask(2 * st + 2);
            swork(2 * st);
            end_split(st, true);
        }
        pv(2 * ns - 2);
        mid_barrier();
    } else {
        if (ns > 2) issue_pair(2);
        mid_barrier();
        qk(1);
        end_split(0, false);
        for (int st = 1; st < ns; ++st) {
            if constexpr (MASK) mask_scores();
            if (st + 2 < ns) issue_pair(st + 2);
            if constexpr (MASK) load_mask(2 * st + 1);
            swork(2 * st - 1);
            mid_barrier();
            mphase2(2 * st - 1, 2 * st + 1);
            end_split(st, true);
        }
        if constexpr (MASK) mask_scores();
        swork(2 * ns - 1);
        mid_barrier();
        pv(2 * ns - 1);
    }
    }
    store_tiles();
    // Merge: group 1 hands its O accumulators, running max and sum to the
    // wave of group 0 that owns the same rows (same lane layout), which
    // rescales both to the larger max and adds them.
    float* const xbuf = (float*)smem;
    const int xb = (wid & 3) * (DB * 16 + 3) * 64 + lane;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    if (grp != 0) {
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) xbuf[xb + (16 * b + i) * 64] = oacc[b][i];
        xbuf[xb + 16 * DB * 64] = m_run;
        xbuf[xb + (16 * DB + 1) * 64] = l_run;
        xbuf[xb + (16 * DB + 2) * 64] = r_run;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    if (grp != 0) return;
    {
        const float m1 = xbuf[xb + 16 * DB * 64];
        const float l1 = xbuf[xb + (16 * DB + 1) * 64];
        const float m = fmaxf(m_run, m1);
        float a0 = 0.0f, a1 = 0.0f;
        if (m != -INFINITY) {
            a0 = fast_exp2(m_run - m);
            a1 = fast_exp2(m1 - m);
        }
        l_run = a0 * l_run + a1 * l1;
        r_run = a0 * r_run + a1 * xbuf[xb + (16 * DB + 2) * 64];
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[b][i] = a0 * oacc[b][i] + a1 * xbuf[xb + (16 * b + i) * 64];
        m_run = m;
    }
    } else if constexpr (DSPLIT) {
    // Pair split (D = 256).  Waves w and w ^ 1 of one group own the same 32
    // query rows; wave w takes the keys 32h .. 32h + 31 of every tile
    // (h = w & 1) -- their scores S_h = K_h Q^T over the full head dimension,
    // masking, row max and probabilities -- and O's columns 128h .. 128h + 127,
    // for which it also needs the mate's probabilities.  The two groups own
    // different rows and alternate phases as in the other instances.  In a
    // matrix phase a wave reads the mate's packed probabilities of the
    // previous tile from LDS, computes S_h of this tile, then O += P V with
    // the full P, masks S_h and publishes its row max in LDS; in the softmax
    // phase it takes the larger of the pair's two maxima (both waves of a
    // pair therefore keep the same running max), forms its probabilities and
    // publishes them packed.  Barriers between the phases carry these LDS
    // exchanges.  A wave keeps its own probabilities in pf[0..1] and the
    // mate's in pf[2..3] and reads the V rows of each from their key half.
    // The K/V ring has two slots of 64 KiB (a 32 KiB K tile and a 32 KiB V
    // tile): in step t group 1 loads K of tile t + 1 (into the K half whose
    // tile t - 1 was last read in step t - 1) and group 0, before its matrix
    // phase, V of tile t (into the V half last read in step t - 1); every
    // step ends with all its loads complete.  The mask words of a tile are
    // requested in the matrix phase before, after that phase applied its own.
    const int h = wid & 1, mate = wid ^ 1;
    float* const xmax = (float*)(smem + NSLOT * SLOT_BYTES);
    i32x4* const xp = (i32x4*)(smem + NSLOT * SLOT_BYTES + XMAX_BYTES);
    auto end_step = [&]() {
        wait_vmcnt<0>();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };
    auto mid_step = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };
    // mask bytes of this lane's query row for the keys 32h + 16g + 4j .. +3
    // of tile t (register 4j + e of S_h: byte e of mkh[j])
    uint32_t mkh[4];
    auto load_mask_half = [&](int t) {
        const int qrow = qw0 + lq;
        const uint32_t row = qrow < Sq ? (uint32_t)qrow * (uint32_t)p.m_ss + (uint32_t)(t * BC + 32 * h + 16 * g)
                                       : 0x80000000u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            mkh[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rm, row + 4 * j, 0, 0);
            asm volatile("" ::: "memory");
        }
    };
    auto qk_half = [&](int t) {
        const int kb = (t & (NSLOT - 1)) * SLOT_BYTES + kbase_l;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[0][i] = 0.0f;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            const i32x4 a = *(const i32x4*)(smem + (kb ^ (c << 5)) + h * 32 * (2 * D));
            s[0] = mfma32<DT>(a, qf[c], s[0]);
        }
    };
    auto pv_pair = [&](int tp) {
        const int vb = (tp & (NSLOT - 1)) * SLOT_BYTES + TILE_BYTES + vbase_l;
        const int vown = 32 * h * (2 * D), vmate = 32 * (1 - h) * (2 * D);
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
            for (int b = 0; b < DO; ++b) {
                const int off = (vb ^ ((b + dob) << 6)) + (kc < 2 ? vown : vmate) + 8 * (kc & 1) * (2 * D);
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4*)(smem + off));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4*)(smem + off + 4 * (2 * D)));
                i32x4 a;
                a[0] = __builtin_bit_cast(int, (short __attribute__((ext_vector_type(2)))){lo[0], lo[1]});
                a[1] = __builtin_bit_cast(int, (short __attribute__((ext_vector_type(2)))){lo[2], lo[3]});
                a[2] = __builtin_bit_cast(int, (short __attribute__((ext_vector_type(2)))){hi[0], hi[1]});
                a[3] = __builtin_bit_cast(int, (short __attribute__((ext_vector_type(2)))){hi[2], hi[3]});
                oacc[b] = mfma32<DT>(a, pf[kc], oacc[b]);
            }
        }
    };
    auto get_mate_p = [&]() {
        pf[2] = xp[(2 * mate) * 64 + lane];
        pf[3] = xp[(2 * mate + 1) * 64 + lane];
    };
    // hidden keys of S_h to -inf, then its row max (times scale log2 e),
    // published for the mate
    float mxh = -INFINITY;
    auto mask_max = [&](int t) {
        const int key0 = t * BC + 32 * h + 16 * g;
        const int qrow = qw0 + lq;
        const bool need_mask = (t * BC + 32 * h + 32 > Sk) || (CAUSAL && t * BC + 32 * h + 31 > qw0 + diag);
        if (need_mask) {
            const int lim = CAUSAL ? min(qrow + diag, Sk - 1) : Sk - 1;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (key0 + i > lim) s[0][i] = -INFINITY;
        }
        if constexpr (MASK) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (((mkh[i >> 2] >> (8 * (i & 3))) & 0xffu) == 0) s[0][i] = -INFINITY;
        }
        float mx = s[0][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
        mxh = xmax32(mx) * c2;
        xmax[wid * 64 + lane] = mxh;
    };
    // Instruction order of a matrix phase (S_h = K_h Q^T then O += P V: 16 + 16
    // MFMAs after the mate's two probability words; 16 K reads, then two
    // transposing V reads per P V MFMA): LDS reads run four MFMAs ahead.
    auto mphase_pair_schedule = [&]() {
        constexpr int MFMA = 0x008, DSR = 0x100;
        constexpr int QK_N = DC, PV_N = 4 * DO, AHEAD = 4;
        __builtin_amdgcn_sched_group_barrier(DSR, 2 + AHEAD, 0);
#pragma unroll
        for (int m = 0; m < QK_N - AHEAD; ++m) {
            __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(DSR, 1, 0);
        }
#pragma unroll
        for (int m = 0; m < PV_N; ++m) {
            __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(DSR, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(MFMA, AHEAD, 0);
    };
    auto mphase_pair = [&](int tp, int t) {
        __builtin_amdgcn_s_setprio(1);
        get_mate_p();
        qk_half(t);
        pv_pair(tp);
        mphase_pair_schedule();
        __builtin_amdgcn_s_setprio(0);
        mask_max(t);
    };
    // probabilities of this wave's keys of tile t against the pair's max
    auto swork_half = [&](int t) {
        if constexpr (DIAG) ++ntiles;
        const float mx = fmaxf(mxh, xmax[mate * 64 + lane]);
        const bool grow = mx > m_run + RESCALE_THRESHOLD;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
            r_run *= alpha;
#pragma unroll
            for (int b = 0; b < DO; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[b][i] *= alpha;
        }
        const float mb = (m_run == -INFINITY) ? 0.0f : m_run;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[0][i] = __builtin_fmaf(s[0][i], c2, -mb);
        asm volatile("" : "+v"(s[0]));
#pragma unroll
        for (int i = 0; i < 16; ++i) s[0][i] = fast_exp2(s[0][i]);
        float lsum = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) lsum += s[0][i];
        l_run += lsum;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            i32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = pack2<DT>(s[0][8 * c + 2 * e], s[0][8 * c + 2 * e + 1]);
            pf[c] = w;
        }
        // O's divisor: the probabilities as rounded for P V (see swork)
        float rsum = 0.0f;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) rsum = dot2_ones<DT>(pf[c][e], rsum);
        r_run += rsum;
        if constexpr (DROP) {
            // keys t*BC + 32h + 16g + 8u + 0..7 (pf[u]) form the Philox block
            // at counter (8t + 4h + 2g + u, query, bh, offset)
            const uint32_t tm1 = p.drop_t - 1u;
            const uint32_t tm1x2 = tm1 | (tm1 << 16);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                uint32_t c[4] = {(uint32_t)(8 * t + 4 * h + 2 * g + u), (uint32_t)(qw0 + lq), (uint32_t)bh, p.offset};
                tile::philox4x32_10(c, p.seed_lo, p.seed_hi);
#pragma unroll
                for (int e = 0; e < 4; ++e) pf[u][e] = drop_pair(pf[u][e], c[e], tm1x2, 0x00010001u);
            }
        }
        xp[(2 * wid) * 64 + lane] = pf[0];
        xp[(2 * wid + 1) * 64 + lane] = pf[1];
    };

    if constexpr (MASK) load_mask_half(0);
    if (grp != 0) issue_tile(0);
    end_step();
    if (grp == 0) {
        issue_tile(0);
        qk_half(0);
        mask_max(0);
        if constexpr (MASK) if (nt > 1) load_mask_half(1);
        mid_step();
        swork_half(0);
        end_step();
        for (int t = 1; t < nt; ++t) {
            issue_tile(t);
            mphase_pair(t - 1, t);
            if constexpr (MASK) if (t + 1 < nt) load_mask_half(t + 1);
            mid_step();
            swork_half(t);
            end_step();
        }
        get_mate_p();
        pv_pair(nt - 1);
        mid_step();
    } else {
        if (nt > 1) issue_tile(1);
        mid_step();
        qk_half(0);
        mask_max(0);
        if constexpr (MASK) if (nt > 1) load_mask_half(1);
        end_step();
        for (int t = 1; t < nt; ++t) {
            if (t + 1 < nt) issue_tile(t + 1);
            swork_half(t - 1);
            mid_step();
            mphase_pair(t - 1, t);
            if constexpr (MASK) if (t + 1 < nt) load_mask_half(t + 1);
            end_step();
        }
        swork_half(nt - 1);
        mid_step();
        get_mate_p();
        pv_pair(nt - 1);
    }
    // the pair's partial sums: both waves add them in the same order (h = 0
    // first), so both hold the same totals.  The region of the row maxima is
    // free: its last reads came before the last barrier.
    {
        float* const xl = (float*)(smem + NSLOT * SLOT_BYTES);
        xl[(2 * wid) * 64 + lane] = l_run;
        xl[(2 * wid + 1) * 64 + lane] = r_run;
        mid_step();
        const float l_mate = xl[(2 * mate) * 64 + lane];
        const float r_mate = xl[(2 * mate + 1) * 64 + lane];
        l_run = h ? l_mate + l_run : l_run + l_mate;
        r_run = h ? r_mate + r_run : r_run + r_mate;
    }
    } else {
    // Prologue: Q, tile 0 and tile 1 requested; tile 0 (and Q) waited for.
    if constexpr (MASK) load_mask(0);
    issue_tile(0);
    if (nt > 1) issue_tile(1);
    end_barrier(-1, false);

    // The two groups run the same sequence of barriers (two per step for
    // steps 0 .. nt-1, one for the final step) with their phases swapped.
    // Step 0: S_0 = K_0 Q^T.  Steps 1 .. nt-1: O += P_{t-1} V_{t-1} and
    // S_t = K_t Q^T in the matrix phase, softmax of S_t in the other.
    // Step nt: the last O += P V.
    if (grp == 0) {
        qk(0);
        make_keep(0);
        mid_barrier();
        if constexpr (MASK) mask_scores();
        if (nt > 2) issue_tile(2);
        if constexpr (MASK) if (nt > 1) load_mask(1);
        swork(0);
        end_barrier(0, true);
        for (int t = 1; t < nt; ++t) {
            mphase(t);
            mid_barrier();
            if constexpr (MASK) mask_scores();
            if (t + 2 < nt) issue_tile(t + 2);
            if constexpr (MASK) if (t + 1 < nt) load_mask(t + 1);
            swork(t);
            end_barrier(t, true);
        }
        pv(nt - 1);
        mid_barrier();
    } else {
        if (nt > 2) issue_tile(2);
        mid_barrier();
        qk(0);
        make_keep(0);
        end_barrier(0, false);
        for (int t = 1; t < nt; ++t) {
            if constexpr (MASK) mask_scores();
            if (t + 2 < nt) issue_tile(t + 2);
            if constexpr (MASK) load_mask(t);
            swork(t - 1);
            mid_barrier();
            mphase(t);
            end_barrier(t, true);
        }
        if constexpr (MASK) mask_scores();
        swork(nt - 1);
        mid_barrier();
        pv(nt - 1);
    }
    }

    if constexpr (!SPLIT) store_tiles();
    const float l_tot = xsum32(l_run);
    const float r_tot = xsum32(r_run);
    // with dropout the kept weights are scaled by 65536 / (65536 - t)
    const float inv = r_tot > 0.0f ? (DROP ? p.keep_scale : 1.0f) / r_tot : 0.0f;
    const int qrow = qw0 + lq;
    if constexpr (DIAG) {
        if (p.o32 != nullptr) {
            // fp32 O, contiguous [B*H, Sq, D]; rows past the sequence dropped
            const __amdgpu_buffer_rsrc_t r32 =
                make_rsrc(p.o32 + (int64_t)bh * Sq * D, (uint32_t)((int64_t)Sq * D * 4));
#pragma unroll
            for (int b = 0; b < DO; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    f32x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = oacc[b][4 * j + e] * inv;
                    const uint32_t off = ((uint32_t)qrow * D + 32 * b + 16 * g + 4 * j) * 4;
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, w), r32, off, 0, 0);
                }
        }
    }
#pragma unroll
    for (int b = 0; b < DO; ++b) {
        i32x4 w0, w1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            w0[e] = pack2<DT>(oacc[b][2 * e] * inv, oacc[b][2 * e + 1] * inv);
            w1[e] = pack2<DT>(oacc[b][8 + 2 * e] * inv, oacc[b][8 + 2 * e + 1] * inv);
        }
        const uint32_t off = ((uint32_t)qrow * p.o_ss + 32 * (b + dob) + 16 * g) * 2;
        __builtin_amdgcn_raw_buffer_store_b128(w0, ro, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(w1, ro, off + 16, 0, 0);
    }
    if (p.lse != nullptr && g == 0 && qrow < Sq && (!DSPLIT || (wid & 1) == 0)) {
        const float lse2 = (l_tot > 0.0f) ? (m_run == -INFINITY ? 0.0f : m_run) + log2f(l_tot) : -INFINITY;
        p.lse[(int64_t)bh * Sq + qrow] = lse2 * 0.69314718055994530942f;
    }
}

}  // namespace fa
