// fa_tile.h -- device helpers shared by the backward and the masked/dropout
// forward kernels: MFMA wrapper, 16-bit packing, LDS tile swizzle, operand
// fragments by rows and by transposing reads, XCD-aware block order.
//
// Operand layout of v_mfma_f32_32x32x16: lane l supplies row (A) or column
// (B) l%32 and the 8 k-values in slots 8*(l/32)..+7; accumulator register r
// of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.  Taking the
// accumulator of one product as an operand of the next makes k-slot e of
// lane half g in k-step s stand for row 16*s + 8*(e/4) + 4*g + e%4; the LDS
// operand of that product is read with the same mapping: two transposing
// reads, each of four consecutive rows.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {
namespace tile {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_t;

constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             (int)(bytes < 0x80000000ull ? bytes : 0x7fffffffull),
                                             (int)0x00020000);
}

template <int DT>
__device__ __forceinline__ f32x16 mma(i32x4 a, i32x4 b, f32x16 c) {
    if constexpr (DT == 0)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two fp32 -> one dword of two 16-bit values (round to nearest even).
template <int DT>
__device__ __forceinline__ int pack2(float x, float y) {
    if constexpr (DT == 0)
        return __builtin_bit_cast(int, __builtin_convertvector((f32x2){x, y}, f16x2));
    else
        return __builtin_bit_cast(int, __builtin_convertvector((f32x2){x, y}, bf16x2));
}

// The 16-bit value in the low (hi = 0) or high half of a dword, as fp32.
template <int DT>
__device__ __forceinline__ float half_f32(int w, int hi) {
    const uint32_t h = ((uint32_t)w >> (16 * hi)) & 0xffffu;
    if constexpr (DT == 0)
        return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
    else
        return __uint_as_float(h << 16);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

// LDS tiles are [rows][W] 16-bit values (W = 32, 64, 128 or 256), stored in
// 16-byte chunks whose index within the row is XOR-ed with swz(row).  With
// 64 banks of 4 bytes, a fragment read (ds_read_b128: 16 lanes on 16
// consecutive rows, one chunk each) and a transposing read
// (ds_read_b64_tr_b16: 32 lanes on four consecutive rows, four adjacent
// chunks each) both fall on distinct banks:
//   W >= 128 (rows of 256 or 512 bytes): the two low bits of the row pick the
//     4-chunk group, the next two the chunk within it;
//   W = 64 (128-byte rows, two rows per bank period): the row's parity picks
//     the bank half, bit 1 the 4-chunk group, bits 2-3 the chunk in it;
//   W = 32 (64-byte rows, only read transposed): four consecutive rows
//     already cover all banks.
template <int W>
__device__ __forceinline__ int swz(int r) {
    if constexpr (W == 32) return 0;
    if constexpr (W >= 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}
template <int W>
__device__ __forceinline__ int toff(int r, int ch) {
    return r * (2 * W) + ((ch ^ swz<W>(r)) << 4);
}

// Operand fragment by rows: 8 consecutive values (chunk ch) of row r.
template <int W>
__device__ __forceinline__ i32x4 row_frag(const lds_t* tile, int r, int ch) {
    return *(const __attribute__((address_space(3))) i32x4*)(tile + toff<W>(r, ch));
}

// Per-lane constants of the transposing reads: source lane 4j + t of each
// 16-lane group G addresses row 4*(G/2) + j (+16 s, +8 for the second read)
// and columns 16*(G%2) + 4t .. +3 of a 32-column block.
struct TrLane {
    int row, ch, byte;
};
__device__ __forceinline__ TrLane tr_lane(int lane) {
    const int G = lane >> 4, m = lane & 15;
    return {4 * (G >> 1) + (m >> 2), 2 * (G & 1) + ((m & 3) >> 1), (m & 1) * 8};
}

// Operand fragment of column block b (columns 32b + lane%32) over rows
// 16s .. 16s+15 in the k-slot order above.
template <int W>
__device__ __forceinline__ i32x4 tr_frag(const lds_t* tile, int s, int b, const TrLane& tl) {
    const int r0 = 16 * s + tl.row, r1 = r0 + 8, ch = 4 * b + tl.ch;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(tile + r0 * (2 * W) + ((ch ^ swz<W>(r0)) << 4) + tl.byte));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(tile + r1 * (2 * W) + ((ch ^ swz<W>(r1)) << 4) + tl.byte));
    i32x4 a;
    a[0] = (int)(uint16_t)lo[0] | ((int)(uint16_t)lo[1] << 16);
    a[1] = (int)(uint16_t)lo[2] | ((int)(uint16_t)lo[3] << 16);
    a[2] = (int)(uint16_t)hi[0] | ((int)(uint16_t)hi[1] << 16);
    a[3] = (int)(uint16_t)hi[2] | ((int)(uint16_t)hi[3] << 16);
    return a;
}

// Per-lane byte offsets of the fragment reads above, computed once.  The
// swizzle depends on a row's index mod 16 and changes only the low four bits
// of a chunk index, so for row reads (chunk 2c + g of row r0 + lq, r0 a
// multiple of 16) the offsets of c < 8 serve every c, the chunk of c + 8
// lying 256 bytes further; for transposing reads (rows 16s + tl.row (+8),
// chunks 4b + tl.ch) the offsets of b < 4 serve every b (256 bytes per four
// blocks) and every s (16 rows).
template <int W>
struct FragOff {
    static constexpr int NR = W / 16 < 8 ? W / 16 : 8;
    static constexpr int NT = W / 32 < 4 ? W / 32 : 4;
    uint32_t rx[NR];
    uint32_t tx[2][NT];
    __device__ __forceinline__ FragOff(int lane, const TrLane& tl) {
        const int lq = lane & 31, g = lane >> 5;
#pragma unroll
        for (int k = 0; k < NR; ++k) rx[k] = (uint32_t)(lq * (2 * W) + (((2 * k + g) ^ swz<W>(lq)) << 4));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = tl.row + 8 * h;
#pragma unroll
            for (int k = 0; k < NT; ++k)
                tx[h][k] = (uint32_t)(r * (2 * W) + (((4 * k + tl.ch) ^ swz<W>(r)) << 4) + tl.byte);
        }
    }
    // row_frag(tile, r0 + lq, 2c + g)
    __device__ __forceinline__ i32x4 row(const lds_t* tile, int r0, int c) const {
        return *(const __attribute__((address_space(3))) i32x4*)(tile + r0 * (2 * W) + rx[c % NR] + 256 * (c / NR));
    }
    // tr_frag(tile, s, b, tl)
    __device__ __forceinline__ i32x4 tr(const lds_t* tile, int s, int b) const {
        const lds_t* t = tile + 16 * s * (2 * W) + 256 * (b / NT);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(t + tx[0][b % NT]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(t + tx[1][b % NT]));
        i32x4 a;
        a[0] = (int)(uint16_t)lo[0] | ((int)(uint16_t)lo[1] << 16);
        a[1] = (int)(uint16_t)lo[2] | ((int)(uint16_t)lo[3] << 16);
        a[2] = (int)(uint16_t)hi[0] | ((int)(uint16_t)hi[1] << 16);
        a[3] = (int)(uint16_t)hi[2] | ((int)(uint16_t)hi[3] << 16);
        return a;
    }
};

// The same reads with two registers per read kind: the swizzle is an XOR of
// a chunk index with a per-lane mask, so an address is
// (16 * chunk step) ^ (16 * mask) + per-lane base, one v_xad_u32 per read.
template <int W>
struct FragXor {
    uint32_t rb, rm;                                       // row reads
    uint32_t tb[2], tm[2];                                 // transposing reads
    __device__ __forceinline__ FragXor(int lane, const TrLane& tl) {
        const int lq = lane & 31, g = lane >> 5;
        rb = (uint32_t)(lq * (2 * W));
        rm = (uint32_t)((g ^ swz<W>(lq)) << 4);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = tl.row + 8 * h;
            tb[h] = (uint32_t)(r * (2 * W) + tl.byte);
            tm[h] = (uint32_t)((tl.ch ^ swz<W>(r)) << 4);
        }
    }
    // row_frag(tile, r0 + lq, 2c + g)
    __device__ __forceinline__ i32x4 row(const lds_t* tile, int r0, int c) const {
        const uint32_t off = ((uint32_t)(32 * c) ^ rm) + rb;
        return *(const __attribute__((address_space(3))) i32x4*)(tile + r0 * (2 * W) + off);
    }
    // tr_frag(tile, s, b, tl)
    __device__ __forceinline__ i32x4 tr(const lds_t* tile, int s, int b) const {
        const lds_t* t = tile + 16 * s * (2 * W);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(t + (((uint32_t)(64 * b) ^ tm[0]) + tb[0])));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(t + (((uint32_t)(64 * b) ^ tm[1]) + tb[1])));
        i32x4 a;
        a[0] = (int)(uint16_t)lo[0] | ((int)(uint16_t)lo[1] << 16);
        a[1] = (int)(uint16_t)lo[2] | ((int)(uint16_t)lo[3] << 16);
        a[2] = (int)(uint16_t)hi[0] | ((int)(uint16_t)hi[1] << 16);
        a[3] = (int)(uint16_t)hi[2] | ((int)(uint16_t)hi[3] << 16);
        return a;
    }
};

// B operand of k-step s from a 32-row-block pair of accumulators (rows
// 32*(s/2) .. of the product), packed to 16 bits.
template <int DT>
__device__ __forceinline__ i32x4 acc_frag(const f32x16& x, int h) {
    i32x4 a;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = pack2<DT>(x[8 * h + 2 * i], x[8 * h + 2 * i + 1]);
    return a;
}

// Workgroup -> (batch*head, block).  When the head count is a multiple of 8,
// each XCD (workgroup ids are dealt round-robin over the 8 XCDs) takes a
// contiguous range of heads, so the blocks of a head share one L2.  Blocks
// of a head come in slot order; `reverse` hands out the last block first.
__device__ __forceinline__ void block_order(int wg, int nblk, int BH, bool reverse, int& bh, int& blk) {
    int slot;
    if ((BH & 7) == 0) {
        const int xcd = wg & 7, k = wg >> 3, hpx = BH >> 3;
        bh = xcd * hpx + k % hpx;
        slot = k / hpx;
    } else {
        bh = wg % BH;
        slot = wg / BH;
    }
    blk = reverse ? (nblk - 1 - slot) : slot;
}

// Direct global->LDS load of 16 bytes per lane: lane l's 16 bytes at byte
// offset `voffset` of the buffer go to LDS address lds_addr + 16*l
// (lds_addr wave-uniform).  Written as inline assembly (it sets M0, which
// nothing else in these kernels uses); the compiler does not see it, so the
// caller waits for it with wait_vmcnt before the barrier that publishes the
// tile.
__device__ __forceinline__ void lds_dma16(i32x4 rsrc_words, uint32_t voffset, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voffset), "s"(rsrc_words), "s"(lds_addr) : "memory", "m0");
}

// As lds_dma16 with 4 bytes per lane (LDS address lds_addr + 4*l).
__device__ __forceinline__ void lds_dma4(i32x4 rsrc_words, uint32_t voffset, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :: "v"(voffset), "s"(rsrc_words), "s"(lds_addr) : "memory", "m0");
}

// Philox4x32-10 block function (Salmon et al., "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds of two 32x32->64 multiplications
// (0xD2511F53, 0xCD9E8D57) whose high halves are XOR-ed with the other two
// counter words and the key; the key is bumped by (0x9E3779B9, 0xBB67AE85)
// between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        // one 32x32->64 multiply-add per product (v_mad_u64_u32 gives both
        // halves) and one three-input XOR (v_bitop3_b32, truth table 0x96)
        const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32(hi1, c[1], k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32(hi0, c[3], k1, 0x96);
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
    }
}

// The dropout words a lane needs for the S^T accumulator layout of a tile of
// RB 32-key blocks (lane l holds query lq = l % 32 and, in register 4a + e of
// block rb, key kt0 + 32 rb + 8a + 4g + e, g = l / 32): for each (rb, a) the
// two words 2g, 2g + 1 of the Philox4x32-10 block at counter
// ((kt0 + 32 rb + 8a) / 8, qi, bh, offset) -- the block covers the 8 keys
// 8a .. 8a + 7, a lane uses the four of them it holds.  Lanes l and l ^ 32
// (the same query) need the two halves of the same blocks, so each computes
// the blocks of two of the four 8-key groups (lane half g: a = 2g, 2g + 1)
// and hands the partner the two words it needs (v_permlane32_swap): four
// Philox blocks per lane and tile instead of eight.
template <int RB>
__device__ __forceinline__ void keep_words(uint32_t kw[RB][4][2], int kt0, int qi, int bh, uint32_t offset,
                                           uint32_t seed_lo, uint32_t seed_hi, int g) {
    auto partner = [&](uint32_t x) {
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return g ? (uint32_t)r[0] : (uint32_t)r[1];
    };
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            uint32_t c[4] = {(uint32_t)((kt0 + 32 * rb + 8 * (2 * g + u)) >> 3), (uint32_t)qi, (uint32_t)bh, offset};
            philox4x32_10(c, seed_lo, seed_hi);
            const uint32_t k0 = g ? c[2] : c[0], k1 = g ? c[3] : c[1];   // this lane's words of group 2g + u
            const uint32_t r0 = partner(g ? c[0] : c[2]);                // the partner's words of group
            const uint32_t r1 = partner(g ? c[1] : c[3]);                // 2(1 - g) + u, computed there
            kw[rb][u][0] = g ? r0 : k0;
            kw[rb][u][1] = g ? r1 : k1;
            kw[rb][2 + u][0] = g ? k0 : r0;
            kw[rb][2 + u][1] = g ? k1 : r1;
        }
    }
}

// s_waitcnt vmcnt(N) alone (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Buffer descriptor as four wave-uniform dwords (for the inline assembly):
// base, stride 0, `bytes` records, raw 32-bit format.
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint64_t bytes) {
    const uint64_t a = (uint64_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffff));
    r[2] = __builtin_amdgcn_readfirstlane((int)(bytes < 0x80000000ull ? bytes : 0x7fffffffull));
    r[3] = 0x00020000;
    return r;
}

// Direct loads of one [rows][W] 16-bit tile (rows = 256 * N / (W / 8), i.e.
// N instructions per thread of a 256-thread workgroup) into the swizzled LDS
// layout of toff(): instruction i of wave w fills LDS chunks
// (4i + w)*64 + lane, and each lane fetches the global chunk that the swizzle
// puts there.  row0: first global row; ss: global row stride in elements.
template <int W, int N>
__device__ __forceinline__ void tile_dma(i32x4 rw, int row0, int ss, uint32_t lds_tile, int w, int lane) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int c = (4 * i + w) * 64 + lane;
        const int r = c / (W / 8), pos = c % (W / 8);
        const int ch = pos ^ swz<W>(r);
        lds_dma16(rw, (uint32_t)(((row0 + r) * ss + 8 * ch) * 2), lds_tile + (uint32_t)((4 * i + w) * 1024));
    }
}

// The loads of tile_dma with the per-lane part of each offset computed once.
// Load i of a wave covers rows i*STEP + w*RPI + lane/(W/8), so its rows
// repeat the swizzle pattern (period 16 rows) every NC loads: the lane parts
// take NC values, kept in registers, and the rest is a wave-uniform row
// offset added at issue time (kept opaque so the sums are not precomputed
// into N registers).  Offsets stay whole in the vector operand, so rows
// past the buffer's end still read as zero.
template <int W, int N>
struct TileDma {
    static constexpr int RPI = 512 / W;                         // rows per load instruction
    static constexpr int STEP = 4 * RPI;                        // rows between loads i and i+1
    static constexpr int NC0 = (STEP % 16) ? 16 / (STEP % 16) : 1;
    static constexpr int NC = NC0 < N ? NC0 : N;
    static_assert(16 % ((STEP % 16) ? STEP % 16 : 16) == 0, "swizzle period");
    uint32_t lo[NC];
    int ss;
    __device__ __forceinline__ TileDma(int ss_, int w, int lane) : ss(ss_) {
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int r = k * STEP + w * RPI + lane / (W / 8), pos = lane % (W / 8);
            lo[k] = (uint32_t)((r * ss + 8 * (pos ^ swz<W>(r))) * 2);
        }
    }
    __device__ __forceinline__ void issue(i32x4 rw, int row0, uint32_t lds_tile, int w) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            int u = (row0 + (i / NC) * NC * STEP) * ss * 2;
            asm volatile("" : "+s"(u));
            lds_dma16(rw, lo[i % NC] + (uint32_t)u, lds_tile + (uint32_t)((4 * i + w) * 1024));
        }
    }
};

}  // namespace tile
}  // namespace fa
