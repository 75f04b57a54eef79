// fa_naive.hip -- unfused attention forward for gfx950: the comparison path.
//
// The three-step flow the pages describe before fusing it -- scores
// S = scale * Q K^T written to device memory, a row softmax producing P in
// device memory, then O = P V -- built from this library's own kernels:
//   naive_scores   S (fp32) = scale * Q K^T with the causal mask applied
//                  (-inf), an MFMA GEMM over the head dimension;
//   naive_softmax  P (input dtype) = exp(S - row max) of each row, the
//                  reciprocal of the sum of those rounded values, and the
//                  row's natural-log log-sum-exp;
//   naive_vt       V^T per head, so that the second product reads both
//                  operands along the key dimension;
//   naive_pv       O = P V, an MFMA GEMM over the keys, times that
//                  reciprocal.
// "FlashAttention-2 on Ascend NPU: how ops-transformer reaches 3x"
// (2048ai.net), section 1 (the N x N matrices S and P materialised), and
// "ops-transformer FlashAttention operator in practice" (ai6s.net),
// section 1 (scores, softmax, multiply by V) and section 4 (the naive
// baseline the fused operator is measured against).
//
// Workspace layout (caller-allocated, see fa_naive_workspace_bytes): per head
// S as Sq x Skp fp32, then P as Sq x Skp of the input dtype, then V^T as
// D x Skp, with Skp = Sk rounded up to a multiple of 64 and the padding
// columns zero in P and V^T.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_naive.h"

namespace fa {
namespace naive {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

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

template <int DT>
__device__ __forceinline__ float from16(uint16_t h) {
    if constexpr (DT == 0) return (float)__builtin_bit_cast(_Float16, h);
    else return __uint_as_float((uint32_t)h << 16);
}

template <int DT>
__device__ __forceinline__ uint16_t to16(float x) {
    if constexpr (DT == 0) {
        _Float16 h = (_Float16)x;
        return __builtin_bit_cast(uint16_t, h);
    } else {
        __bf16 h = (__bf16)x;
        return __builtin_bit_cast(uint16_t, h);
    }
}

// In the 32x32 accumulator, register i of lane l holds row
// 8*(i/4) + 4*(l/32) + i%4 and column l%32.  Operand fragments: lane l
// supplies row (A) or column (B) l%32 and 8 consecutive k values from
// 8*(l/32) on, i.e. 16 contiguous bytes of a row-major operand.
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// S = scale * Q K^T, 128 x 128 output tile per workgroup, 64 x 64 per wave.
template <int D, int DT>
__global__ __launch_bounds__(256) void naive_scores(NaiveParams p) {
    const int bh = blockIdx.z;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r0 = blockIdx.y * 128 + (w >> 1) * 64;
    const int c0 = blockIdx.x * 128 + (w & 1) * 64;
    const __amdgpu_buffer_rsrc_t rq = rsrc((const char*)p.q + (int64_t)bh * p.Sq * D * 2, (uint64_t)p.Sq * D * 2);
    const __amdgpu_buffer_rsrc_t rk = rsrc((const char*)p.k + (int64_t)bh * p.Sk * D * 2, (uint64_t)p.Sk * D * 2);
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;
    const int kq = 8 * (lane >> 5);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
        i32x4 af[2], bf[2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
            af[a] = __builtin_amdgcn_raw_buffer_load_b128(rq, ((r0 + 32 * a + (lane & 31)) * D + 16 * c + kq) * 2, 0, 0);
#pragma unroll
        for (int b = 0; b < 2; ++b)
            bf[b] = __builtin_amdgcn_raw_buffer_load_b128(rk, ((c0 + 32 * b + (lane & 31)) * D + 16 * c + kq) * 2, 0, 0);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) acc[a][b] = mma<DT>(af[a], bf[b], acc[a][b]);
    }
    float* S = p.s + (int64_t)bh * p.Sq * p.Skp;
    const int diag = p.Sk - p.Sq;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int col = c0 + 32 * b + (lane & 31);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = r0 + 32 * a + acc_row(i, lane);
                if (row < p.Sq && col < p.Sk) {
                    const bool hidden = p.causal && col > row + diag;
                    S[(int64_t)row * p.Skp + col] = hidden ? -INFINITY : acc[a][b][i] * p.scale;
                }
            }
        }
}

// One workgroup per row: P = exp(s - max) / sum (zero in the padding
// columns), lse = max + ln(sum); a row with no visible key gets P = 0 and
// lse = -inf.  NE values per thread (256 * NE >= Skp).
template <int DT, int NE>
__global__ __launch_bounds__(256) void naive_softmax(NaiveParams p) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x;                 // bh * Sq + i
    const float* s = p.s + row * p.Skp;
    uint16_t* P = p.p + row * p.Skp;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    float x[NE];
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const int j = tid + 256 * e;
        x[e] = j < p.Sk ? s[j] : -INFINITY;
        m = fmaxf(m, x[e]);
    }
    auto block_reduce = [&](float v, bool is_max) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const float u = __shfl_xor(v, o);
            v = is_max ? fmaxf(v, u) : v + u;
        }
        __syncthreads();
        if (lane == 0) red[w] = v;
        __syncthreads();
        return is_max ? fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))
                      : (red[0] + red[1]) + (red[2] + red[3]);
    };
    m = block_reduce(m, true);
    const float mb = m == -INFINITY ? 0.0f : m;
    float l = 0.0f;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        x[e] = __expf(x[e] - mb);
        l += x[e];
    }
    l = block_reduce(l, false);
    // P is stored unnormalised (the largest entry exactly 1) and O is divided
    // by the sum of the stored, rounded values: the weights applied to V are
    // then the rounded probabilities normalised by their own total, so the
    // rounding of a dominant probability does not reach the output.
    float r = 0.0f;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const int j = tid + 256 * e;
        const uint16_t h = to16<DT>(j < p.Sk ? x[e] : 0.0f);
        if (j < p.Skp) P[j] = h;
        r += from16<DT>(h);
    }
    r = block_reduce(r, false);
    // the divisor's reciprocal replaces the row's first score (every thread
    // has read its scores before the reductions' barriers)
    if (tid == 0) p.s[row * p.Skp] = r > 0.0f ? 1.0f / r : 0.0f;
    if (tid == 0 && p.lse) p.lse[row] = l > 0.0f ? m + __logf(l) : -INFINITY;
}

// V^T per head through a 64 x 64 LDS tile; padding columns (keys Sk..Skp-1) zero.
template <int D>
__global__ __launch_bounds__(256) void naive_vt(NaiveParams p) {
    __shared__ uint16_t t[64][65];
    const int bh = blockIdx.z;
    const int j0 = blockIdx.x * 64, d0 = blockIdx.y * 64;
    const uint16_t* V = (const uint16_t*)p.v + (int64_t)bh * p.Sk * D;
    uint16_t* Vt = p.vt + (int64_t)bh * D * p.Skp;
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int j = j0 + e / 64, d = d0 + e % 64;
        t[e / 64][e % 64] = (j < p.Sk && d < D) ? V[(int64_t)j * D + d] : (uint16_t)0;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int d = d0 + e / 64, j = j0 + e % 64;
        if (d < D && j < p.Skp) Vt[(int64_t)d * p.Skp + j] = t[e % 64][e / 64];
    }
}

// O = P V: 128 query rows per workgroup, 32 per wave, all D columns; the
// key loop runs over Skp in steps of 16 (both operands read along the keys).
template <int D, int DT>
__global__ __launch_bounds__(256) void naive_pv(NaiveParams p) {
    const int bh = blockIdx.y;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r0 = blockIdx.x * 128 + 32 * w;
    const uint64_t pbytes = (uint64_t)p.Sq * p.Skp * 2;
    const __amdgpu_buffer_rsrc_t rp = rsrc((const char*)p.p + (int64_t)bh * p.Sq * p.Skp * 2, pbytes);
    const __amdgpu_buffer_rsrc_t rv = rsrc((const char*)p.vt + (int64_t)bh * D * p.Skp * 2, (uint64_t)D * p.Skp * 2);
    f32x16 acc[D / 32];
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[b][i] = 0.0f;
    const int kq = 8 * (lane >> 5);
    const uint32_t arow = (uint32_t)(r0 + (lane & 31)) * p.Skp;
    // four 16-key steps per iteration (Skp is a multiple of 64): all their
    // loads are issued before the first of their MFMAs
    for (int k0 = 0; k0 < p.Skp; k0 += 64) {
        i32x4 af[4], bf[4][D / 32];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            af[u] = __builtin_amdgcn_raw_buffer_load_b128(rp, (arow + k0 + 16 * u + kq) * 2, 0, 0);
#pragma unroll
            for (int b = 0; b < D / 32; ++b)
                bf[u][b] = __builtin_amdgcn_raw_buffer_load_b128(
                    rv, ((uint32_t)(32 * b + (lane & 31)) * p.Skp + k0 + 16 * u + kq) * 2, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int b = 0; b < D / 32; ++b) acc[b] = mma<DT>(af[u], bf[u][b], acc[b]);
    }
    uint16_t* O = (uint16_t*)p.o + (int64_t)bh * p.Sq * D;
    // 1 / (sum of the row's rounded probabilities), left by the softmax in
    // the row's first score slot
    float rinv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int row = r0 + acc_row(i, lane);
        rinv[i] = row < p.Sq ? p.s[((int64_t)bh * p.Sq + row) * p.Skp] : 0.0f;
    }
#pragma unroll
    for (int b = 0; b < D / 32; ++b) {
        const int col = 32 * b + (lane & 31);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = r0 + acc_row(i, lane);
            if (row < p.Sq) O[(int64_t)row * D + col] = to16<DT>(acc[b][i] * rinv[i]);
        }
    }
}

template <int D, int DT>
static hipError_t run(const NaiveParams& p, int BH, hipStream_t st) {
    hipLaunchKernelGGL((naive_scores<D, DT>), dim3((p.Sk + 127) / 128, (p.Sq + 127) / 128, BH), dim3(256), 0, st, p);
    const int ne = (p.Skp + 255) / 256;
    const dim3 rows((unsigned)((int64_t)BH * p.Sq));
    if (ne <= 1) hipLaunchKernelGGL((naive_softmax<DT, 1>), rows, dim3(256), 0, st, p);
    else if (ne <= 2) hipLaunchKernelGGL((naive_softmax<DT, 2>), rows, dim3(256), 0, st, p);
    else if (ne <= 4) hipLaunchKernelGGL((naive_softmax<DT, 4>), rows, dim3(256), 0, st, p);
    else if (ne <= 8) hipLaunchKernelGGL((naive_softmax<DT, 8>), rows, dim3(256), 0, st, p);
    else if (ne <= 16) hipLaunchKernelGGL((naive_softmax<DT, 16>), rows, dim3(256), 0, st, p);
    else if (ne <= 32) hipLaunchKernelGGL((naive_softmax<DT, 32>), rows, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((naive_softmax<DT, 64>), rows, dim3(256), 0, st, p);
    hipLaunchKernelGGL((naive_vt<D>), dim3((p.Skp + 63) / 64, (D + 63) / 64, BH), dim3(256), 0, st, p);
    hipLaunchKernelGGL((naive_pv<D, DT>), dim3((p.Sq + 127) / 128, BH), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_naive(const NaiveParams& p, int BH, int D, int dtype, hipStream_t stream) {
    if (D == 64) return dtype == 0 ? run<64, 0>(p, BH, stream) : run<64, 1>(p, BH, stream);
    return dtype == 0 ? run<128, 0>(p, BH, stream) : run<128, 1>(p, BH, stream);
}

}  // namespace naive
}  // namespace fa
