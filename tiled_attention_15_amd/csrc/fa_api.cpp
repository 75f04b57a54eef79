// fa_api.cpp -- C ABI of the fused attention forward: argument validation,
// launch planning and dispatch.  Declarations and the meaning of every
// argument are in include/fa.h.
//
// Validation runs entirely on the host, before any HIP call, so a rejected
// call enqueues nothing.  The launch is asynchronous on the caller's stream;
// the library never allocates, frees or synchronises.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>

#include "fa.h"
#include "fa_launch.h"
#include "fa_bwd.h"
#include "fa_ext.h"
#include "fa_naive.h"

namespace fa {

// Compute units per device, read from the device the first time a call runs
// on it (0 = not read yet).  Queried, not assumed: a partitioned part or
// another SKU has a different count, and the key-split choice depends on it.
constexpr int kMaxDevices = 64;
constexpr int kDefaultComputeUnits = 256;   // MI355X, when no device answers
static std::atomic<int> g_compute_units[kMaxDevices];

int compute_units() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();   // clear our own failure only
        return kDefaultComputeUnits;
    }
    if (dev < 0 || dev >= kMaxDevices) return kDefaultComputeUnits;
    int n = g_compute_units[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        n = kDefaultComputeUnits;
    }
    g_compute_units[dev].store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace fa

namespace {

constexpr int kVersion = 1 * 10000 + 6 * 100 + 0;

int validate_shape(int B, int H, int Sq, int Sk, int D, int dtype) {
    if (B < 1 || H < 1 || Sq < 1 || Sk < 1) return FA_ERR_SHAPE;
    // sequence lengths up to 2^30, so that every ceiling division by a block
    // size below stays inside int
    if (Sq > (1 << 30) || Sk > (1 << 30)) return FA_ERR_SHAPE;
    if (D != 64 && D != 128 && D != 256) return FA_ERR_UNSUPPORTED;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    const int S = Sq > Sk ? Sq : Sk;
    // in double: the product of four ints can exceed 2^63 (exact below 2^53)
    const double elems = (double)B * (double)H * (double)S * (double)D;
    if (elems >= 1099511627776.0) return FA_ERR_SHAPE;    // 2^40
    const int64_t grid = (int64_t)B * H * ((Sq + fa::kBlockQ - 1) / fa::kBlockQ);
    if (grid >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
    return FA_OK;
}

// Causal diagonal of the kernels: key j visible to query i iff j <= i + diag.
// Without an explicit offset it is bottom-right (Sk - Sq); an explicit one
// is clamped to [-Sq, Sk], where it already hides every key from every row
// or shows every key to every row, so that i + diag stays in int range.
int diag_of(int Sq, int Sk, const int64_t* causal_offset) {
    if (causal_offset == nullptr) return Sk - Sq;
    return (int)std::min<int64_t>(std::max<int64_t>(*causal_offset, -(int64_t)Sq), (int64_t)Sk);
}

// The key-split instances of the tuned kernel (D = 64 or 128, with or
// without a mask):
// 128-row blocks with the key range split between the two wave groups
// double the workgroups and halve each one's chain of K/V steps.  Used when
// the doubled grid still runs in one round (at most half as many 256-row
// blocks as compute units), or, under the causal rule, whenever the 256-row
// blocks leave compute units idle (their chains differ in length, so the
// longest one sets the time).
bool use_split(int B, int H, int Sq, int D, bool causal, int cus) {
    const int64_t blocks = (int64_t)B * H * ((Sq + fa::kBlockQ - 1) / fa::kBlockQ);
    if (D == 256) return false;
    return 2 * blocks <= cus || (causal && blocks < cus);
}

// Byte offsets inside one head are 32-bit (buffer descriptors): every row a
// query block (rows up to a multiple of kBlockQ) or a key tile (up to 64
// rows past the end) can address must lie below 2^31 bytes.
bool head_span_ok(int S, int64_t row_stride, int D) {
    const int64_t rows = ((int64_t)S + fa::kBlockQ - 1) / fa::kBlockQ * fa::kBlockQ + fa::kBlockKV;
    return (rows * row_stride + D) * 2 < (int64_t(1) << 31);
}

bool overlap(uintptr_t x, uintptr_t xe, uintptr_t y, uintptr_t ye) { return x < ye && y < xe; }

// Byte range [lo, hi) covered by a [B, H, S, D] tensor with element strides
// st (strides are >= 0).
void span(const void* p, int B, int H, int S, int D, const int64_t* st, uintptr_t& lo, uintptr_t& hi) {
    lo = (uintptr_t)p;
    hi = lo + (uintptr_t)(((B - 1) * st[0] + (H - 1) * st[1] + (int64_t)(S - 1) * st[2] + D) * 2);
}

int check_strides(const int64_t* st, int D) {
    for (int i = 0; i < 3; ++i)
        if (st[i] < 0 || (st[i] & 7) != 0) return FA_ERR_STRIDE;
    if (st[2] < D) return FA_ERR_STRIDE;
    if (st[2] >= (int64_t(1) << 30)) return FA_ERR_SHAPE;
    return FA_OK;
}

// o's elements must not share addresses: with its three strides sorted
// (largest first, extents n1 n2 n3), s3 >= D, s2 >= n3*s3, s1 >= n2*s2.
// A dimension of extent 1 is ignored.
bool no_self_overlap(const int64_t* st, int B, int H, int S, int D) {
    int64_t s[3] = {st[0], st[1], st[2]};
    int64_t n[3] = {B, H, S};
    for (int i = 0; i < 3; ++i)
        if (n[i] == 1) s[i] = 0;
    for (int i = 0; i < 3; ++i)
        for (int j = i + 1; j < 3; ++j)
            if (s[j] > s[i]) {
                std::swap(s[i], s[j]);
                std::swap(n[i], n[j]);
            }
    // s[0] >= s[1] >= s[2]; zero strides only for extent-1 dimensions
    int64_t need = D;
    for (int i = 2; i >= 0; --i) {
        if (n[i] == 1) continue;
        if (s[i] < need) return false;
        need = s[i] * n[i];
    }
    return true;
}

}  // namespace

// Diagnostic outputs of fa_fwd_diag (null for the product entry points).
struct DiagArgs {
    int flags;
    float* o32;
    uint32_t* tiles;
};

// Dropout arguments of the tuned kernel: threshold t = round(p * 65536)
// (0: no dropout), Philox key and counter offset.
struct DropArgs {
    uint32_t t = 0;
    uint64_t seed = 0;
    uint32_t offset = 0;
};

// The tuned kernel on validated arguments; mask (with its byte strides) may
// be null; drop selects the dropout instances when drop.t > 0; diag selects
// the diagnostic instance.
static int launch_tuned(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Sq,
                        int Sk, int D, const int64_t* q_strides, const int64_t* k_strides,
                        const int64_t* v_strides, const int64_t* o_strides, const uint8_t* mask,
                        const int64_t* mask_strides, float scale, int causal, int dtype, void* stream,
                        const DiagArgs* diag = nullptr, DropArgs drop = DropArgs(),
                        const int64_t* causal_offset = nullptr) {
    fa::FwdParams p = {};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.Sq = Sq;
    p.Sk = Sk;
    p.H = H;
    p.BH = B * H;
    const bool split = use_split(B, H, Sq, D, causal != 0, fa::compute_units());
    // 128-row blocks for the key-split instances and at D = 256 (the pair
    // split: 64 rows per wave group, each pair of waves on 32 of them)
    const int br = (split || D == 256) ? fa::kBlockQSplit : fa::kBlockQ;
    p.nqb = (Sq + br - 1) / br;
    p.diag = diag_of(Sq, Sk, causal_offset);
    p.scale_log2e = (float)((double)scale * 1.4426950408889634074);
    p.q_sb = q_strides[0], p.q_sh = q_strides[1], p.q_ss = (int)q_strides[2];
    p.k_sb = k_strides[0], p.k_sh = k_strides[1], p.k_ss = (int)k_strides[2];
    p.v_sb = v_strides[0], p.v_sh = v_strides[1], p.v_ss = (int)v_strides[2];
    p.o_sb = o_strides[0], p.o_sh = o_strides[1], p.o_ss = (int)o_strides[2];
    p.mask = mask;
    p.m_sb = mask ? mask_strides[0] : 0;
    p.m_sh = mask ? mask_strides[1] : 0;
    p.m_ss = mask ? (int)mask_strides[2] : 0;
    p.drop_t = drop.t;
    p.keep_scale = (float)(65536.0 / (65536.0 - (double)drop.t));
    p.seed_lo = (uint32_t)drop.seed;
    p.seed_hi = (uint32_t)(drop.seed >> 32);
    p.offset = drop.offset;
    const int64_t grid = (int64_t)p.BH * p.nqb;
    if (diag != nullptr) {
        p.diag_flags = diag->flags;
        p.o32 = diag->o32;
        p.tiles = diag->tiles;
        const hipError_t err = fa::launch_fwd_diag(p, D, dtype, causal != 0, grid, split, (hipStream_t)stream);
        return err == hipSuccess ? FA_OK : FA_ERR_HIP;
    }
    const hipError_t err = drop.t != 0
                               ? fa::launch_fwd_drop(p, D, dtype, causal != 0, grid, split, (hipStream_t)stream)
                               : fa::launch_fwd(p, D, dtype, causal != 0, grid, split, (hipStream_t)stream);
    return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" {

int fa_version(void) { return kVersion; }

const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_NULL: return "null pointer argument";
        case FA_ERR_SHAPE: return "invalid or too large shape";
        case FA_ERR_UNSUPPORTED: return "unsupported head dimension or dtype";
        case FA_ERR_ALIGN: return "pointer not 16-byte aligned";
        case FA_ERR_SCALE: return "scale not finite and positive";
        case FA_ERR_HIP: return "HIP runtime error at launch";
        case FA_ERR_ALIAS: return "output buffer overlaps an input or the other output";
        case FA_ERR_STRIDE: return "invalid strides (negative, not a multiple of 8, row stride < D, or overlapping output)";
        case FA_ERR_MASK_DROPOUT: return "invalid mask layout or dropout probability";
        case FA_ERR_SCRATCH: return "the call needs more scratch than the allocation-free entry point holds";
        default: return "unknown status";
    }
}

int fa_fwd_plan(int B, int H, int S, int D, int causal, int dtype, int* block_q, int* block_kv,
                int64_t* grid, int64_t* tiles) {
    int st = validate_shape(B, H, S, S, D, dtype);
    if (st == FA_OK && !head_span_ok(S, D, D)) st = FA_ERR_SHAPE;
    if (st != FA_OK) return st;
    // 128-row blocks at D = 256 (pair split) and on small grids
    // (key split)
    const int br = (D == 256 || use_split(B, H, S, D, causal != 0, fa::compute_units())) ? fa::kBlockQSplit
                                                                                         : fa::kBlockQ;
    const int bc = fa::kBlockKV;
    const int64_t nqb = (S + br - 1) / br;
    const int64_t nkv = (S + bc - 1) / bc;
    if (block_q) *block_q = br;
    if (block_kv) *block_kv = bc;
    if (grid) *grid = (int64_t)B * H * nqb;
    if (tiles) {
        int64_t per_head = 0;
        for (int64_t qb = 0; qb < nqb; ++qb) {
            if (!causal) { per_head += nkv; continue; }
            const int64_t last = std::min<int64_t>(S, (qb + 1) * br);
            per_head += std::min<int64_t>(nkv, (last + bc - 1) / bc);
        }
        *tiles = per_head * B * H;
    }
    return FA_OK;
}

int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Sq, int Sk, int D,
                   const int64_t* q_strides, const int64_t* k_strides,
                   const int64_t* v_strides, const int64_t* o_strides,
                   float scale, int causal, int dtype, void* stream) {
    if (!q || !k || !v || !o || !q_strides || !k_strides || !v_strides || !o_strides)
        return FA_ERR_NULL;
    int st = validate_shape(B, H, Sq, Sk, D, dtype);
    if (st != FA_OK) return st;
    const int64_t* strides[4] = {q_strides, k_strides, v_strides, o_strides};
    for (const int64_t* s4 : strides)
        if ((st = check_strides(s4, D)) != FA_OK) return st;
    if (!head_span_ok(Sq, q_strides[2], D) || !head_span_ok(Sk, k_strides[2], D) ||
        !head_span_ok(Sk, v_strides[2], D) || !head_span_ok(Sq, o_strides[2], D))
        return FA_ERR_SHAPE;
    if (o_strides[0] == 0 && B > 1) return FA_ERR_STRIDE;
    if (o_strides[1] == 0 && H > 1) return FA_ERR_STRIDE;
    if (!no_self_overlap(o_strides, B, H, Sq, D)) return FA_ERR_STRIDE;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse) & 15)
        return FA_ERR_ALIGN;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_SCALE;
    uintptr_t ql, qh, kl, kh, vl, vh, ol, oh;
    span(q, B, H, Sq, D, q_strides, ql, qh);
    span(k, B, H, Sk, D, k_strides, kl, kh);
    span(v, B, H, Sk, D, v_strides, vl, vh);
    span(o, B, H, Sq, D, o_strides, ol, oh);
    if (overlap(ol, oh, ql, qh) || overlap(ol, oh, kl, kh) || overlap(ol, oh, vl, vh))
        return FA_ERR_ALIAS;
    if (lse) {
        const uintptr_t ll = (uintptr_t)lse, lh = ll + (uintptr_t)((int64_t)B * H * Sq * 4);
        if (overlap(ll, lh, ql, qh) || overlap(ll, lh, kl, kh) || overlap(ll, lh, vl, vh) ||
            overlap(ll, lh, ol, oh))
            return FA_ERR_ALIAS;
    }

    return launch_tuned(q, k, v, o, lse, B, H, Sq, Sk, D, q_strides, k_strides, v_strides, o_strides, nullptr,
                        nullptr, scale, causal, dtype, stream);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int S,
           int D, float scale, int causal, int dtype, void* stream) {
    // the shape first: the contiguous strides below overflow for absurd shapes
    const int vs = validate_shape(B, H, S, S, D, dtype);
    if (vs != FA_OK) return (!q || !k || !v || !o) ? FA_ERR_NULL : vs;
    // contiguous [B, H, S, D]
    const int64_t st[3] = {(int64_t)H * S * D, (int64_t)S * D, D};
    return fa_fwd_strided(q, k, v, o, lse, B, H, S, S, D, st, st, st, st, scale, causal, dtype,
                          stream);
}

int64_t fa_fwd_diag_tile_slots(int B, int H, int Sq, int D, int causal) {
    if (validate_shape(B, H, Sq, Sq, D, FA_F16) != FA_OK || D == 256) return 0;
    const int br = use_split(B, H, Sq, D, causal != 0, fa::compute_units()) ? fa::kBlockQSplit : fa::kBlockQ;
    return (int64_t)B * H * ((Sq + br - 1) / br) * 8;
}

int fa_fwd_diag(const void* q, const void* k, const void* v, void* o, float* lse, float* o32,
                uint32_t* tile_counts, int B, int H, int Sq, int Sk, int D, float scale, int causal,
                int dtype, int flags, void* stream) {
    if (!q || !k || !v || !o) return FA_ERR_NULL;
    int st = validate_shape(B, H, Sq, Sk, D, dtype);
    if (st != FA_OK) return st;
    if (D == 256 || (flags & ~fa::kDiagReverseOrder) != 0) return FA_ERR_UNSUPPORTED;
    const int64_t sq[3] = {(int64_t)H * Sq * D, (int64_t)Sq * D, D};
    const int64_t sk[3] = {(int64_t)H * Sk * D, (int64_t)Sk * D, D};
    if (!head_span_ok(Sq, D, D) || !head_span_ok(Sk, D, D)) return FA_ERR_SHAPE;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse | (uintptr_t)o32 |
         (uintptr_t)tile_counts) & 15)
        return FA_ERR_ALIGN;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_SCALE;
    const uintptr_t qb = (uintptr_t)((int64_t)B * H * Sq * D * 2), kb = (uintptr_t)((int64_t)B * H * Sk * D * 2);
    const uintptr_t in[3][2] = {{(uintptr_t)q, (uintptr_t)q + qb}, {(uintptr_t)k, (uintptr_t)k + kb},
                                {(uintptr_t)v, (uintptr_t)v + kb}};
    const int64_t nslots = fa_fwd_diag_tile_slots(B, H, Sq, D, causal);
    const uintptr_t out[4][2] = {
        {(uintptr_t)o, (uintptr_t)o + qb},
        {(uintptr_t)lse, (uintptr_t)lse + (lse ? (uintptr_t)((int64_t)B * H * Sq * 4) : 0)},
        {(uintptr_t)o32, (uintptr_t)o32 + (o32 ? (uintptr_t)((int64_t)B * H * Sq * D * 4) : 0)},
        {(uintptr_t)tile_counts, (uintptr_t)tile_counts + (tile_counts ? (uintptr_t)(nslots * 4) : 0)}};
    for (int i = 0; i < 4; ++i) {
        if (out[i][1] == out[i][0]) continue;
        for (int j = 0; j < 3; ++j)
            if (overlap(out[i][0], out[i][1], in[j][0], in[j][1])) return FA_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (out[j][1] > out[j][0] && overlap(out[i][0], out[i][1], out[j][0], out[j][1])) return FA_ERR_ALIAS;
    }
    const DiagArgs diag = {flags, o32, tile_counts};
    return launch_tuned(q, k, v, o, lse, B, H, Sq, Sk, D, sq, sk, sk, sq, nullptr, nullptr, scale, causal, dtype,
                        stream, &diag);
}

namespace {

// Workspace regions of the unfused path, each rounded up to 256 bytes.
struct NaiveLayout {
    int64_t s_bytes, p_bytes, vt_bytes, total;
};

bool naive_layout(int B, int H, int S, int D, NaiveLayout& L) {
    if (validate_shape(B, H, S, S, D, FA_F16) != FA_OK || D == 256) return false;
    const int64_t Sp = (S + 63) / 64 * 64;
    if (Sp > 16384 || (int64_t)B * H > 65535) return false;
    if (S * Sp * 4 >= (int64_t(1) << 31)) return false;
    auto r256 = [](int64_t x) { return (x + 255) / 256 * 256; };
    const int64_t bh = (int64_t)B * H;
    L.s_bytes = r256(bh * S * Sp * 4);
    L.p_bytes = r256(bh * S * Sp * 2);
    L.vt_bytes = r256(bh * D * Sp * 2);
    L.total = L.s_bytes + L.p_bytes + L.vt_bytes;
    return true;
}

}  // namespace

int64_t fa_naive_workspace_bytes(int B, int H, int S, int D) {
    NaiveLayout L;
    return naive_layout(B, H, S, D, L) ? L.total : 0;
}

int fa_naive_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int S, int D, float scale, int causal, int dtype, void* workspace,
                 int64_t workspace_bytes, void* stream) {
    if (!q || !k || !v || !o || !workspace) return FA_ERR_NULL;
    int st = validate_shape(B, H, S, S, D, dtype);
    if (st != FA_OK) return st;
    if (D == 256) return FA_ERR_UNSUPPORTED;
    NaiveLayout L;
    if (!naive_layout(B, H, S, D, L) || workspace_bytes < L.total) return FA_ERR_SHAPE;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse |
         (uintptr_t)workspace) & 15)
        return FA_ERR_ALIGN;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_SCALE;
    const uintptr_t tb = (uintptr_t)((int64_t)B * H * S * D * 2);
    const uintptr_t lb = (uintptr_t)((int64_t)B * H * S * 4);
    const uintptr_t w0 = (uintptr_t)workspace, w1 = w0 + (uintptr_t)L.total;
    const uintptr_t io[5][2] = {{(uintptr_t)q, (uintptr_t)q + tb}, {(uintptr_t)k, (uintptr_t)k + tb},
                                {(uintptr_t)v, (uintptr_t)v + tb}, {(uintptr_t)o, (uintptr_t)o + tb},
                                {(uintptr_t)lse, (uintptr_t)lse + (lse ? lb : 0)}};
    for (int i = 0; i < 5; ++i)
        if (io[i][1] > io[i][0] && overlap(w0, w1, io[i][0], io[i][1])) return FA_ERR_ALIAS;
    for (int i = 0; i < 3; ++i)
        for (int j = 3; j < 5; ++j)
            if (io[j][1] > io[j][0] && overlap(io[i][0], io[i][1], io[j][0], io[j][1])) return FA_ERR_ALIAS;
    if (lse && overlap(io[3][0], io[3][1], io[4][0], io[4][1])) return FA_ERR_ALIAS;

    fa::naive::NaiveParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.s = (float*)workspace;
    p.p = (uint16_t*)((char*)workspace + L.s_bytes);
    p.vt = (uint16_t*)((char*)workspace + L.s_bytes + L.p_bytes);
    p.Sq = S;
    p.Sk = S;
    p.Skp = (S + 63) / 64 * 64;
    p.causal = causal != 0;
    p.scale = scale;
    const hipError_t err = fa::naive::launch_naive(p, B * H, D, dtype, (hipStream_t)stream);
    return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

namespace {

struct BwdLayout {
    int64_t dvec_bytes = 0, total = 0;
};

int64_t r256b(int64_t x) { return (x + 255) / 256 * 256; }

// The workspace holds D_i, one fp32 per query row.
bool bwd_layout(int B, int H, int Sq, int D, BwdLayout& L) {
    if (validate_shape(B, H, Sq, Sq, D, FA_F16) != FA_OK) return false;
    const int64_t rows = (int64_t)B * H * Sq;
    L.dvec_bytes = r256b(rows * 4);
    L.total = L.dvec_bytes;
    return true;
}

// Offsets inside one head are 32-bit: tiles reach up to 128 rows past the
// sequence end.
bool bwd_span_ok(int S, int64_t row_stride, int D) {
    const int64_t rows = ((int64_t)S + fa::bwd::kKeyBlock - 1) / fa::bwd::kKeyBlock * fa::bwd::kKeyBlock +
                         fa::bwd::kKeyBlock;
    return (rows * row_stride + D) * 2 < (int64_t(1) << 31);
}

}  // namespace

// Shared body of the masked / dropout forward entry points.  `strides`
// holds batch, head and row element strides of q, k, v, o in that order.
static int ext_common(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Sq,
                      int Sk, int D, const int64_t* strides, const uint8_t* mask, const int64_t* mask_strides,
                      float dropout_p, uint64_t seed, uint32_t offset, float scale, int causal, int dtype,
                      void* stream, const int64_t* causal_offset) {
    if (!q || !k || !v || !o || !strides) return FA_ERR_NULL;
    int st = validate_shape(B, H, Sq, Sk, D, dtype);
    if (st != FA_OK) return st;
    const int len[4] = {Sq, Sk, Sk, Sq};
    for (int t = 0; t < 4; ++t) {
        if ((st = check_strides(strides + 3 * t, D)) != FA_OK) return st;
        if (!bwd_span_ok(len[t], strides[3 * t + 2], D)) return FA_ERR_SHAPE;
    }
    if (!no_self_overlap(strides + 9, B, H, Sq, D)) return FA_ERR_STRIDE;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse) & 15) return FA_ERR_ALIGN;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_SCALE;
    if (!(dropout_p >= 0.0f) || !(dropout_p < 1.0f)) return FA_ERR_MASK_DROPOUT;
    const long t = lrintf(dropout_p * 65536.0f);
    if (t > 65535) return FA_ERR_MASK_DROPOUT;
    uintptr_t m0 = 0, m1 = 0;
    if (mask) {
        if (!mask_strides || ((uintptr_t)mask & 3)) return FA_ERR_MASK_DROPOUT;
        for (int i = 0; i < 3; ++i)
            if (mask_strides[i] < 0 || (mask_strides[i] & 3) != 0) return FA_ERR_MASK_DROPOUT;
        if (mask_strides[2] < Sk || mask_strides[2] >= (int64_t(1) << 31)) return FA_ERR_MASK_DROPOUT;
        if ((int64_t)(Sq - 1) * mask_strides[2] + Sk + 3 >= (int64_t(1) << 31)) return FA_ERR_MASK_DROPOUT;
        m0 = (uintptr_t)mask;
        m1 = m0 + (uintptr_t)((int64_t)(B - 1) * mask_strides[0] + (int64_t)(H - 1) * mask_strides[1] +
                              (int64_t)(Sq - 1) * mask_strides[2] + Sk);
    }
    const void* ptr[4] = {q, k, v, o};
    uintptr_t sp[4][2];
    for (int i = 0; i < 4; ++i) span(ptr[i], B, H, len[i], D, strides + 3 * i, sp[i][0], sp[i][1]);
    const uintptr_t lb = (uintptr_t)((int64_t)B * H * Sq * 4);
    const uintptr_t in[4][2] = {{sp[0][0], sp[0][1]}, {sp[1][0], sp[1][1]}, {sp[2][0], sp[2][1]}, {m0, m1}};
    const uintptr_t out[2][2] = {{sp[3][0], sp[3][1]}, {(uintptr_t)lse, (uintptr_t)lse + (lse ? lb : 0)}};
    for (int i = 0; i < 2; ++i) {
        if (out[i][1] == out[i][0]) continue;
        for (int j = 0; j < 4; ++j)
            if (in[j][1] > in[j][0] && overlap(out[i][0], out[i][1], in[j][0], in[j][1])) return FA_ERR_ALIAS;
    }
    if (lse && overlap(out[0][0], out[0][1], out[1][0], out[1][1])) return FA_ERR_ALIAS;

    // The tuned kernel, with the mask and the dropout if there are any,
    // whenever its 32-bit head offsets reach (they pad a head to whole
    // 256-row blocks); without mask or dropout this is the plain forward
    // exactly as fa_fwd_strided runs it (the two calls agree bit for bit).
    // Beyond that reach, the general kernel below (128-row blocks).
    if (head_span_ok(Sq, strides[2], D) && head_span_ok(Sk, strides[5], D) && head_span_ok(Sk, strides[8], D) &&
        head_span_ok(Sq, strides[11], D)) {
        DropArgs drop;
        drop.t = (uint32_t)t;
        drop.seed = seed;
        drop.offset = offset;
        return launch_tuned(q, k, v, o, lse, B, H, Sq, Sk, D, strides, strides + 3, strides + 6, strides + 9, mask,
                            mask_strides, scale, causal, dtype, stream, nullptr, drop, causal_offset);
    }

    fa::ext::ExtParams p = {};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.q_sb = strides[0], p.q_sh = strides[1], p.q_ss = (int)strides[2];
    p.k_sb = strides[3], p.k_sh = strides[4], p.k_ss = (int)strides[5];
    p.v_sb = strides[6], p.v_sh = strides[7], p.v_ss = (int)strides[8];
    p.o_sb = strides[9], p.o_sh = strides[10], p.o_ss = (int)strides[11];
    p.mask = mask;
    p.m_sb = mask ? mask_strides[0] : 0;
    p.m_sh = mask ? mask_strides[1] : 0;
    p.m_ss = mask ? mask_strides[2] : 0;
    p.Sq = Sq;
    p.Sk = Sk;
    p.H = H;
    p.BH = B * H;
    p.nqb = (Sq + fa::ext::kQueryBlock - 1) / fa::ext::kQueryBlock;
    p.diag = diag_of(Sq, Sk, causal_offset);
    p.scale_log2e = (float)((double)scale * 1.4426950408889634074);
    p.drop_t = (uint32_t)t;
    p.keep_scale = (float)(65536.0 / (65536.0 - (double)t));
    p.seed_lo = (uint32_t)seed;
    p.seed_hi = (uint32_t)(seed >> 32);
    p.offset = offset;
    const hipError_t err = fa::ext::launch_ext(p, D, dtype, causal != 0, (hipStream_t)stream);
    return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Sq,
               int Sk, int D, const uint8_t* mask, const int64_t* mask_strides, float dropout_p,
               uint64_t seed, uint32_t offset, float scale, int causal, int dtype, void* stream) {
    const int vs = validate_shape(B, H, Sq, Sk, D, dtype);
    if (vs != FA_OK) return (!q || !k || !v || !o) ? FA_ERR_NULL : vs;
    // contiguous [B, H, S, D]
    const int64_t st[12] = {(int64_t)H * Sq * D, (int64_t)Sq * D, D, (int64_t)H * Sk * D, (int64_t)Sk * D, D,
                            (int64_t)H * Sk * D, (int64_t)Sk * D, D, (int64_t)H * Sq * D, (int64_t)Sq * D, D};
    return ext_common(q, k, v, o, lse, B, H, Sq, Sk, D, st, mask, mask_strides, dropout_p, seed, offset, scale,
                      causal, dtype, stream, nullptr);
}

int fa_fwd_ext_strided(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                       int Sq, int Sk, int D, const int64_t* strides, const uint8_t* mask,
                       const int64_t* mask_strides, float dropout_p, uint64_t seed, uint32_t offset,
                       float scale, int causal, int dtype, void* stream) {
    return ext_common(q, k, v, o, lse, B, H, Sq, Sk, D, strides, mask, mask_strides, dropout_p, seed, offset,
                      scale, causal, dtype, stream, nullptr);
}

int fa_fwd_causal_offset(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                         int Sq, int Sk, int D, const int64_t* strides, const uint8_t* mask,
                         const int64_t* mask_strides, float dropout_p, uint64_t seed, uint32_t offset,
                         float scale, int64_t causal_offset, int dtype, void* stream) {
    return ext_common(q, k, v, o, lse, B, H, Sq, Sk, D, strides, mask, mask_strides, dropout_p, seed, offset,
                      scale, 1, dtype, stream, &causal_offset);
}

int64_t fa_bwd_workspace_bytes(int B, int H, int Sq, int D, int deterministic) {
    (void)deterministic;   // every backward is deterministic
    BwdLayout L;
    return bwd_layout(B, H, Sq, D, L) ? L.total : 0;
}

// Shared body of the backward entry points.  `strides` holds batch, head
// and row element strides of q, k, v, o, dout, dq, dk, dv in that order.
static int bwd_common(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, int B, int H, int Sq, int Sk, int D,
                      const int64_t* strides, const uint8_t* mask, const int64_t* mask_strides,
                      float dropout_p, uint64_t seed, uint32_t offset, float scale, int causal, int dtype,
                      void* workspace, int64_t workspace_bytes, void* stream, const int64_t* causal_offset) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace || !strides) return FA_ERR_NULL;
    int st = validate_shape(B, H, Sq, Sk, D, dtype);
    if (st != FA_OK) return st;
    // tensor t has sequence length len[t] (Sq for q, o, dout, dq; Sk for k, v, dk, dv)
    const int len[8] = {Sq, Sk, Sk, Sq, Sq, Sq, Sk, Sk};
    for (int t = 0; t < 8; ++t) {
        if ((st = check_strides(strides + 3 * t, D)) != FA_OK) return st;
        if (!bwd_span_ok(len[t], strides[3 * t + 2], D)) return FA_ERR_SHAPE;
    }
    for (int t = 5; t < 8; ++t)
        if (!no_self_overlap(strides + 3 * t, B, H, len[t], D)) return FA_ERR_STRIDE;
    BwdLayout L;
    if (!bwd_layout(B, H, Sq, D, L) || workspace_bytes < L.total) return FA_ERR_SHAPE;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)lse |
         (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)workspace) & 15)
        return FA_ERR_ALIGN;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_SCALE;
    if (!(dropout_p >= 0.0f) || !(dropout_p < 1.0f)) return FA_ERR_MASK_DROPOUT;
    const long drop_t = lrintf(dropout_p * 65536.0f);
    if (drop_t > 65535) return FA_ERR_MASK_DROPOUT;
    uintptr_t m0 = 0, m1 = 0;
    if (mask) {
        if (!mask_strides || ((uintptr_t)mask & 3)) return FA_ERR_MASK_DROPOUT;
        for (int i = 0; i < 3; ++i)
            if (mask_strides[i] < 0 || (mask_strides[i] & 3) != 0) return FA_ERR_MASK_DROPOUT;
        if (mask_strides[2] < Sk || mask_strides[2] >= (int64_t(1) << 31)) return FA_ERR_MASK_DROPOUT;
        // mask rows are read up to 31 past the last query (the last tile)
        if ((int64_t)(Sq + 31) * mask_strides[2] + Sk + 3 >= (int64_t(1) << 31)) return FA_ERR_MASK_DROPOUT;
        m0 = (uintptr_t)mask;
        m1 = m0 + (uintptr_t)((int64_t)(B - 1) * mask_strides[0] + (int64_t)(H - 1) * mask_strides[1] +
                              (int64_t)(Sq - 1) * mask_strides[2] + Sk);
    }
    const void* ptr[8] = {q, k, v, o, dout, dq, dk, dv};
    uintptr_t sp[8][2];
    for (int t = 0; t < 8; ++t) span(ptr[t], B, H, len[t], D, strides + 3 * t, sp[t][0], sp[t][1]);
    const uintptr_t lb = (uintptr_t)((int64_t)B * H * Sq * 4);
    const uintptr_t in[7][2] = {{sp[0][0], sp[0][1]}, {sp[1][0], sp[1][1]}, {sp[2][0], sp[2][1]},
                                {sp[3][0], sp[3][1]}, {sp[4][0], sp[4][1]}, {(uintptr_t)lse, (uintptr_t)lse + lb},
                                {m0, m1}};
    const uintptr_t out[4][2] = {{sp[5][0], sp[5][1]}, {sp[6][0], sp[6][1]}, {sp[7][0], sp[7][1]},
                                 {(uintptr_t)workspace, (uintptr_t)workspace + (uintptr_t)L.total}};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 7; ++j)
            if (in[j][1] > in[j][0] && overlap(out[i][0], out[i][1], in[j][0], in[j][1])) return FA_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(out[i][0], out[i][1], out[j][0], out[j][1])) return FA_ERR_ALIAS;
    }

    fa::bwd::BwdParams p = {};
    p.H = H;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.dout = dout;
    p.lse = lse;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    fa::bwd::Lay* lay[8] = {&p.Lq, &p.Lk, &p.Lv, &p.Lo, &p.Ldo, &p.Ldq, &p.Ldk, &p.Ldv};
    for (int t = 0; t < 8; ++t) *lay[t] = {strides[3 * t], strides[3 * t + 1], (int)strides[3 * t + 2]};
    p.dvec = (float*)workspace;
    p.Sq = Sq;
    p.Sk = Sk;
    p.BH = B * H;
    p.diag = diag_of(Sq, Sk, causal_offset);
    p.nkb = (Sk + fa::bwd::kKeyBlock - 1) / fa::bwd::kKeyBlock;
    p.nqb = (Sq + fa::bwd::kQueryBlock - 1) / fa::bwd::kQueryBlock;
    p.scale = scale;
    p.scale_log2e = scale * 1.4426950408889634f;
    p.mask = mask;
    p.m_sb = mask ? mask_strides[0] : 0;
    p.m_sh = mask ? mask_strides[1] : 0;
    p.m_ss = mask ? mask_strides[2] : 0;
    p.drop_t = (uint32_t)drop_t;
    p.keep_scale = (float)(65536.0 / (65536.0 - (double)drop_t));
    p.seed_lo = (uint32_t)seed;
    p.seed_hi = (uint32_t)(seed >> 32);
    p.offset = offset;
    const hipError_t err = fa::bwd::launch_bwd(p, D, dtype, causal != 0, (hipStream_t)stream);
    return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

namespace {
// contiguous [B, H, S, D] strides for q, k, v, o, dout, dq, dk, dv
void contiguous_bwd_strides(int H, int Sq, int Sk, int D, int64_t* st) {
    const int len[8] = {Sq, Sk, Sk, Sq, Sq, Sq, Sk, Sk};
    for (int t = 0; t < 8; ++t) {
        st[3 * t] = (int64_t)H * len[t] * D;
        st[3 * t + 1] = (int64_t)len[t] * D;
        st[3 * t + 2] = D;
    }
}
}  // namespace

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int H, int Sq, int Sk, int D,
           float scale, int causal, int dtype, int deterministic, void* workspace,
           int64_t workspace_bytes, void* stream) {
    const int vs = validate_shape(B, H, Sq, Sk, D, dtype);
    if (vs != FA_OK) return (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace) ? FA_ERR_NULL : vs;
    (void)deterministic;   // every backward is deterministic
    int64_t st[24];
    contiguous_bwd_strides(H, Sq, Sk, D, st);
    return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, B, H, Sq, Sk, D, st, nullptr, nullptr, 0.0f, 0, 0,
                      scale, causal, dtype, workspace, workspace_bytes, stream, nullptr);
}

int fa_bwd_ext(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, int B, int H, int Sq, int Sk, int D,
               const uint8_t* mask, const int64_t* mask_strides, float dropout_p, uint64_t seed,
               uint32_t offset, float scale, int causal, int dtype, void* workspace,
               int64_t workspace_bytes, void* stream) {
    const int vs = validate_shape(B, H, Sq, Sk, D, dtype);
    if (vs != FA_OK) return (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace) ? FA_ERR_NULL : vs;
    int64_t st[24];
    contiguous_bwd_strides(H, Sq, Sk, D, st);
    return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, B, H, Sq, Sk, D, st, mask, mask_strides, dropout_p,
                      seed, offset, scale, causal, dtype, workspace, workspace_bytes, stream, nullptr);
}

int fa_bwd_strided(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int B, int H, int Sq, int Sk, int D,
                   const int64_t* strides, const uint8_t* mask, const int64_t* mask_strides,
                   float dropout_p, uint64_t seed, uint32_t offset, float scale, int causal, int dtype,
                   int deterministic, void* workspace, int64_t workspace_bytes, void* stream) {
    (void)deterministic;   // every backward is deterministic
    return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, B, H, Sq, Sk, D, strides, mask, mask_strides,
                      dropout_p, seed, offset, scale, causal, dtype, workspace, workspace_bytes, stream, nullptr);
}

int fa_bwd_causal_offset(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, void* dq, void* dk, void* dv, int B, int H, int Sq, int Sk, int D,
                         const int64_t* strides, const uint8_t* mask, const int64_t* mask_strides,
                         float dropout_p, uint64_t seed, uint32_t offset, float scale, int64_t causal_offset,
                         int dtype, void* workspace, int64_t workspace_bytes, void* stream) {
    return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, B, H, Sq, Sk, D, strides, mask, mask_strides,
                      dropout_p, seed, offset, scale, 1, dtype, workspace, workspace_bytes, stream, &causal_offset);
}

}  // extern "C"
