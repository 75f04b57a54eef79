// host_checks.cpp -- the host side of the C ABI (argument validation, launch
// planning, workspace layout) under AddressSanitizer and
// UndefinedBehaviorSanitizer, with the launchers replaced by the stubs of
// launch_stubs.cpp.  Device pointers are fake, aligned addresses: the host
// code must never dereference them.  Exits non-zero on the first failed
// check; a sanitizer report aborts the run.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>

#include "fa.h"
#include "launch_stubs.h"

static int g_checks = 0;

#define CHECK_EQ(a, b)                                                                          \
    do {                                                                                        \
        ++g_checks;                                                                             \
        const long long va_ = (long long)(a), vb_ = (long long)(b);                             \
        if (va_ != vb_) {                                                                       \
            std::fprintf(stderr, "%s:%d: %s = %lld, expected %lld\n", __FILE__, __LINE__, #a, va_, vb_); \
            std::exit(1);                                                                       \
        }                                                                                       \
    } while (0)

// fake device addresses: 1 TiB apart, 256-byte aligned
static void* dev(int i) { return (void*)(uintptr_t)((uint64_t)(i + 1) << 40); }
static float* devf(int i) { return (float*)dev(i); }

static void fwd_checks() {
    const float sc = 0.125f;
    void *q = dev(0), *k = dev(1), *v = dev(2), *o = dev(3);
    float* lse = devf(4);
    CHECK_EQ(fa_fwd(nullptr, k, v, o, lse, 1, 1, 64, 64, sc, 0, FA_F16, nullptr), FA_ERR_NULL);
    CHECK_EQ(fa_fwd(q, k, v, nullptr, lse, 1, 1, 64, 64, sc, 0, FA_F16, nullptr), FA_ERR_NULL);
    CHECK_EQ(fa_fwd(q, k, v, o, lse, 0, 1, 64, 64, sc, 0, FA_F16, nullptr), FA_ERR_SHAPE);
    CHECK_EQ(fa_fwd(q, k, v, o, lse, 1, -3, 64, 64, sc, 0, FA_F16, nullptr), FA_ERR_SHAPE);
    CHECK_EQ(fa_fwd(q, k, v, o, lse, 1, 1, 0, 64, sc, 0, FA_F16, nullptr), FA_ERR_SHAPE);
    CHECK_EQ(fa_fwd(q, k, v, o, lse, 1, 1, 64, 96, sc, 0, FA_F16, nullptr), FA_ERR_UNSUPPORTED);
    CHECK_EQ(fa_fwd(q, k, v, o, lse, 1, 1, 64, 64, sc, 0, 7, nullptr), FA_ERR_UNSUPPORTED);
    CHECK_EQ(fa_fwd((char*)q + 8, k, v, o, lse, 1, 1, 64, 64, sc, 0, FA_F16, nullptr), FA_ERR_ALIGN);
    CHECK_EQ(fa_fwd(q, k, v, o, (float*)((char*)lse + 4), 1, 1, 64, 64, sc, 0, FA_F16, nullptr), FA_ERR_ALIGN);
    CHECK_EQ(fa_fwd(q, k, v, o, lse, 1, 1, 64, 64, 0.0f, 0, FA_F16, nullptr), FA_ERR_SCALE);
    CHECK_EQ(fa_fwd(q, k, v, o, lse, 1, 1, 64, 64, -1.0f, 0, FA_F16, nullptr), FA_ERR_SCALE);
    CHECK_EQ(fa_fwd(q, k, v, o, lse, 1, 1, 64, 64, std::numeric_limits<float>::quiet_NaN(), 0, FA_F16, nullptr),
             FA_ERR_SCALE);
    CHECK_EQ(fa_fwd(q, k, v, o, lse, 1, 1, 64, 64, std::numeric_limits<float>::infinity(), 0, FA_F16, nullptr),
             FA_ERR_SCALE);
    // outputs overlapping inputs or each other
    CHECK_EQ(fa_fwd(q, k, v, q, lse, 1, 1, 64, 64, sc, 0, FA_F16, nullptr), FA_ERR_ALIAS);
    CHECK_EQ(fa_fwd(q, k, v, (char*)v + 64, lse, 1, 1, 64, 64, sc, 0, FA_F16, nullptr), FA_ERR_ALIAS);
    CHECK_EQ(fa_fwd(q, k, v, o, (float*)((char*)o + 16), 1, 1, 64, 64, sc, 0, FA_F16, nullptr), FA_ERR_ALIAS);
    // extreme sizes must be rejected without overflow
    CHECK_EQ(fa_fwd(q, k, v, o, lse, INT_MAX, INT_MAX, INT_MAX, 128, sc, 1, FA_BF16, nullptr), FA_ERR_SHAPE);
    CHECK_EQ(fa_fwd(q, k, v, o, lse, 1, 1, INT_MAX, 128, sc, 1, FA_BF16, nullptr), FA_ERR_SHAPE);
    CHECK_EQ(fa_fwd(q, k, v, o, lse, 65536, 65536, 256, 64, sc, 1, FA_BF16, nullptr), FA_ERR_SHAPE);
    // valid: the headline shape, one launch of 32 heads x 32 blocks of 256 rows
    g_stub.last = StubState::kNone;
    CHECK_EQ(fa_fwd(q, k, v, o, lse, 1, 32, 8192, 128, sc, 1, FA_BF16, nullptr), FA_OK);
    CHECK_EQ(g_stub.last, StubState::kFwd);
    CHECK_EQ(g_stub.grid, 1024);
    CHECK_EQ(g_stub.split, 0);
    CHECK_EQ(g_stub.nqb, 32);
    // a small causal grid takes the key split (128-row blocks)
    CHECK_EQ(fa_fwd(q, k, v, o, nullptr, 2, 12, 2048, 64, sc, 1, FA_F16, nullptr), FA_OK);
    CHECK_EQ(g_stub.split, 1);
    CHECK_EQ(g_stub.grid, 2 * 12 * 16);
    // D = 256: 128-row blocks, never the key split
    CHECK_EQ(fa_fwd(q, k, v, o, lse, 1, 16, 8192, 256, sc, 1, FA_BF16, nullptr), FA_OK);
    CHECK_EQ(g_stub.split, 0);
    CHECK_EQ(g_stub.grid, 16 * 64);
}

static void strided_checks() {
    const float sc = 0.125f;
    void *q = dev(0), *k = dev(1), *v = dev(2), *o = dev(3);
    const int B = 2, H = 4, Sq = 100, Sk = 300, D = 64;
    const int64_t bhsd_q[3] = {(int64_t)H * Sq * D, (int64_t)Sq * D, D};
    const int64_t bhsd_k[3] = {(int64_t)H * Sk * D, (int64_t)Sk * D, D};
    const int64_t bshd_q[3] = {(int64_t)Sq * H * D, D, (int64_t)H * D};
    const int64_t neg[3] = {-8, (int64_t)Sq * D, D};
    const int64_t odd[3] = {(int64_t)H * Sq * D, (int64_t)Sq * D + 4, D};
    const int64_t short_row[3] = {(int64_t)H * Sq * D, (int64_t)Sq * D, D - 8};
    const int64_t shared_head_o[3] = {(int64_t)Sq * D, 0, D};
    const int64_t self_overlap[3] = {(int64_t)H * Sq * D, 64, D};   // heads one row apart
    const int64_t huge_row[3] = {0, 0, int64_t(1) << 29};
    CHECK_EQ(fa_fwd_strided(q, k, v, o, nullptr, B, H, Sq, Sk, D, nullptr, bhsd_k, bhsd_k, bhsd_q, sc, 1, FA_F16,
                            nullptr), FA_ERR_NULL);
    CHECK_EQ(fa_fwd_strided(q, k, v, o, nullptr, B, H, Sq, Sk, D, neg, bhsd_k, bhsd_k, bhsd_q, sc, 1, FA_F16,
                            nullptr), FA_ERR_STRIDE);
    CHECK_EQ(fa_fwd_strided(q, k, v, o, nullptr, B, H, Sq, Sk, D, odd, bhsd_k, bhsd_k, bhsd_q, sc, 1, FA_F16,
                            nullptr), FA_ERR_STRIDE);
    CHECK_EQ(fa_fwd_strided(q, k, v, o, nullptr, B, H, Sq, Sk, D, short_row, bhsd_k, bhsd_k, bhsd_q, sc, 1, FA_F16,
                            nullptr), FA_ERR_STRIDE);
    CHECK_EQ(fa_fwd_strided(q, k, v, o, nullptr, B, H, Sq, Sk, D, bhsd_q, bhsd_k, bhsd_k, shared_head_o, sc, 1,
                            FA_F16, nullptr), FA_ERR_STRIDE);
    CHECK_EQ(fa_fwd_strided(q, k, v, o, nullptr, B, H, Sq, Sk, D, bhsd_q, bhsd_k, bhsd_k, self_overlap, sc, 1,
                            FA_F16, nullptr), FA_ERR_STRIDE);
    CHECK_EQ(fa_fwd_strided(q, k, v, o, nullptr, 1, 1, 5000, Sk, D, huge_row, bhsd_k, bhsd_k, bhsd_q, sc, 1,
                            FA_F16, nullptr), FA_ERR_SHAPE);
    CHECK_EQ(fa_fwd_strided(q, k, v, o, nullptr, B, H, Sq, Sk, D, bshd_q, bhsd_k, bhsd_k, bshd_q, sc, 1, FA_F16,
                            nullptr), FA_OK);
    // K/V shared by the heads (head stride 0)
    const int64_t shared_kv[3] = {(int64_t)Sk * D, 0, D};
    CHECK_EQ(fa_fwd_strided(q, k, v, o, nullptr, B, H, Sq, Sk, D, bhsd_q, shared_kv, shared_kv, bhsd_q, sc, 1,
                            FA_F16, nullptr), FA_OK);
}

static void plan_checks(int cus) {
    int bq = 0, bkv = 0;
    int64_t grid = 0, tiles = 0;
    // the five workloads (at 256 compute units)
    struct W { int B, H, S, D, causal; int bq; int64_t grid, tiles; } ws[] = {
        {1, 2, 256, 64, 0, 128, 4, 4 * 4},
        {2, 12, 2048, 64, 1, 128, 2 * 12 * 16, 0},
        {1, 32, 2048, 128, 0, 256, 32 * 8, 32 * 8 * 32},
        {1, 32, 8192, 128, 1, 256, 32 * 32, 0},
        {1, 40, 16384, 128, 1, 256, 40 * 64, 0},
    };
    for (const W& w : ws) {
        CHECK_EQ(fa_fwd_plan(w.B, w.H, w.S, w.D, w.causal, FA_BF16, &bq, &bkv, &grid, &tiles), FA_OK);
        if (cus == 256) {
            CHECK_EQ(bq, w.bq);
            CHECK_EQ(grid, w.grid);
        }
        CHECK_EQ(bkv, 64);
        // causal: T(T+1)/2-style counts per head from the skip rule
        int64_t per_head = 0;
        const int64_t nqb = (w.S + bq - 1) / bq, nkv = (w.S + 63) / 64;
        for (int64_t qb = 0; qb < nqb; ++qb) {
            const int64_t last = (qb + 1) * bq < w.S ? (qb + 1) * bq : w.S;
            per_head += w.causal ? ((last + 63) / 64 < nkv ? (last + 63) / 64 : nkv) : nkv;
        }
        CHECK_EQ(tiles, per_head * w.B * w.H);
    }
    CHECK_EQ(fa_fwd_plan(1, 1, 0, 64, 0, FA_F16, &bq, &bkv, &grid, &tiles), FA_ERR_SHAPE);
    CHECK_EQ(fa_fwd_plan(1, 1, 64, 80, 0, FA_F16, nullptr, nullptr, nullptr, nullptr), FA_ERR_UNSUPPORTED);
    CHECK_EQ(fa_fwd_plan(INT_MAX, INT_MAX, INT_MAX, 64, 1, FA_F16, &bq, &bkv, &grid, &tiles), FA_ERR_SHAPE);
}

static void naive_checks() {
    const float sc = 0.125f;
    void *q = dev(0), *k = dev(1), *v = dev(2), *o = dev(3), *ws = dev(5);
    float* lse = devf(4);
    const int64_t need = fa_naive_workspace_bytes(1, 2, 1000, 64);
    CHECK_EQ(need > 0, 1);
    CHECK_EQ(fa_naive_workspace_bytes(1, 1, 16385, 64), 0);
    CHECK_EQ(fa_naive_workspace_bytes(INT_MAX, INT_MAX, INT_MAX, 64), 0);
    CHECK_EQ(fa_naive_fwd(q, k, v, o, lse, 1, 2, 1000, 64, sc, 1, FA_F16, ws, need - 1, nullptr), FA_ERR_SHAPE);
    CHECK_EQ(fa_naive_fwd(q, k, v, o, lse, 1, 2, 1000, 64, sc, 1, FA_F16, nullptr, need, nullptr), FA_ERR_NULL);
    CHECK_EQ(fa_naive_fwd(q, k, v, o, lse, 1, 2, 1000, 64, sc, 1, FA_F16, q, need, nullptr), FA_ERR_ALIAS);
    CHECK_EQ(fa_naive_fwd(q, k, v, o, lse, 1, 2, 1000, 256, sc, 1, FA_F16, ws, need, nullptr), FA_ERR_UNSUPPORTED);
    CHECK_EQ(fa_naive_fwd(q, k, v, o, lse, 1, 2, 1000, 64, sc, 1, FA_F16, ws, need, nullptr), FA_OK);
    CHECK_EQ(g_stub.last, StubState::kNaive);
}

static void bwd_checks() {
    const float sc = 0.125f;
    void *q = dev(0), *k = dev(1), *v = dev(2), *o = dev(3), *g = dev(5);
    void *dq = dev(6), *dk = dev(7), *dv = dev(8), *ws = dev(9);
    float* lse = devf(4);
    const int B = 1, H = 3, Sq = 200, Sk = 333, D = 128;
    const int64_t wd = fa_bwd_workspace_bytes(B, H, Sq, D, 1), wa = fa_bwd_workspace_bytes(B, H, Sq, D, 0);
    CHECK_EQ(wd, ((int64_t)B * H * Sq * 4 + 255) / 256 * 256);
    CHECK_EQ(wa, wd);   // the flag is ignored: no atomic dq accumulator
    CHECK_EQ(fa_bwd_workspace_bytes(0, 1, 1, 64, 1), 0);
    CHECK_EQ(fa_bwd_workspace_bytes(INT_MAX, INT_MAX, INT_MAX, 128, 0), 0);
    CHECK_EQ(fa_bwd(q, k, v, o, g, lse, dq, dk, dv, INT_MAX, INT_MAX, INT_MAX, INT_MAX, D, sc, 1, FA_BF16, 1, ws,
                    wd, nullptr), FA_ERR_SHAPE);
    CHECK_EQ(fa_bwd(q, k, v, o, g, lse, dq, dk, dv, B, H, Sq, Sk, D, sc, 1, FA_BF16, 1, ws, wd - 1, nullptr),
             FA_ERR_SHAPE);
    CHECK_EQ(fa_bwd(q, k, v, o, g, nullptr, dq, dk, dv, B, H, Sq, Sk, D, sc, 1, FA_BF16, 1, ws, wd, nullptr),
             FA_ERR_NULL);
    CHECK_EQ(fa_bwd(q, k, v, o, g, lse, dq, dq, dv, B, H, Sq, Sk, D, sc, 1, FA_BF16, 1, ws, wd, nullptr),
             FA_ERR_ALIAS);
    CHECK_EQ(fa_bwd(q, k, v, o, g, lse, dq, dk, dv, B, H, Sq, Sk, D, sc, 1, FA_BF16, 1, g, wd, nullptr),
             FA_ERR_ALIAS);
    CHECK_EQ(fa_bwd(q, k, v, o, g, lse, dq, dk, dv, B, H, Sq, Sk, D, sc, 1, FA_BF16, 1, ws, wd, nullptr), FA_OK);
    CHECK_EQ(g_stub.last, StubState::kBwd);
    g_stub.last = StubState::kNone;
    CHECK_EQ(fa_bwd(q, k, v, o, g, lse, dq, dk, dv, B, H, Sq, Sk, D, sc, 1, FA_BF16, 0, ws, wd, nullptr), FA_OK);
    CHECK_EQ(g_stub.last, StubState::kBwd);
    // mask and dropout arguments
    const uint8_t* mask = (const uint8_t*)dev(10);
    const int64_t ms_ok[3] = {0, 0, 336};
    const int64_t ms_short[3] = {0, 0, 332};
    const int64_t ms_odd[3] = {0, 2, 336};
    CHECK_EQ(fa_bwd_ext(q, k, v, o, g, lse, dq, dk, dv, B, H, Sq, Sk, D, mask, ms_short, 0.0f, 1, 0, sc, 1,
                        FA_BF16, ws, wd, nullptr), FA_ERR_MASK_DROPOUT);
    CHECK_EQ(fa_bwd_ext(q, k, v, o, g, lse, dq, dk, dv, B, H, Sq, Sk, D, mask, ms_odd, 0.0f, 1, 0, sc, 1,
                        FA_BF16, ws, wd, nullptr), FA_ERR_MASK_DROPOUT);
    CHECK_EQ(fa_bwd_ext(q, k, v, o, g, lse, dq, dk, dv, B, H, Sq, Sk, D, mask + 2, ms_ok, 0.0f, 1, 0, sc, 1,
                        FA_BF16, ws, wd, nullptr), FA_ERR_MASK_DROPOUT);
    CHECK_EQ(fa_bwd_ext(q, k, v, o, g, lse, dq, dk, dv, B, H, Sq, Sk, D, mask, ms_ok, 1.0f, 1, 0, sc, 1,
                        FA_BF16, ws, wd, nullptr), FA_ERR_MASK_DROPOUT);
    CHECK_EQ(fa_bwd_ext(q, k, v, o, g, lse, dq, dk, dv, B, H, Sq, Sk, D, mask, ms_ok, -0.5f, 1, 0, sc, 1,
                        FA_BF16, ws, wd, nullptr), FA_ERR_MASK_DROPOUT);
    CHECK_EQ(fa_bwd_ext(q, k, v, o, g, lse, dq, dk, dv, B, H, Sq, Sk, D, mask, ms_ok,
                        std::numeric_limits<float>::quiet_NaN(), 1, 0, sc, 1, FA_BF16, ws, wd, nullptr),
             FA_ERR_MASK_DROPOUT);
    CHECK_EQ(fa_bwd_ext(q, k, v, o, g, lse, dq, dk, dv, B, H, Sq, Sk, D, mask, ms_ok, 0.25f, 1, 0, sc, 1,
                        FA_BF16, ws, wd, nullptr), FA_OK);
    // strided: 24 strides, the gradients [B, S, H, D]
    int64_t st[24];
    const int len[8] = {Sq, Sk, Sk, Sq, Sq, Sq, Sk, Sk};
    for (int t = 0; t < 8; ++t) {
        st[3 * t] = (int64_t)H * len[t] * D;
        st[3 * t + 1] = t >= 5 ? D : (int64_t)len[t] * D;
        st[3 * t + 2] = t >= 5 ? (int64_t)H * D : D;
    }
    CHECK_EQ(fa_bwd_strided(q, k, v, o, g, lse, dq, dk, dv, B, H, Sq, Sk, D, st, nullptr, nullptr, 0.0f, 0, 0, sc,
                            1, FA_BF16, 1, ws, wd, nullptr), FA_OK);
    CHECK_EQ(g_stub.diag, Sk - Sq);
    // the causal diagonal at an explicit offset, clamped to [-Sq, Sk]
    const int64_t offs[4] = {-3, INT64_MIN, INT64_MAX, 0};
    const int want[4] = {-3, -Sq, Sk, 0};
    for (int i = 0; i < 4; ++i) {
        g_stub.last = StubState::kNone;
        CHECK_EQ(fa_bwd_causal_offset(q, k, v, o, g, lse, dq, dk, dv, B, H, Sq, Sk, D, st, nullptr, nullptr, 0.0f,
                                      0, 0, sc, offs[i], FA_BF16, ws, wd, nullptr), FA_OK);
        CHECK_EQ(g_stub.last, StubState::kBwd);
        CHECK_EQ(g_stub.diag, want[i]);
    }
    st[3 * 6 + 2] = 8;   // dk rows overlapping
    CHECK_EQ(fa_bwd_strided(q, k, v, o, g, lse, dq, dk, dv, B, H, Sq, Sk, D, st, nullptr, nullptr, 0.0f, 0, 0, sc,
                            1, FA_BF16, 1, ws, wd, nullptr), FA_ERR_STRIDE);
}

static void ext_checks() {
    const float sc = 0.125f;
    void *q = dev(0), *k = dev(1), *v = dev(2), *o = dev(3);
    float* lse = devf(4);
    const uint8_t* mask = (const uint8_t*)dev(10);
    const int64_t ms_ok[3] = {0, 0, 300};
    const int64_t ms_short[3] = {0, 0, 296};
    CHECK_EQ(fa_fwd_ext(q, k, v, o, lse, 1, 4, 256, 300, 128, mask, ms_short, 0.0f, 1, 0, sc, 1, FA_F16, nullptr),
             FA_ERR_MASK_DROPOUT);
    CHECK_EQ(fa_fwd_ext(q, k, v, o, lse, 1, 4, 256, 300, 128, mask, nullptr, 0.0f, 1, 0, sc, 1, FA_F16, nullptr),
             FA_ERR_MASK_DROPOUT);
    CHECK_EQ(fa_fwd_ext(q, k, v, o, lse, 1, 4, 256, 300, 128, nullptr, nullptr, 1.5f, 1, 0, sc, 1, FA_F16,
                        nullptr), FA_ERR_MASK_DROPOUT);
    CHECK_EQ(fa_fwd_ext(q, k, v, o, lse, INT_MAX, INT_MAX, INT_MAX, INT_MAX, 128, nullptr, nullptr, 0.0f, 1, 0, sc,
                        1, FA_F16, nullptr), FA_ERR_SHAPE);
    // no dropout: the tuned kernel (masked instance with a mask)
    CHECK_EQ(fa_fwd_ext(q, k, v, o, lse, 1, 4, 256, 300, 128, mask, ms_ok, 0.0f, 1, 0, sc, 1, FA_F16, nullptr),
             FA_OK);
    CHECK_EQ(g_stub.last, StubState::kFwd);
    CHECK_EQ(g_stub.masked, 1);
    CHECK_EQ(g_stub.drop_t, 0);
    // dropout: the dropout instances of the tuned kernel, threshold round(p * 65536)
    CHECK_EQ(fa_fwd_ext(q, k, v, o, lse, 1, 4, 256, 300, 128, mask, ms_ok, 0.1f, 1, 0, sc, 1, FA_F16, nullptr),
             FA_OK);
    CHECK_EQ(g_stub.last, StubState::kFwdDrop);
    CHECK_EQ(g_stub.masked, 1);
    CHECK_EQ(g_stub.drop_t, 6554);
    // a row stride the tuned kernel's 32-bit head offsets do not reach (a head
    // padded to 320 rows spans 2^31 bytes or more) but the general kernel's do
    // (256 rows): the general kernel
    {
        const int64_t r = 4000000;
        const int64_t st[12] = {100 * r, 100 * r, r, 100 * r, 100 * r, r, 100 * r, 100 * r, r, 100 * r, 100 * r, r};
        g_stub.last = StubState::kNone;
        CHECK_EQ(fa_fwd_ext_strided(q, k, v, o, lse, 1, 1, 100, 100, 128, st, nullptr, nullptr, 0.1f, 1, 0, sc, 1,
                                    FA_F16, nullptr), FA_OK);
        CHECK_EQ(g_stub.last, StubState::kExt);
        CHECK_EQ(g_stub.drop_t, 6554);
    }
    // the causal diagonal: bottom-right by default, an explicit offset clamped to [-Sq, Sk]
    {
        const int64_t st[12] = {4 * 256 * 128, 256 * 128, 128, 4 * 300 * 128, 300 * 128, 128,
                                4 * 300 * 128, 300 * 128, 128, 4 * 256 * 128, 256 * 128, 128};
        CHECK_EQ(fa_fwd_ext_strided(q, k, v, o, lse, 1, 4, 256, 300, 128, st, nullptr, nullptr, 0.0f, 1, 0, sc, 1,
                                    FA_F16, nullptr), FA_OK);
        CHECK_EQ(g_stub.diag, 300 - 256);
        const int64_t offs[6] = {0, -17, 299, INT64_MIN, INT64_MAX, -256};
        const int want[6] = {0, -17, 299, -256, 300, -256};
        for (int i = 0; i < 6; ++i) {
            CHECK_EQ(fa_fwd_causal_offset(q, k, v, o, lse, 1, 4, 256, 300, 128, st, nullptr, nullptr, 0.1f, 1, 0,
                                          sc, offs[i], FA_F16, nullptr), FA_OK);
            CHECK_EQ(g_stub.last, StubState::kFwdDrop);
            CHECK_EQ(g_stub.diag, want[i]);
        }
        CHECK_EQ(fa_fwd_causal_offset(q, k, v, o, lse, 1, 4, 256, 300, 128, nullptr, nullptr, nullptr, 0.0f, 1, 0,
                                      sc, 5, FA_F16, nullptr), FA_ERR_NULL);
    }
    // a dropout probability that rounds to 65536 is refused
    CHECK_EQ(fa_fwd_ext(q, k, v, o, lse, 1, 4, 256, 300, 128, nullptr, nullptr, 0.99999994f, 1, 0, sc, 1, FA_F16,
                        nullptr), FA_ERR_MASK_DROPOUT);
}

static void diag_checks() {
    const float sc = 0.125f;
    void *q = dev(0), *k = dev(1), *v = dev(2), *o = dev(3);
    float *lse = devf(4), *o32 = devf(5);
    uint32_t* tiles = (uint32_t*)dev(6);
    CHECK_EQ(fa_fwd_diag(q, k, v, o, lse, o32, tiles, 1, 2, 300, 300, 256, sc, 1, FA_F16, 0, nullptr),
             FA_ERR_UNSUPPORTED);
    CHECK_EQ(fa_fwd_diag(q, k, v, o, lse, o32, tiles, 1, 2, 300, 300, 64, sc, 1, FA_F16, 4, nullptr),
             FA_ERR_UNSUPPORTED);
    CHECK_EQ(fa_fwd_diag(q, k, v, o, lse, (float*)q, tiles, 1, 2, 300, 300, 64, sc, 1, FA_F16, 0, nullptr),
             FA_ERR_ALIAS);
    CHECK_EQ(fa_fwd_diag(q, k, v, o, lse, o32, (uint32_t*)o32, 1, 2, 300, 300, 64, sc, 1, FA_F16, 0, nullptr),
             FA_ERR_ALIAS);
    CHECK_EQ(fa_fwd_diag(q, k, v, o, lse, o32, tiles, 1, 2, 300, 300, 64, sc, 1, FA_F16, FA_DIAG_REVERSE_ORDER,
                         nullptr), FA_OK);
    CHECK_EQ(g_stub.last, StubState::kDiag);
    CHECK_EQ(fa_fwd_diag_tile_slots(1, 2, 300, 64, 1), (int64_t)g_stub.grid * 8);
    CHECK_EQ(fa_fwd_diag_tile_slots(1, 2, 300, 256, 1), 0);
}

static void status_checks() {
    for (int s = -1; s <= 12; ++s) {
        const char* t = fa_status_string(s);
        CHECK_EQ(t != nullptr && std::strlen(t) > 0, 1);
    }
    CHECK_EQ(fa_version() >= 10400, 1);
}

int main() {
    // no device answers: the compute-unit count falls back to 256
    g_stub.device_cus = 0;
    fwd_checks();
    strided_checks();
    plan_checks(256);
    naive_checks();
    bwd_checks();
    ext_checks();
    diag_checks();
    status_checks();
    // a device with 304 compute units: read once, then cached
    g_stub.device_cus = 304;
    g_stub.attribute_queries = 0;
    const float sc = 0.125f;
    // 1x40x8192x128 causal: 40 * 32 = 1280 blocks, no split either way; 1x4x8192: 128 blocks,
    // causal -> split; 1x1x32768 non-causal: 128 blocks, 2n = 256 <= 304 -> split, but not at 256
    CHECK_EQ(fa_fwd(dev(0), dev(1), dev(2), dev(3), nullptr, 1, 1, 32768, 128, sc, 0, FA_BF16, nullptr), FA_OK);
    CHECK_EQ(g_stub.split, 1);
    CHECK_EQ(fa_fwd(dev(0), dev(1), dev(2), dev(3), nullptr, 1, 2, 32768, 128, sc, 0, FA_BF16, nullptr), FA_OK);
    CHECK_EQ(g_stub.split, 0);
    CHECK_EQ(g_stub.attribute_queries, 1);
    plan_checks(304);
    CHECK_EQ(g_stub.attribute_queries, 1);
    std::printf("host checks passed: %d\n", g_checks);
    return 0;
}
