// fa_api.cpp -- C ABI of the fused attention forward: argument validation,
// launch planning and dispatch.  Declarations and the meaning of every
// argument are in include/fa.h.
//
// Validation runs entirely on the host, before any HIP call, so a rejected
// call enqueues nothing.  The launch is asynchronous on the caller's stream;
// the library never allocates, frees or synchronises.
#include <algorithm>
#include <cmath>
#include <cstdint>

#include "fa.h"
#include "fa_launch.h"

namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;

int validate_shape(int B, int H, int S, int D, int dtype) {
    if (B < 1 || H < 1 || S < 1) return FA_ERR_SHAPE;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    // Per-head byte offsets are 32-bit (buffer descriptors): the head plus the
    // padding rows of its last query block must stay below 2^31 bytes.
    const int64_t head_bytes = ((int64_t)S + fa::kBlockQ) * D * 2;
    if (head_bytes >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
    const int64_t elems = (int64_t)B * H * S * D;
    if (elems >= (int64_t(1) << 40)) return FA_ERR_SHAPE;
    const int64_t grid = (int64_t)B * H * ((S + fa::kBlockQ - 1) / fa::kBlockQ);
    if (grid >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
    return FA_OK;
}

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

}  // namespace

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
        default: return "unknown status";
    }
}

int fa_fwd_plan(int B, int H, int S, int D, int causal, int dtype, int* block_q, int* block_kv,
                int64_t* grid, int64_t* tiles) {
    const int st = validate_shape(B, H, S, D, dtype);
    if (st != FA_OK) return st;
    const int br = fa::kBlockQ, bc = fa::kBlockKV;
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

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int S,
           int D, float scale, int causal, int dtype, void* stream) {
    if (!q || !k || !v || !o) return FA_ERR_NULL;
    const int st = validate_shape(B, H, S, D, dtype);
    if (st != FA_OK) return st;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse) & 15)
        return FA_ERR_ALIGN;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_SCALE;
    const int64_t tbytes = (int64_t)B * H * S * D * 2;
    const int64_t lbytes = (int64_t)B * H * S * 4;
    if (overlap(o, tbytes, q, tbytes) || overlap(o, tbytes, k, tbytes) || overlap(o, tbytes, v, tbytes))
        return FA_ERR_ALIAS;
    if (lse && (overlap(lse, lbytes, q, tbytes) || overlap(lse, lbytes, k, tbytes) ||
                overlap(lse, lbytes, v, tbytes) || overlap(lse, lbytes, o, tbytes)))
        return FA_ERR_ALIAS;

    fa::FwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.S = S;
    p.BH = B * H;
    p.nqb = (S + fa::kBlockQ - 1) / fa::kBlockQ;
    p.scale_log2e = (float)((double)scale * 1.4426950408889634074);
    const int64_t grid = (int64_t)p.BH * p.nqb;
    const hipError_t err = fa::launch_fwd(p, D, dtype, causal != 0, grid, (hipStream_t)stream);
    return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
