// fa_bwd_noalloc.hip -- the allocation-free form of the deterministic
// backward: fa_bwd with its workspace taken from a fixed, file-scope device
// array instead of a caller-supplied buffer.
//
// The array (kNoAllocScratchBytes) holds the backward's row dot products
// D_i = dout_i . o_i (4 bytes per query row, written in full by the first
// kernel before any kernel reads them, so nothing needs clearing).  Each GPU
// holds its own copy, for the life of the process.  Its device address is
// looked up once per device, with that device current, on the first call
// there (hipGetSymbolAddress; the array's name in host code is a host-side
// stand-in, never a device address).
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa.h"

namespace {

constexpr int64_t kNoAllocScratchBytes = int64_t(16) << 20;   // 16 MiB: B*H*Sq <= 4,194,304 rows
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // per device; null until looked up

// The device address of `scratch` on the current device, or null.
void* scratch_on_current_device(int* status) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        *status = FA_ERR_HIP;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        const hipError_t err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            *status = FA_ERR_HIP;
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *status = FA_OK;
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int64_t fa_bwd_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

extern "C" int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv, int B, int H, int Sq, int Sk, int D,
                              float scale, int causal, int dtype, void* stream) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
    const int64_t need = fa_bwd_workspace_bytes(B, H, Sq, D, 1);
    if (need <= 0) return FA_ERR_SHAPE;
    if (need > kNoAllocScratchBytes) return FA_ERR_SCRATCH;
    int st = FA_OK;
    void* ws = scratch_on_current_device(&st);
    if (ws == nullptr) return st;
    return fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Sq, Sk, D, scale, causal, dtype, 1, ws,
                  kNoAllocScratchBytes, stream);
}
