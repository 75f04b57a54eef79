// launch_stubs.cpp -- host-only stand-ins for the kernel launchers and the
// three HIP runtime calls fa_api.cpp makes, so that the host validation and
// launch planning can be built with AddressSanitizer and
// UndefinedBehaviorSanitizer and exercised without a GPU.  Each launcher
// records what it was asked to launch; nothing is dereferenced.
#include <hip/hip_runtime_api.h>

#include "fa_bwd.h"
#include "fa_ext.h"
#include "fa_launch.h"
#include "fa_naive.h"
#include "launch_stubs.h"

StubState g_stub;

extern "C" hipError_t hipGetDevice(int* dev) {
    ++g_stub.device_queries;
    if (g_stub.device_cus <= 0) return hipErrorNoDevice;
    *dev = 0;
    return hipSuccess;
}

extern "C" hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int dev) {
    ++g_stub.attribute_queries;
    if (attr != hipDeviceAttributeMultiprocessorCount || dev != 0 || g_stub.device_cus <= 0)
        return hipErrorInvalidValue;
    *value = g_stub.device_cus;
    return hipSuccess;
}

extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }

namespace fa {
hipError_t launch_fwd(const FwdParams& p, int D, int dtype, bool causal, int64_t grid, bool split, hipStream_t) {
    g_stub.last = StubState::kFwd;
    g_stub.grid = grid;
    g_stub.split = split;
    g_stub.nqb = p.nqb;
    g_stub.D = D;
    g_stub.dtype = dtype;
    g_stub.causal = causal;
    g_stub.masked = p.mask != nullptr;
    g_stub.drop_t = p.drop_t;
    g_stub.diag = p.diag;
    return hipSuccess;
}
hipError_t launch_fwd_drop(const FwdParams& p, int D, int dtype, bool causal, int64_t grid, bool split,
                           hipStream_t s) {
    launch_fwd(p, D, dtype, causal, grid, split, s);
    g_stub.last = StubState::kFwdDrop;
    return hipSuccess;
}
hipError_t launch_fwd_diag(const FwdParams& p, int D, int, bool, int64_t grid, bool split, hipStream_t) {
    g_stub.last = StubState::kDiag;
    g_stub.grid = grid;
    g_stub.split = split;
    g_stub.nqb = p.nqb;
    g_stub.D = D;
    return hipSuccess;
}
namespace bwd {
hipError_t launch_bwd(const BwdParams& p, int D, int, int, hipStream_t) {
    g_stub.last = StubState::kBwd;
    g_stub.D = D;
    g_stub.diag = p.diag;
    g_stub.nqb = p.nqb;
    return hipSuccess;
}
}  // namespace bwd
namespace ext {
hipError_t launch_ext(const ExtParams& p, int D, int, int, hipStream_t) {
    g_stub.last = StubState::kExt;
    g_stub.D = D;
    g_stub.diag = p.diag;
    g_stub.nqb = p.nqb;
    g_stub.drop_t = p.drop_t;
    return hipSuccess;
}
}  // namespace ext
namespace naive {
hipError_t launch_naive(const NaiveParams&, int, int D, int, hipStream_t) {
    g_stub.last = StubState::kNaive;
    g_stub.D = D;
    return hipSuccess;
}
}  // namespace naive
}  // namespace fa
