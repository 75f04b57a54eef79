// launch_stubs.h -- what the stand-in launchers of launch_stubs.cpp record.
#pragma once
#include <stdint.h>

struct StubState {
    enum Kind { kNone, kFwd, kFwdDrop, kDiag, kBwd, kExt, kNaive };
    Kind last = kNone;
    int64_t grid = 0;
    bool split = false;
    int nqb = 0;
    int D = 0;
    int dtype = 0;
    bool causal = false;
    bool masked = false;
    uint32_t drop_t = 0;
    int diag = 0;
    int device_cus = 0;          // 0: no device answers (compute units fall back to 256)
    int device_queries = 0;
    int attribute_queries = 0;
};

extern StubState g_stub;
