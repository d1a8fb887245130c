// abi_backend_stub.hpp -- what the stub launchers record (test infrastructure).
#pragma once

#include "kda_internal.hpp"

struct StubRecord {
    enum Kind { None, Decode, Output, PrefillMfma, PrefillF32, PrefillF32Mfma, Backward } kind = None;
    int n_pairs = 0, dk = 0, dv = 0, gate = -1, form_flags = 0;
    int64_t rows = 0;
    bool bf16 = false;
    float scale = 0.f;
    const void *q = nullptr;
    const float *g = nullptr;
    float *state = nullptr;
    void *o = nullptr;
    kda::ChunkProblem prefill{};
    kda::ChunkBwdProblem bwd{};
};

extern StubRecord g_stub;
extern hipError_t g_stub_status;
extern int g_stub_device, g_stub_stream_device;
