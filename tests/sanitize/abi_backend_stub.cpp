// abi_backend_stub.cpp -- host-only stand-in for the kernel side of libkda,
// used to build the C ABI layer (kda_api.cpp) with AddressSanitizer and
// UndefinedBehaviorSanitizer on a machine without a GPU.
//
// Test infrastructure: the predicates follow the built combinations that
// include/kda.h documents, the workspace sizes are arbitrary positive values,
// and every launcher records the problem it was handed (so the driver can
// check what the validation forwarded) and returns g_stub_status.
#include <hip/hip_runtime.h>

#include "kda_internal.hpp"
#include "abi_backend_stub.hpp"

StubRecord g_stub;
hipError_t g_stub_status = hipSuccess;

int g_stub_device = 0;          // the current device the stub reports
int g_stub_stream_device = 0;   // the device every non-null stream belongs to

extern "C" const char *hipGetErrorString(hipError_t e) {
    return e == hipSuccess ? "hipSuccess" : "stub launch failure";
}
extern "C" hipError_t hipGetDevice(int *device) {
    *device = g_stub_device;
    return hipSuccess;
}
extern "C" hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t *device) {
    *device = g_stub_stream_device;
    return hipSuccess;
}

namespace kda {

bool decode_supported(int dk, int dv) {
    return dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128);
}
hipError_t launch_decode(int n_pairs, int dk, int dv, bool bf16, Gate gate, InputForm form,
                         const void *q, const void *, const void *, const float *g,
                         const float *, float scale, float *state, void *o, hipStream_t) {
    g_stub = StubRecord();
    g_stub.kind = StubRecord::Decode;
    g_stub.n_pairs = n_pairs;
    g_stub.dk = dk;
    g_stub.dv = dv;
    g_stub.bf16 = bf16;
    g_stub.gate = static_cast<int>(gate);
    g_stub.form_flags = form.flags();
    g_stub.q = q;
    g_stub.g = g;
    g_stub.scale = scale;
    g_stub.state = state;
    g_stub.o = o;
    return g_stub_status;
}

bool output_stage_supported(int dv) {
    return dv == 16 || dv == 32 || dv == 64 || dv == 128 || dv == 256;
}
hipError_t launch_output_rmsnorm_gate(int64_t rows, int dv, bool bf16, const void *o,
                                      const void *, const float *, float, void *out,
                                      hipStream_t) {
    g_stub = StubRecord();
    g_stub.kind = StubRecord::Output;
    g_stub.rows = rows;
    g_stub.dv = dv;
    g_stub.bf16 = bf16;
    g_stub.o = out;
    g_stub.q = o;
    return g_stub_status;
}

// A fake device address per device (never dereferenced).
hipError_t noalloc_scratch(int device, void **ptr) {
    *ptr = reinterpret_cast<void *>(uintptr_t(0x7f0000000000ull) + (uintptr_t(device) << 32));
    return hipSuccess;
}

bool mfma_path_supported(int dk, int dv, int chunk, bool bf16) {
    return bf16 && dk == 128 && dv == 128 && chunk == 64;
}
size_t mfma_workspace_bytes(int64_t total_tokens, int64_t n_seqs, int heads, int chunk) {
    return (size_t)(max_chunks(total_tokens, n_seqs, chunk) * heads + 1) * 4096;
}
hipError_t launch_chunk_fwd_mfma(const ChunkProblem &p) {
    g_stub = StubRecord();
    g_stub.kind = StubRecord::PrefillMfma;
    g_stub.prefill = p;
    return g_stub_status;
}

bool f32_path_supported(int dk, int dv, int chunk, bool bf16) {
    if (bf16 || dk != dv) return false;
    const bool small = (dk == 16 || dk == 32 || dk == 64) &&
                       (chunk == 16 || chunk == 32 || chunk == 64);
    return small || (dk == 128 && chunk == 64);
}
size_t f32_workspace_bytes(int64_t, int64_t, int, int) { return 0; }
hipError_t launch_chunk_fwd_f32(const ChunkProblem &p) {
    g_stub = StubRecord();
    g_stub.kind = StubRecord::PrefillF32;
    g_stub.prefill = p;
    return g_stub_status;
}
bool f32_mfma_applies(int dk, int dv, bool bf16, Gate, InputForm) {
    return !bf16 && dk == 128 && dv == 128;
}
size_t f32_mfma_workspace_bytes(int64_t total_tokens, int64_t n_seqs, int heads) {
    return (size_t)(total_tokens / 16 + n_seqs + 1) * heads * 2048;
}
hipError_t launch_chunk_fwd_f32_mfma(const ChunkProblem &p) {
    g_stub = StubRecord();
    g_stub.kind = StubRecord::PrefillF32Mfma;
    g_stub.prefill = p;
    return g_stub_status;
}

bool bwd_supported(int dk, int dv, int chunk) {
    if (dk != dv) return false;
    if (dk == 16) return chunk == 16 || chunk == 32 || chunk == 64;
    if (dk == 32 || dk == 64) return chunk == 16 || chunk == 32;
    return dk == 128 && (chunk == 16 || chunk == 32 || chunk == 64);
}
size_t bwd_workspace_bytes(int64_t total_tokens, int n_seqs, int heads, int d, int chunk) {
    return (size_t)(total_tokens / chunk + n_seqs + 1) * heads * d * 8;
}
hipError_t launch_chunk_bwd(const ChunkBwdProblem &p) {
    g_stub = StubRecord();
    g_stub.kind = StubRecord::Backward;
    g_stub.bwd = p;
    return g_stub_status;
}

}  // namespace kda
