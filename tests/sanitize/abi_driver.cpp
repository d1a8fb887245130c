// abi_driver.cpp -- exercises every entry point of the C ABI layer against the
// stub backend, built with AddressSanitizer and UndefinedBehaviorSanitizer
// (test infrastructure; no GPU).  Device pointers are fake, aligned addresses:
// the ABI layer never dereferences them, and the stub launchers only record
// them.  Exits non-zero on the first failed check; a sanitizer report aborts.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>

#include "kda.h"
#include "abi_backend_stub.hpp"

extern "C" {
kda_status c_fwd_with_dtype(const kda_shape *s, int dtype, const void *q, const void *k,
                            const void *v, const float *g, const float *beta, void *o, void *ws,
                            size_t wsb);
size_t c_workspace_with_dtype(const kda_shape *s, int dtype);
kda_status c_decode_with_dtype(int dtype, const void *q, const void *k, const void *v,
                               const float *g, const float *beta, float *state, void *o);
kda_status c_output_with_dtype(int dtype, const void *o, const void *gate, const float *w,
                               void *out);
kda_status c_bwd_with_dtype(const kda_shape *s, int dtype);
}

static int g_checks = 0;

#define CHECK(cond)                                                                   \
    do {                                                                              \
        ++g_checks;                                                                   \
        if (!(cond)) {                                                                \
            std::fprintf(stderr, "%s:%d: check failed: %s (last error: %s)\n",         \
                         __FILE__, __LINE__, #cond, kda_last_error());                \
            std::exit(1);                                                             \
        }                                                                             \
    } while (0)

// Distinct fake device addresses, 256-byte aligned, never dereferenced.
static void *dev(int i) { return reinterpret_cast<void *>(uintptr_t(0x7000000000ull) + 0x100000ull * i); }
static float *devf(int i) { return static_cast<float *>(dev(i)); }
static const int32_t *devi(int i) { return static_cast<const int32_t *>(dev(i)); }
static void *misaligned(int i) { return static_cast<char *>(dev(i)) + 8; }

static kda_shape bf16_shape(int B = 2, int T = 300, int H = 4) {
    kda_shape s;
    s.batch = B;
    s.seqlen = T;
    s.num_heads = H;
    s.d_k = 128;
    s.d_v = 128;
    s.chunk_size = 64;
    s.num_seqs = B;
    s.dtype = KDA_BF16;
    return s;
}

static kda_status fwd(const kda_shape &s, void *ws, size_t wsb, const void *q = dev(1),
                      void *o = dev(7), const int32_t *cu = nullptr, const float *s0 = devf(8),
                      float *sf = devf(9)) {
    return kda_chunk_fwd(&s, q, dev(2), dev(3), devf(4), devf(5), 0.088f, s0, cu, o, sf, ws, wsb,
                         nullptr);
}

static void prefill_checks() {
    kda_shape s = bf16_shape();
    const size_t need = kda_chunk_fwd_workspace_bytes(&s);
    CHECK(need > 0);
    // A valid call reaches the MFMA launcher with every field forwarded.
    CHECK(fwd(s, dev(20), need) == KDA_OK);
    CHECK(g_stub.kind == StubRecord::PrefillMfma);
    CHECK(g_stub.prefill.batch == 2 && g_stub.prefill.seqlen == 300 && g_stub.prefill.heads == 4);
    CHECK(g_stub.prefill.allow_overlap);
    CHECK(g_stub.prefill.q == dev(1) && g_stub.prefill.o == dev(7) && g_stub.prefill.cu == nullptr);
    CHECK(g_stub.prefill.gate == kda::Gate::PerChannel && g_stub.prefill.form.flags() == 0);
    CHECK(std::strcmp(kda_last_error(), "") == 0);

    // Shape errors.
    CHECK(kda_chunk_fwd(nullptr, dev(1), dev(2), dev(3), devf(4), devf(5), 1.f, nullptr, nullptr,
                        dev(7), nullptr, dev(20), need, nullptr) == KDA_ERR_INVALID_ARGUMENT);
    CHECK(std::strlen(kda_last_error()) > 0);
    for (int dt : {7, -1, 2})
        CHECK(c_fwd_with_dtype(&s, dt, dev(1), dev(2), dev(3), devf(4), devf(5), dev(7), dev(20),
                               need) == KDA_ERR_INVALID_ARGUMENT &&
              c_workspace_with_dtype(&s, dt) == 0);
    kda_shape bad = s;
    int32_t kda_shape::*const fields[] = {&kda_shape::batch, &kda_shape::num_heads, &kda_shape::d_k,
                                           &kda_shape::d_v, &kda_shape::chunk_size,
                                           &kda_shape::num_seqs};
    for (auto f : fields) {
        bad = s;
        bad.*f = 0;
        CHECK(fwd(bad, dev(20), need) == KDA_ERR_INVALID_ARGUMENT);
        bad.*f = -5;
        CHECK(fwd(bad, dev(20), need) == KDA_ERR_INVALID_ARGUMENT);
    }
    bad = s;
    bad.d_k = 96;
    bad.d_v = 96;
    CHECK(fwd(bad, dev(20), need) == KDA_ERR_UNSUPPORTED);
    bad = s;
    bad.chunk_size = 32;
    CHECK(fwd(bad, dev(20), need) == KDA_ERR_UNSUPPORTED);
    bad = s;
    bad.seqlen = INT32_MAX;
    CHECK(fwd(bad, dev(20), need) == KDA_ERR_INVALID_ARGUMENT);
    bad = s;
    bad.num_seqs = 3;   // without cu_seqlens num_seqs must equal batch
    CHECK(fwd(bad, dev(20), kda_chunk_fwd_workspace_bytes(&bad)) == KDA_ERR_INVALID_ARGUMENT);

    // Pointer errors: NULL, misaligned, aliased.
    CHECK(fwd(s, dev(20), need, nullptr) == KDA_ERR_INVALID_ARGUMENT);
    CHECK(fwd(s, dev(20), need, misaligned(1)) == KDA_ERR_INVALID_ARGUMENT);
    CHECK(fwd(s, dev(20), need, dev(1), dev(1)) == KDA_ERR_INVALID_ARGUMENT);   // o aliases q
    CHECK(fwd(s, dev(20), need, dev(1), misaligned(7)) == KDA_ERR_INVALID_ARGUMENT);
    CHECK(fwd(s, dev(20), need, dev(1), dev(7), nullptr, devf(8), devf(8)) == KDA_OK);   // in place
    CHECK(fwd(s, dev(20), need, dev(1), dev(7), nullptr, nullptr, nullptr) == KDA_OK);
    CHECK(g_stub.prefill.s0 == nullptr && g_stub.prefill.s_final == nullptr);
    CHECK(kda_chunk_fwd(&s, dev(1), dev(2), dev(3), nullptr, devf(5), 1.f, nullptr, nullptr,
                        dev(7), nullptr, dev(20), need, nullptr) == KDA_ERR_INVALID_ARGUMENT);

    // Workspace errors.
    CHECK(fwd(s, nullptr, need) == KDA_ERR_INVALID_ARGUMENT);
    CHECK(fwd(s, static_cast<char *>(dev(20)) + 16, need) == KDA_ERR_INVALID_ARGUMENT);
    CHECK(fwd(s, dev(20), need - 1) == KDA_ERR_WORKSPACE_TOO_SMALL);
    CHECK(fwd(s, dev(20), 0) == KDA_ERR_WORKSPACE_TOO_SMALL);

    // Packed sequences.
    kda_shape v = bf16_shape(1, 1000, 4);
    v.num_seqs = 5;
    const size_t vneed = kda_chunk_fwd_workspace_bytes(&v);
    CHECK(vneed >= need / 2);
    CHECK(fwd(v, dev(20), vneed, dev(1), dev(7), devi(10)) == KDA_OK);
    CHECK(g_stub.prefill.cu == devi(10) && g_stub.prefill.n_seqs == 5);
    kda_shape v2 = v;
    v2.batch = 2;   // cu_seqlens needs batch 1
    CHECK(fwd(v2, dev(20), vneed, dev(1), dev(7), devi(10)) == KDA_ERR_INVALID_ARGUMENT);
    CHECK(kda_chunk_fwd(&v, dev(1), dev(2), dev(3), devf(4), devf(5), 1.f, nullptr,
                        reinterpret_cast<const int32_t *>(static_cast<char *>(dev(10)) + 2),
                        dev(7), nullptr, dev(20), vneed, nullptr) == KDA_ERR_INVALID_ARGUMENT);

    // An empty problem needs no tensors.
    kda_shape e = bf16_shape(1, 0, 4);
    CHECK(kda_chunk_fwd(&e, nullptr, nullptr, nullptr, nullptr, nullptr, 1.f, nullptr, nullptr,
                        nullptr, nullptr, dev(20), kda_chunk_fwd_workspace_bytes(&e),
                        nullptr) == KDA_OK);

    // fp32 storage goes to the fp32 path; at d = 128 to the MFMA factors path,
    // which needs a workspace.
    kda_shape f = bf16_shape(1, 50, 2);
    f.dtype = KDA_F32;
    f.d_k = f.d_v = 32;
    f.chunk_size = 16;
    CHECK(kda_chunk_fwd_workspace_bytes(&f) == 0);
    CHECK(fwd(f, nullptr, 0) == KDA_OK && g_stub.kind == StubRecord::PrefillF32);
    f.d_k = f.d_v = 128;
    f.chunk_size = 64;
    const size_t fneed = kda_chunk_fwd_workspace_bytes(&f);
    CHECK(fneed > 0);
    CHECK(fwd(f, nullptr, 0) == KDA_ERR_INVALID_ARGUMENT);
    CHECK(fwd(f, dev(20), fneed - 1) == KDA_ERR_WORKSPACE_TOO_SMALL);
    CHECK(fwd(f, dev(20), fneed) == KDA_OK && g_stub.kind == StubRecord::PrefillF32Mfma);
    CHECK(g_stub.prefill.workspace == dev(20) && g_stub.prefill.chunk == 64);
    // Every gate layout and input form too.
    CHECK(kda_chunk_fwd_scalar_gate(&f, dev(1), dev(2), dev(3), nullptr, devf(5), 1.f, nullptr,
                                    nullptr, dev(7), nullptr, dev(20), fneed, nullptr) == KDA_OK &&
          g_stub.kind == StubRecord::PrefillF32Mfma && g_stub.prefill.gate == kda::Gate::None);
    {
        kda_inputs_form lf = {KDA_GATE_PER_CHANNEL, 1, 1, 1, 1e-6f};
        CHECK(kda_chunk_fwd_ex(&f, &lf, dev(1), dev(2), dev(3), devf(4), devf(5), 1.f, nullptr,
                               nullptr, dev(7), nullptr, dev(20), fneed, nullptr) == KDA_OK &&
              g_stub.kind == StubRecord::PrefillF32Mfma && g_stub.prefill.form.flags() == 7);
    }

    // Scalar gate: NULL g is "no gate"; the ex form descriptor.
    CHECK(kda_chunk_fwd_scalar_gate(&s, dev(1), dev(2), dev(3), nullptr, devf(5), 1.f, nullptr,
                                    nullptr, dev(7), nullptr, dev(20), need, nullptr) == KDA_OK);
    CHECK(g_stub.prefill.gate == kda::Gate::None && g_stub.prefill.g == nullptr);
    const float *g4 = reinterpret_cast<const float *>(static_cast<char *>(dev(4)) + 4);
    CHECK(kda_chunk_fwd_scalar_gate(&s, dev(1), dev(2), dev(3), g4, devf(5), 1.f, nullptr, nullptr,
                                    dev(7), nullptr, dev(20), need, nullptr) == KDA_OK);
    CHECK(g_stub.prefill.gate == kda::Gate::Scalar && g_stub.prefill.g == g4);
    kda_inputs_form form = {KDA_GATE_PER_CHANNEL, 1, 1, 1, 1e-6f};
    CHECK(kda_chunk_fwd_ex(&s, &form, dev(1), dev(2), dev(3), devf(4), devf(5), 1.f, nullptr,
                           nullptr, dev(7), nullptr, dev(20), need, nullptr) == KDA_OK);
    CHECK(g_stub.prefill.form.flags() == 7 && g_stub.prefill.form.eps == 1e-6f);
    form.eps = 0.f;
    CHECK(kda_chunk_fwd_ex(&s, &form, dev(1), dev(2), dev(3), devf(4), devf(5), 1.f, nullptr,
                           nullptr, dev(7), nullptr, dev(20), need, nullptr) ==
          KDA_ERR_INVALID_ARGUMENT);
    form = {9, 0, 0, 0, 0.f};
    CHECK(kda_chunk_fwd_ex(&s, &form, dev(1), dev(2), dev(3), devf(4), devf(5), 1.f, nullptr,
                           nullptr, dev(7), nullptr, dev(20), need, nullptr) ==
          KDA_ERR_INVALID_ARGUMENT);
    form = {KDA_GATE_NONE, 0, 0, 0, 0.f};
    CHECK(kda_chunk_fwd_ex(&s, &form, dev(1), dev(2), dev(3), devf(4), devf(5), 1.f, nullptr,
                           nullptr, dev(7), nullptr, dev(20), need, nullptr) ==
          KDA_ERR_INVALID_ARGUMENT);   // g must be NULL without a gate
    form = {KDA_GATE_SCALAR, 0, 0, 0, 0.f};
    CHECK(kda_chunk_fwd_ex(&s, &form, dev(1), dev(2), dev(3), nullptr, devf(5), 1.f, nullptr,
                           nullptr, dev(7), nullptr, dev(20), need, nullptr) ==
          KDA_ERR_INVALID_ARGUMENT);

    // A failing launch is reported as KDA_ERR_HIP with the runtime's text.
    g_stub_status = hipErrorInvalidConfiguration;
    CHECK(fwd(s, dev(20), need) == KDA_ERR_HIP);
    CHECK(std::strstr(kda_last_error(), "2^32") != nullptr);
    g_stub_status = hipErrorLaunchFailure;
    CHECK(fwd(s, dev(20), need) == KDA_ERR_HIP);
    g_stub_status = hipSuccess;
    CHECK(fwd(s, dev(20), need) == KDA_OK && std::strcmp(kda_last_error(), "") == 0);
}

static void noalloc_checks() {
    kda_shape s = bf16_shape(1, 2000, 8);
    auto call = [](const kda_shape &sh, hipStream_t stream) {
        return kda_chunk_fwd_noalloc(&sh, dev(1), dev(2), dev(3), devf(4), devf(5), 0.1f,
                                     nullptr, nullptr, dev(7), devf(9), stream);
    };
    // Fits: the launcher receives the device's scratch address as its workspace.
    CHECK(kda_chunk_fwd_workspace_bytes(&s) <= KDA_NOALLOC_SCRATCH_BYTES);
    g_stub_device = g_stub_stream_device = 3;
    CHECK(call(s, static_cast<hipStream_t>(dev(30))) == KDA_OK && g_stub.kind == StubRecord::PrefillMfma);
    CHECK(g_stub.prefill.workspace == reinterpret_cast<void *>(0x7f0000000000ull + (3ull << 32)));
    CHECK(g_stub.prefill.workspace_bytes == KDA_NOALLOC_SCRATCH_BYTES);
    CHECK(!g_stub.prefill.allow_overlap);   // the no-allocation path never creates a stream
    CHECK(call(s, nullptr) == KDA_OK);
    // A stream of another device is refused (the buffer is the current device's).
    g_stub_stream_device = 1;
    CHECK(call(s, static_cast<hipStream_t>(dev(30))) == KDA_ERR_INVALID_ARGUMENT);
    CHECK(std::strstr(kda_last_error(), "device 1") != nullptr);
    g_stub_device = g_stub_stream_device = 0;
    // Too large for the buffer: refused with a clear message, nothing enqueued.
    kda_shape big = bf16_shape(1, 1 << 20, 32);
    CHECK(kda_chunk_fwd_workspace_bytes(&big) > KDA_NOALLOC_SCRATCH_BYTES);
    g_stub = StubRecord();
    CHECK(call(big, nullptr) == KDA_ERR_WORKSPACE_TOO_SMALL);
    CHECK(g_stub.kind == StubRecord::None);
    CHECK(std::strstr(kda_last_error(), "kda_chunk_fwd with a workspace") != nullptr);
    // fp32 at d = 128: the MFMA factors path while its workspace fits the
    // buffer, else the fp32 kernel (no workspace), so every size runs.
    kda_shape f = bf16_shape(1, 2000, 8);
    f.dtype = KDA_F32;
    CHECK(kda_chunk_fwd_workspace_bytes(&f) <= KDA_NOALLOC_SCRATCH_BYTES);
    CHECK(call(f, nullptr) == KDA_OK && g_stub.kind == StubRecord::PrefillF32Mfma);
    CHECK(g_stub.prefill.workspace == reinterpret_cast<void *>(0x7f0000000000ull));
    f = bf16_shape(1, 1 << 20, 32);
    f.dtype = KDA_F32;
    CHECK(kda_chunk_fwd_workspace_bytes(&f) > KDA_NOALLOC_SCRATCH_BYTES);
    CHECK(call(f, nullptr) == KDA_OK && g_stub.kind == StubRecord::PrefillF32);
    // The usual validation still applies.
    CHECK(kda_chunk_fwd_noalloc(nullptr, dev(1), dev(2), dev(3), devf(4), devf(5), 0.1f, nullptr,
                                nullptr, dev(7), nullptr, nullptr) == KDA_ERR_INVALID_ARGUMENT);
    CHECK(kda_chunk_fwd_noalloc(&s, dev(1), dev(2), dev(3), devf(4), devf(5), 0.1f, nullptr,
                                nullptr, dev(1), nullptr, nullptr) == KDA_ERR_INVALID_ARGUMENT);
}

static void decode_checks() {
    auto dec = [](int N, int H, int d, kda_dtype t, const void *q, const float *g, float *st,
                  void *o) {
        return kda_decode_step(N, H, d, d, t, q, dev(2), dev(3), g, devf(5), 0.1f, st, o, nullptr);
    };
    CHECK(dec(128, 32, 128, KDA_BF16, dev(1), devf(4), devf(8), dev(7)) == KDA_OK);
    CHECK(g_stub.kind == StubRecord::Decode && g_stub.n_pairs == 128 * 32 && g_stub.bf16);
    CHECK(dec(0, 32, 128, KDA_BF16, dev(1), devf(4), devf(8), dev(7)) == KDA_ERR_INVALID_ARGUMENT);
    CHECK(dec(4, 32, 96, KDA_BF16, dev(1), devf(4), devf(8), dev(7)) == KDA_ERR_UNSUPPORTED);
    CHECK(c_decode_with_dtype(3, dev(1), dev(2), dev(3), devf(4), devf(5), devf(8), dev(7)) ==
          KDA_ERR_INVALID_ARGUMENT);
    CHECK(dec(4, 32, 64, KDA_F32, nullptr, devf(4), devf(8), dev(7)) == KDA_ERR_INVALID_ARGUMENT);
    CHECK(dec(4, 32, 64, KDA_F32, misaligned(1), devf(4), devf(8), dev(7)) ==
          KDA_ERR_INVALID_ARGUMENT);
    CHECK(dec(4, 32, 64, KDA_F32, dev(1), devf(4), devf(8), devf(8)) == KDA_ERR_INVALID_ARGUMENT);
    CHECK(dec(65536, 65536, 64, KDA_F32, dev(1), devf(4), devf(8), dev(7)) ==
          KDA_ERR_INVALID_ARGUMENT);
    CHECK(kda_decode_step_scalar_gate(4, 2, 64, 64, KDA_BF16, dev(1), dev(2), dev(3), nullptr,
                                      devf(5), 1.f, devf(8), dev(7), nullptr) == KDA_OK);
    CHECK(g_stub.gate == static_cast<int>(kda::Gate::None));
    kda_inputs_form form = {KDA_GATE_SCALAR, 1, 0, 1, 1e-6f};
    CHECK(kda_decode_step_ex(4, 2, 64, 64, KDA_BF16, &form, dev(1), dev(2), dev(3), devf(4),
                             devf(5), 1.f, devf(8), dev(7), nullptr) == KDA_OK);
    CHECK(g_stub.gate == static_cast<int>(kda::Gate::Scalar) && g_stub.form_flags == 5);
}

static void output_stage_checks() {
    auto post = [](int64_t rows, int dv, kda_dtype t, const void *o, const void *gate, void *out,
                   float eps) {
        return kda_output_rmsnorm_gate(rows, dv, t, o, gate, devf(6), eps, out, nullptr);
    };
    CHECK(post(1000, 128, KDA_BF16, dev(1), dev(2), dev(3), 1e-6f) == KDA_OK);
    CHECK(g_stub.kind == StubRecord::Output && g_stub.rows == 1000);
    CHECK(post(1000, 128, KDA_BF16, dev(1), dev(2), dev(1), 1e-6f) == KDA_OK);   // out == o
    CHECK(post(1000, 128, KDA_BF16, dev(1), dev(2), dev(2), 1e-6f) == KDA_ERR_INVALID_ARGUMENT);
    CHECK(post(1000, 100, KDA_BF16, dev(1), dev(2), dev(3), 1e-6f) == KDA_ERR_UNSUPPORTED);
    CHECK(post(-1, 128, KDA_BF16, dev(1), dev(2), dev(3), 1e-6f) == KDA_ERR_INVALID_ARGUMENT);
    CHECK(post(10, 128, KDA_BF16, dev(1), dev(2), dev(3), 0.f) == KDA_ERR_INVALID_ARGUMENT);
    CHECK(post(10, 128, KDA_F32, misaligned(1), dev(2), dev(3), 1e-6f) == KDA_ERR_INVALID_ARGUMENT);
    CHECK(c_output_with_dtype(5, dev(1), dev(2), devf(6), dev(3)) == KDA_ERR_INVALID_ARGUMENT);
    g_stub = StubRecord();
    CHECK(post(0, 128, KDA_BF16, nullptr, nullptr, nullptr, 1e-6f) == KDA_OK);
    CHECK(g_stub.kind == StubRecord::None);   // nothing enqueued for zero rows
}

static void backward_checks() {
    kda_shape s = bf16_shape(1, 4096, 8);
    s.chunk_size = 16;
    const size_t need = kda_chunk_bwd_workspace_bytes(&s);
    CHECK(need > 0);
    auto bwd = [&](const kda_shape &sh, void *ws, size_t wsb, float *dq) {
        return kda_chunk_bwd(&sh, dev(1), dev(2), dev(3), devf(4), devf(5), 0.1f, nullptr, nullptr,
                             dev(6), nullptr, dq, devf(11), devf(12), devf(13), devf(14), nullptr,
                             ws, wsb, nullptr);
    };
    CHECK(bwd(s, dev(20), need, devf(10)) == KDA_OK && g_stub.kind == StubRecord::Backward);
    CHECK(g_stub.bwd.d == 128 && g_stub.bwd.chunk == 16 && g_stub.bwd.bf16);
    CHECK(bwd(s, dev(20), need - 4, devf(10)) == KDA_ERR_WORKSPACE_TOO_SMALL);
    CHECK(bwd(s, dev(20), need, devf(1)) == KDA_ERR_INVALID_ARGUMENT);   // dq aliases q
    CHECK(bwd(s, nullptr, need, devf(10)) == KDA_ERR_INVALID_ARGUMENT);
    kda_shape u = s;
    u.chunk_size = 64;   // at d = 128 run as 16-token chunks by the backend
    CHECK(bwd(u, dev(20), need, devf(10)) == KDA_OK && g_stub.bwd.chunk == 64);
    u.chunk_size = 48;
    CHECK(bwd(u, dev(20), need, devf(10)) == KDA_ERR_UNSUPPORTED);
    CHECK(c_bwd_with_dtype(&s, 9) == KDA_ERR_UNSUPPORTED);
    CHECK(kda_chunk_bwd(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0.f, nullptr,
                        nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr, nullptr, 0, nullptr) == KDA_ERR_INVALID_ARGUMENT);
}

static void misc_checks() {
    CHECK(kda_abi_version() == KDA_ABI_VERSION);
    // The prefill order: modes 0-3, the previous mode returned, unknown modes refused.
    const int prev = kda_set_prefill_overlap(0);
    CHECK(prev == 1 && kda::prefill_overlap_mode() == 0);
    CHECK(kda_set_prefill_overlap(3) == 0 && kda::prefill_overlap_mode() == 3);
    CHECK(kda_set_prefill_overlap(4) == -1 && kda_set_prefill_overlap(-1) == -1);
    CHECK(kda::prefill_overlap_mode() == 3);
    CHECK(kda_set_prefill_overlap(prev) == 3 && kda::prefill_overlap_mode() == 1);
    for (int st = 0; st <= 6; ++st) CHECK(kda_status_string(static_cast<kda_status>(st)) != nullptr);
    CHECK(std::strcmp(kda_status_string(KDA_ERR_HIP), "KDA_ERR_HIP") == 0);
    // The last-error text is per thread: a failure on another thread leaves this one's alone.
    kda_shape s = bf16_shape();
    CHECK(fwd(s, dev(20), kda_chunk_fwd_workspace_bytes(&s)) == KDA_OK);
    std::string other;
    std::thread t([&] {
        kda_shape b = s;
        b.d_k = 7;
        (void)fwd(b, dev(20), 0);
        other = kda_last_error();
    });
    t.join();
    CHECK(!other.empty() && std::strcmp(kda_last_error(), "") == 0);
}

int main() {
    prefill_checks();
    noalloc_checks();
    decode_checks();
    output_stage_checks();
    backward_checks();
    misc_checks();
    std::printf("abi driver: %d checks passed\n", g_checks);
    return 0;
}
