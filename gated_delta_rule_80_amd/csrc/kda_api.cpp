// kda_api.cpp -- the C ABI of libkda: validation, workspace sizing, dispatch.
//
// Every argument is checked on the host before anything is enqueued; an
// invalid call returns a status and leaves every buffer untouched.  Messages
// for the last failure are kept per thread.
#include "../../include/kda.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "kda_internal.hpp"

namespace {

thread_local char g_last_error[512] = "";

// The prefill order chosen by kda_set_prefill_overlap (1 = overlapped where it applies).
std::atomic<int> g_prefill_overlap{1};

kda_status fail(kda_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

kda_status hip_fail(hipError_t e, const char *what) {
    if (e == hipErrorInvalidConfiguration)
        return fail(KDA_ERR_HIP, "%s: %s (a kernel grid for this problem would exceed 2^32 - 1 "
                    "threads)", what, hipGetErrorString(e));
    return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The integer a caller stored in a kda_dtype.  A C caller may store any int
// there; in C++ reading an enum object whose value lies outside the enum's
// range is undefined, so its bytes are read as an int32_t instead.
int dtype_code(const kda_dtype &d) {
    static_assert(sizeof(kda_dtype) == sizeof(int32_t), "kda_dtype is an int-sized enum");
    int32_t v;
    std::memcpy(&v, &d, sizeof(v));
    return v;
}
bool known_dtype(int dt) { return dt == KDA_F32 || dt == KDA_BF16; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Checks the fields every prefill call needs; on success fills the token count.
kda_status check_shape(const kda_shape *s, int64_t *total_tokens) {
    if (!s) return fail(KDA_ERR_INVALID_ARGUMENT, "shape is NULL");
    if (!known_dtype(dtype_code(s->dtype)))
        return fail(KDA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype_code(s->dtype));
    if (s->batch <= 0 || s->seqlen < 0 || s->num_heads <= 0 || s->d_k <= 0 || s->d_v <= 0 ||
        s->chunk_size <= 0 || s->num_seqs <= 0)
        return fail(KDA_ERR_INVALID_ARGUMENT,
                    "non-positive size (batch %d seqlen %d heads %d d_k %d d_v %d chunk %d "
                    "num_seqs %d)",
                    s->batch, s->seqlen, s->num_heads, s->d_k, s->d_v, s->chunk_size,
                    s->num_seqs);
    const bool bf16 = dtype_code(s->dtype) == KDA_BF16;
    if (!kda::mfma_path_supported(s->d_k, s->d_v, s->chunk_size, bf16) &&
        !kda::f32_path_supported(s->d_k, s->d_v, s->chunk_size, bf16))
        return fail(KDA_ERR_UNSUPPORTED,
                    "no kernel for d_k %d d_v %d chunk %d dtype %s (built: 128/128/64 bf16; "
                    "d in {16,32,64,128} with chunk in {16,32,64} fp32)",
                    s->d_k, s->d_v, s->chunk_size, bf16 ? "bf16" : "f32");
    *total_tokens = (int64_t)s->batch * s->seqlen;
    if (*total_tokens > INT32_MAX / 2)
        return fail(KDA_ERR_INVALID_ARGUMENT, "too many tokens (%lld)",
                    (long long)*total_tokens);
    if ((int64_t)s->num_seqs * s->num_heads > INT32_MAX / 4)
        return fail(KDA_ERR_INVALID_ARGUMENT, "too many sequences x heads");
    return KDA_OK;
}

// The workspace is sized for the packed-sequence chunk bound T/C + N, which
// is never below the equal-rows count B * ceil(T/C); one size fits both.
// For fp32 storage at d = 128 it is what the MFMA factors path needs.
size_t workspace_for(const kda_shape *s, int64_t total) {
    const bool bf16 = dtype_code(s->dtype) == KDA_BF16;
    if (kda::mfma_path_supported(s->d_k, s->d_v, s->chunk_size, bf16))
        return kda::mfma_workspace_bytes(total, s->num_seqs, s->num_heads, s->chunk_size);
    if (kda::f32_mfma_applies(s->d_k, s->d_v, bf16, kda::Gate::PerChannel, kda::InputForm()))
        return kda::f32_mfma_workspace_bytes(total, s->num_seqs, s->num_heads);
    return kda::f32_workspace_bytes(total, s->num_seqs, s->num_heads, s->chunk_size);
}

// Shared body of the two prefill entry points.  With Gate::PerChannel, g is
// [B, T, H, d_k] and required; with Gate::Scalar it is [B, T, H] and NULL
// means no decay (Gate::None).
// Decodes and checks an input-form descriptor (NULL = the plain KDA form).
kda_status read_form(const kda_inputs_form *f, kda::Gate *gate, kda::InputForm *form) {
    *form = kda::InputForm();
    if (!f) return KDA_OK;
    if (f->gate_layout < KDA_GATE_PER_CHANNEL || f->gate_layout > KDA_GATE_NONE)
        return fail(KDA_ERR_INVALID_ARGUMENT, "unknown gate_layout %d", (int)f->gate_layout);
    *gate = static_cast<kda::Gate>(f->gate_layout);
    form->gate_logit = f->gate_is_logit != 0;
    form->beta_logit = f->beta_is_logit != 0;
    form->l2norm = f->l2norm_qk != 0;
    form->eps = f->eps;
    if (form->l2norm && !(std::isfinite(f->eps) && f->eps > 0.f))
        return fail(KDA_ERR_INVALID_ARGUMENT, "l2norm_qk needs a finite eps > 0 (got %g)",
                    (double)f->eps);
    return KDA_OK;
}

// Finds the no-allocation workspace of the current device once every argument
// has been validated; `stream` must belong to that device.
kda_status noalloc_workspace(hipStream_t stream, void **ws) {
    int dev = -1, sdev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "current device");
    if (stream) {
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess) return hip_fail(e, "device of the stream");
        if (sdev != dev)
            return fail(KDA_ERR_INVALID_ARGUMENT,
                        "the stream belongs to device %d but the current device is %d; the "
                        "no-allocation workspace is the current device's", sdev, dev);
    }
    e = kda::noalloc_scratch(dev, ws);
    if (e != hipSuccess) return hip_fail(e, "no-allocation workspace");
    return KDA_OK;
}

// Shared body of the prefill entry points.  With `noalloc` the workspace
// arguments are ignored and the library's own device buffer is used.
kda_status chunk_fwd(kda::Gate gate, kda::InputForm form, const kda_shape *shape, const void *q,
                     const void *k, const void *v, const float *g, const float *beta,
                     float scale, const float *initial_state, const int32_t *cu_seqlens,
                     void *o, float *final_state, void *workspace, size_t workspace_bytes,
                     hipStream_t stream, bool noalloc = false) {
    if (gate == kda::Gate::Scalar && !g) gate = kda::Gate::None;
    if (gate == kda::Gate::None && g)
        return fail(KDA_ERR_INVALID_ARGUMENT, "g must be NULL when there is no gate");
    const bool varlen = cu_seqlens != nullptr;
    int64_t total = 0;
    kda_status st = check_shape(shape, &total);
    if (st != KDA_OK) return st;
    if (varlen && shape->batch != 1)
        return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens needs batch == 1 (got %d)",
                    shape->batch);
    if (!varlen && shape->num_seqs != shape->batch)
        return fail(KDA_ERR_INVALID_ARGUMENT,
                    "without cu_seqlens num_seqs must equal batch (%d vs %d)", shape->num_seqs,
                    shape->batch);
    if (total > 0 && (!q || !k || !v || !beta || !o || (gate == kda::Gate::PerChannel && !g)))
        return fail(KDA_ERR_INVALID_ARGUMENT, "a required tensor pointer is NULL");
    const void *g16 = gate == kda::Gate::PerChannel ? g : nullptr;
    const void *ptrs[] = {q, k, v, g16, o, initial_state, final_state};
    for (const void *p : ptrs)
        if (p && !aligned16(p))
            return fail(KDA_ERR_INVALID_ARGUMENT, "tensor pointer %p is not 16-byte aligned", p);
    if ((beta && !aligned4(beta)) || (cu_seqlens && !aligned4(cu_seqlens)) ||
        (gate == kda::Gate::Scalar && !aligned4(g)))
        return fail(KDA_ERR_INVALID_ARGUMENT,
                    "beta / cu_seqlens / a scalar gate must be 4-byte aligned");
    if (o && (o == q || o == k || o == v || (g && o == (const void *)g) ||
              o == (const void *)beta))
        return fail(KDA_ERR_INVALID_ARGUMENT, "o must not alias an input");
    // fp32 at d = 128 takes the MFMA factors path (any gate layout and input
    // form).  Without allocation it does so while its workspace fits
    // the library's buffer; beyond that the other fp32 kernel, which needs no
    // workspace, keeps every fp32 size available.
    const bool bf16 = dtype_code(shape->dtype) == KDA_BF16;
    bool mfma_f32 = kda::f32_mfma_applies(shape->d_k, shape->d_v, bf16, gate, form);
    size_t need = (bf16 || mfma_f32) ? workspace_for(shape, total) : 0;
    if (noalloc && mfma_f32 && need > KDA_NOALLOC_SCRATCH_BYTES) {
        mfma_f32 = false;
        need = 0;
    }
    if (noalloc) {
        if (need > KDA_NOALLOC_SCRATCH_BYTES)
            return fail(KDA_ERR_WORKSPACE_TOO_SMALL,
                        "this problem needs %zu bytes of workspace; kda_chunk_fwd_noalloc has %zu "
                        "(KDA_NOALLOC_SCRATCH_BYTES): call kda_chunk_fwd with a workspace instead",
                        need, (size_t)KDA_NOALLOC_SCRATCH_BYTES);
        workspace = nullptr;
        workspace_bytes = KDA_NOALLOC_SCRATCH_BYTES;
        if (need > 0) {
            st = noalloc_workspace(stream, &workspace);
            if (st != KDA_OK) return st;
        }
    }
    if (need > 0 && !workspace)
        return fail(KDA_ERR_INVALID_ARGUMENT, "workspace is NULL (%zu bytes needed)", need);
    if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return fail(KDA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    if (workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed",
                    workspace_bytes, need);

    kda::ChunkProblem p;
    p.n_seqs = shape->num_seqs;
    p.batch = shape->batch;
    p.seqlen = shape->seqlen;
    p.heads = shape->num_heads;
    p.dk = shape->d_k;
    p.dv = shape->d_v;
    p.chunk = shape->chunk_size;
    p.bf16 = dtype_code(shape->dtype) == KDA_BF16;
    p.q = q;
    p.k = k;
    p.v = v;
    p.gate = gate;
    p.form = form;
    p.g = gate == kda::Gate::None ? nullptr : g;
    p.beta = beta;
    p.scale = scale;
    p.s0 = initial_state;
    p.cu = cu_seqlens;
    p.o = o;
    p.s_final = final_state;
    p.workspace = workspace;
    p.workspace_bytes = workspace_bytes;
    p.stream = stream;
    p.allow_overlap = !noalloc;

    hipError_t e = kda::mfma_path_supported(p.dk, p.dv, p.chunk, p.bf16)
                       ? kda::launch_chunk_fwd_mfma(p)
                       : mfma_f32 ? kda::launch_chunk_fwd_f32_mfma(p)
                                  : kda::launch_chunk_fwd_f32(p);
    if (e != hipSuccess) return hip_fail(e, "chunk prefill launch");
    return KDA_OK;
}

// Shared body of the two decode entry points (gate layouts as for chunk_fwd,
// per pair instead of per token).
kda_status decode_step(kda::Gate gate, kda::InputForm form, int32_t num_sessions,
                       int32_t num_heads, int32_t d_k, int32_t d_v, int dtype,
                       const void *q, const void *k, const void *v, const float *g,
                       const float *beta, float scale, float *state_inout, void *o,
                       hipStream_t stream) {
    if (gate == kda::Gate::Scalar && !g) gate = kda::Gate::None;
    if (gate == kda::Gate::None && g)
        return fail(KDA_ERR_INVALID_ARGUMENT, "g must be NULL when there is no gate");
    if (!known_dtype(dtype))
        return fail(KDA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
    if (num_sessions <= 0 || num_heads <= 0 || d_k <= 0 || d_v <= 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "non-positive size (sessions %d heads %d d_k %d "
                    "d_v %d)", num_sessions, num_heads, d_k, d_v);
    if (!kda::decode_supported(d_k, d_v))
        return fail(KDA_ERR_UNSUPPORTED, "no decode kernel for d_k %d d_v %d (built: d_k == "
                    "d_v in {16, 32, 64, 128})", d_k, d_v);
    const int64_t pairs = (int64_t)num_sessions * num_heads;
    if (pairs > INT32_MAX) return fail(KDA_ERR_INVALID_ARGUMENT, "too many pairs");
    if (!q || !k || !v || !beta || !state_inout || !o || (gate == kda::Gate::PerChannel && !g))
        return fail(KDA_ERR_INVALID_ARGUMENT, "a required tensor pointer is NULL");
    const void *g16 = gate == kda::Gate::PerChannel ? g : q;
    const void *ptrs[] = {q, k, v, g16, state_inout, o};
    for (const void *p : ptrs)
        if (!aligned16(p))
            return fail(KDA_ERR_INVALID_ARGUMENT, "tensor pointer %p is not 16-byte aligned", p);
    if (!aligned4(beta) || (gate == kda::Gate::Scalar && !aligned4(g)))
        return fail(KDA_ERR_INVALID_ARGUMENT, "beta / a scalar gate must be 4-byte aligned");
    if (o == (void *)state_inout)
        return fail(KDA_ERR_INVALID_ARGUMENT, "o must not alias state_inout");
    hipError_t e = kda::launch_decode((int)pairs, d_k, d_v, dtype == KDA_BF16, gate, form, q, k, v,
                                      gate == kda::Gate::None ? nullptr : g, beta, scale,
                                      state_inout, o, stream);
    if (e != hipSuccess) return hip_fail(e, "decode step launch");
    return KDA_OK;
}

}  // namespace

int kda::prefill_overlap_mode() { return g_prefill_overlap.load(std::memory_order_relaxed); }

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

int kda_set_prefill_overlap(int mode) {
    if (mode < 0 || mode > 3) return -1;
    return g_prefill_overlap.exchange(mode);
}

const char *kda_status_string(kda_status status) {
    switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "KDA_ERR_WORKSPACE_TOO_SMALL";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
    }
    return "KDA_ERR_UNKNOWN";
}

const char *kda_last_error(void) { return g_last_error; }

size_t kda_chunk_fwd_workspace_bytes(const kda_shape *shape) {
    int64_t total = 0;
    char saved[sizeof(g_last_error)];
    memcpy(saved, g_last_error, sizeof(saved));
    const kda_status st = check_shape(shape, &total);
    memcpy(g_last_error, saved, sizeof(saved));
    if (st != KDA_OK) return 0;
    return workspace_for(shape, total);
}

kda_status kda_chunk_fwd(const kda_shape *shape, const void *q, const void *k, const void *v,
                         const float *g_log_decay, const float *beta, float scale,
                         const float *initial_state, const int32_t *cu_seqlens, void *o,
                         float *final_state, void *workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    g_last_error[0] = '\0';
    return chunk_fwd(kda::Gate::PerChannel, kda::InputForm(), shape, q, k, v, g_log_decay, beta,
                     scale, initial_state, cu_seqlens, o, final_state, workspace,
                     workspace_bytes, stream);
}

kda_status kda_chunk_fwd_noalloc(const kda_shape *shape, const void *q, const void *k,
                                 const void *v, const float *g_log_decay, const float *beta,
                                 float scale, const float *initial_state,
                                 const int32_t *cu_seqlens, void *o, float *final_state,
                                 hipStream_t stream) {
    g_last_error[0] = '\0';
    return chunk_fwd(kda::Gate::PerChannel, kda::InputForm(), shape, q, k, v, g_log_decay, beta,
                     scale, initial_state, cu_seqlens, o, final_state, nullptr, 0, stream,
                     /*noalloc=*/true);
}

kda_status kda_chunk_fwd_scalar_gate(const kda_shape *shape, const void *q, const void *k,
                                     const void *v, const float *g_log_decay, const float *beta,
                                     float scale, const float *initial_state,
                                     const int32_t *cu_seqlens, void *o, float *final_state,
                                     void *workspace, size_t workspace_bytes, hipStream_t stream) {
    g_last_error[0] = '\0';
    return chunk_fwd(kda::Gate::Scalar, kda::InputForm(), shape, q, k, v, g_log_decay, beta,
                     scale, initial_state, cu_seqlens, o, final_state, workspace,
                     workspace_bytes, stream);
}

kda_status kda_chunk_fwd_ex(const kda_shape *shape, const kda_inputs_form *form, const void *q,
                            const void *k, const void *v, const float *g_log_decay,
                            const float *beta, float scale, const float *initial_state,
                            const int32_t *cu_seqlens, void *o, float *final_state,
                            void *workspace, size_t workspace_bytes, hipStream_t stream) {
    g_last_error[0] = '\0';
    kda::Gate gate = kda::Gate::PerChannel;
    kda::InputForm f;
    const kda_status st = read_form(form, &gate, &f);
    if (st != KDA_OK) return st;
    if (gate == kda::Gate::Scalar && !g_log_decay)
        return fail(KDA_ERR_INVALID_ARGUMENT, "KDA_GATE_SCALAR needs g (use KDA_GATE_NONE)");
    return chunk_fwd(gate, f, shape, q, k, v, g_log_decay, beta, scale, initial_state,
                     cu_seqlens, o, final_state, workspace, workspace_bytes, stream);
}

kda_status kda_decode_step(int32_t num_sessions, int32_t num_heads, int32_t d_k, int32_t d_v,
                           kda_dtype dtype, const void *q, const void *k, const void *v,
                           const float *g, const float *beta, float scale, float *state_inout,
                           void *o, hipStream_t stream) {
    g_last_error[0] = '\0';
    return decode_step(kda::Gate::PerChannel, kda::InputForm(), num_sessions, num_heads, d_k, d_v,
                       dtype_code(dtype), q, k, v, g, beta, scale, state_inout, o, stream);
}

kda_status kda_decode_step_scalar_gate(int32_t num_sessions, int32_t num_heads, int32_t d_k,
                                       int32_t d_v, kda_dtype dtype, const void *q,
                                       const void *k, const void *v, const float *g,
                                       const float *beta, float scale, float *state_inout,
                                       void *o, hipStream_t stream) {
    g_last_error[0] = '\0';
    return decode_step(kda::Gate::Scalar, kda::InputForm(), num_sessions, num_heads, d_k, d_v,
                       dtype_code(dtype), q, k, v, g, beta, scale, state_inout, o, stream);
}

kda_status kda_decode_step_ex(int32_t num_sessions, int32_t num_heads, int32_t d_k, int32_t d_v,
                              kda_dtype dtype, const kda_inputs_form *form, const void *q,
                              const void *k, const void *v, const float *g, const float *beta,
                              float scale, float *state_inout, void *o, hipStream_t stream) {
    g_last_error[0] = '\0';
    kda::Gate gate = kda::Gate::PerChannel;
    kda::InputForm f;
    const kda_status st = read_form(form, &gate, &f);
    if (st != KDA_OK) return st;
    if (gate == kda::Gate::Scalar && !g)
        return fail(KDA_ERR_INVALID_ARGUMENT, "KDA_GATE_SCALAR needs g (use KDA_GATE_NONE)");
    return decode_step(gate, f, num_sessions, num_heads, d_k, d_v, dtype_code(dtype), q, k, v, g,
                       beta, scale,
                       state_inout, o, stream);
}

kda_status kda_output_rmsnorm_gate(int64_t rows, int32_t d_v, kda_dtype dtype, const void *o,
                                   const void *gate, const float *weight, float eps, void *out,
                                   hipStream_t stream) {
    g_last_error[0] = '\0';
    const int dt = dtype_code(dtype);
    if (!known_dtype(dt)) return fail(KDA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dt);
    if (rows < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "negative rows (%lld)", (long long)rows);
    if (!kda::output_stage_supported(d_v))
        return fail(KDA_ERR_UNSUPPORTED, "no output-stage kernel for d_v %d (built: 16, 32, 64, "
                    "128, 256)", d_v);
    if (!(std::isfinite(eps) && eps > 0.f))
        return fail(KDA_ERR_INVALID_ARGUMENT, "eps must be finite and > 0 (got %g)", (double)eps);
    if (rows == 0) return KDA_OK;
    if ((rows + 255) / 256 * 4 > (int64_t)INT32_MAX)
        return fail(KDA_ERR_INVALID_ARGUMENT, "too many rows (%lld)", (long long)rows);
    if (!o || !gate || !weight || !out)
        return fail(KDA_ERR_INVALID_ARGUMENT, "a required tensor pointer is NULL");
    const uintptr_t mask = dt == KDA_F32 ? 15u : 7u;
    if ((reinterpret_cast<uintptr_t>(o) & mask) || (reinterpret_cast<uintptr_t>(gate) & mask) ||
        (reinterpret_cast<uintptr_t>(out) & mask) || !aligned16(weight))
        return fail(KDA_ERR_INVALID_ARGUMENT, "o / gate / out / weight are misaligned");
    if (out == gate) return fail(KDA_ERR_INVALID_ARGUMENT, "out must not alias gate");
    hipError_t e = kda::launch_output_rmsnorm_gate(rows, d_v, dt == KDA_BF16, o, gate, weight,
                                                   eps, out, stream);
    if (e != hipSuccess) return hip_fail(e, "output stage launch");
    return KDA_OK;
}

size_t kda_chunk_bwd_workspace_bytes(const kda_shape *shape) {
    if (!shape || shape->batch <= 0 || shape->seqlen < 0 || shape->num_heads <= 0 ||
        shape->d_k <= 0 || shape->chunk_size <= 0 || shape->num_seqs <= 0 ||
        !kda::bwd_supported(shape->d_k, shape->d_v, shape->chunk_size))
        return 0;
    const int64_t total = (int64_t)shape->batch * shape->seqlen;
    return kda::bwd_workspace_bytes(total, shape->num_seqs, shape->num_heads, shape->d_k,
                                    shape->chunk_size);
}

kda_status kda_chunk_bwd(const kda_shape *shape, const void *q, const void *k, const void *v,
                         const float *g_log_decay, const float *beta, float scale,
                         const float *initial_state, const int32_t *cu_seqlens, const void *d_o,
                         const float *d_final_state, float *dq, float *dk, float *dv, float *dg,
                         float *dbeta, float *d_initial_state, void *workspace,
                         size_t workspace_bytes, hipStream_t stream) {
    g_last_error[0] = '\0';
    if (!shape) return fail(KDA_ERR_INVALID_ARGUMENT, "shape is NULL");
    if (!known_dtype(dtype_code(shape->dtype)))
        return fail(KDA_ERR_UNSUPPORTED, "unknown dtype %d", dtype_code(shape->dtype));
    if (shape->batch <= 0 || shape->seqlen < 0 || shape->num_heads <= 0 || shape->d_k <= 0 ||
        shape->d_v <= 0 || shape->chunk_size <= 0 || shape->num_seqs <= 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "non-positive size");
    if (!kda::bwd_supported(shape->d_k, shape->d_v, shape->chunk_size))
        return fail(KDA_ERR_UNSUPPORTED,
                    "no backward kernel for d_k %d d_v %d chunk %d (built: d_k = d_v = 16 with "
                    "chunk 16/32/64, 32 or 64 with chunk 16/32, 128 with chunk 16)",
                    shape->d_k, shape->d_v, shape->chunk_size);
    const int64_t total = (int64_t)shape->batch * shape->seqlen;
    if (total > INT32_MAX / 2) return fail(KDA_ERR_INVALID_ARGUMENT, "too many tokens");
    const bool varlen = cu_seqlens != nullptr;
    if (varlen && shape->batch != 1)
        return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens needs batch == 1 (got %d)",
                    shape->batch);
    if (!varlen && shape->num_seqs != shape->batch)
        return fail(KDA_ERR_INVALID_ARGUMENT,
                    "without cu_seqlens num_seqs must equal batch (%d vs %d)", shape->num_seqs,
                    shape->batch);
    if (total > 0 && (!q || !k || !v || !g_log_decay || !beta || !d_o || !dq || !dk || !dv ||
                      !dg || !dbeta))
        return fail(KDA_ERR_INVALID_ARGUMENT, "a required tensor pointer is NULL");
    const void *p16[] = {q, k, v, g_log_decay, d_o, dq, dk, dv, dg, initial_state,
                         d_final_state, d_initial_state};
    for (const void *p : p16)
        if (p && !aligned16(p))
            return fail(KDA_ERR_INVALID_ARGUMENT, "tensor pointer %p is not 16-byte aligned", p);
    if ((beta && !aligned4(beta)) || (dbeta && !aligned4(dbeta)) ||
        (cu_seqlens && !aligned4(cu_seqlens)))
        return fail(KDA_ERR_INVALID_ARGUMENT, "beta / dbeta / cu_seqlens must be 4-byte aligned");
    const void *ins[] = {q, k, v, g_log_decay, beta, d_o, initial_state, d_final_state};
    const void *outs[] = {dq, dk, dv, dg, dbeta, d_initial_state};
    for (const void *o : outs)
        for (const void *in : ins)
            if (o && o == in)
                return fail(KDA_ERR_INVALID_ARGUMENT, "gradient outputs must not alias inputs");
    const size_t need = kda_chunk_bwd_workspace_bytes(shape);
    if (!workspace) return fail(KDA_ERR_INVALID_ARGUMENT, "workspace is NULL (%zu bytes needed)", need);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(KDA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    if (workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed",
                    workspace_bytes, need);
    kda::ChunkBwdProblem p;
    p.n_seqs = shape->num_seqs;
    p.seqlen = shape->seqlen;
    p.heads = shape->num_heads;
    p.d = shape->d_k;
    p.chunk = shape->chunk_size;
    p.bf16 = dtype_code(shape->dtype) == KDA_BF16;
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g_log_decay;
    p.beta = beta;
    p.scale = scale;
    p.s0 = initial_state;
    p.cu = cu_seqlens;
    p.dfinal = d_final_state;
    p.dout = d_o;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.dg = dg;
    p.dbeta = dbeta;
    p.ds0 = d_initial_state;
    p.work = static_cast<float *>(workspace);
    p.stream = stream;
    hipError_t e = kda::launch_chunk_bwd(p);
    if (e != hipSuccess) return hip_fail(e, "chunk backward launch");
    return KDA_OK;
}

}  // extern "C"
