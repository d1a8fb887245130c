/*
 * abi_c_calls.c -- calls that store an out-of-range integer in a kda_dtype,
 * which C allows (an enum object holds any value of its integer type) and a
 * C caller of the library can do.  Compiled as C so that the C++ driver never
 * forms such an enum value itself (test infrastructure).
 */
#include "kda.h"

kda_status c_fwd_with_dtype(const kda_shape *s, int dtype, const void *q, const void *k,
                            const void *v, const float *g, const float *beta, void *o,
                            void *ws, size_t wsb) {
    kda_shape t = *s;
    t.dtype = dtype;
    return kda_chunk_fwd(&t, q, k, v, g, beta, 1.f, 0, 0, o, 0, ws, wsb, 0);
}

size_t c_workspace_with_dtype(const kda_shape *s, int dtype) {
    kda_shape t = *s;
    t.dtype = dtype;
    return kda_chunk_fwd_workspace_bytes(&t);
}

kda_status c_decode_with_dtype(int dtype, const void *q, const void *k, const void *v,
                               const float *g, const float *beta, float *state, void *o) {
    return kda_decode_step(4, 2, 64, 64, dtype, q, k, v, g, beta, 1.f, state, o, 0);
}

kda_status c_output_with_dtype(int dtype, const void *o, const void *gate, const float *w,
                               void *out) {
    return kda_output_rmsnorm_gate(16, 128, dtype, o, gate, w, 1e-6f, out, 0);
}

kda_status c_bwd_with_dtype(const kda_shape *s, int dtype) {
    kda_shape t = *s;
    t.dtype = dtype;
    return kda_chunk_bwd(&t, 0, 0, 0, 0, 0, 1.f, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0);
}
