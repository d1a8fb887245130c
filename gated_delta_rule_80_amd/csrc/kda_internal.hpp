// kda_internal.hpp -- host-side declarations shared by the C ABI and the
// kernel launchers (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// How the per-token decay a_t = exp(g_t) is given: one log-decay per key
// channel (KDA), one per (token, head) shared by all channels (a scalar gate,
// as in Gated DeltaNet), or none (a_t = 1: DeltaNet).
enum class Gate : int { PerChannel = 0, Scalar = 1, None = 2 };

// Elementwise steps applied to the inputs as the kernels read them.
struct InputForm {
    bool gate_logit = false;   // g holds logits x: log a = log sigmoid(x)
    bool beta_logit = false;   // beta holds logits x: beta = sigmoid(x)
    bool l2norm = false;       // q, k divided by sqrt(sum of squares + eps) per row
    float eps = 0.f;
    // Kernel-argument encoding: bit 0 gate_logit, bit 1 beta_logit, bit 2 l2norm.
    int flags() const { return (gate_logit ? 1 : 0) | (beta_logit ? 2 : 0) | (l2norm ? 4 : 0); }
};
constexpr int kFormGateLogit = 1, kFormBetaLogit = 2, kFormL2Norm = 4;

// ---- decode -----------------------------------------------------------------
bool decode_supported(int dk, int dv);
hipError_t launch_decode(int n_pairs, int dk, int dv, bool bf16, Gate gate, InputForm form,
                         const void *q, const void *k, const void *v, const float *g,
                         const float *beta, float scale, float *state, void *o,
                         hipStream_t stream);

// ---- output stage: RMS norm over d_v, weight, sigmoid gate -------------------------
bool output_stage_supported(int dv);
hipError_t launch_output_rmsnorm_gate(int64_t rows, int dv, bool bf16, const void *o,
                                      const void *gate, const float *weight, float eps,
                                      void *out, hipStream_t stream);

// ---- chunked prefill ----------------------------------------------------------
// Everything a prefill launch needs, already validated by the C ABI layer.
struct ChunkProblem {
    int n_seqs;        // N
    int batch;         // B rows (1 with cu_seqlens)
    int seqlen;        // tokens per row (packed total with cu_seqlens)
    int heads;         // H
    int dk, dv, chunk; // d_k, d_v, C
    bool bf16;         // storage type of q, k, v, o
    const void *q, *k, *v;
    Gate gate;             // layout of g (null when gate == Gate::None)
    InputForm form;        // elementwise steps applied as q, k, g, beta are read
    const float *g, *beta;
    float scale;
    const float *s0;       // may be null (zeros)
    const int32_t *cu;     // may be null (equal rows)
    void *o;
    float *s_final;        // may be null
    void *workspace;
    size_t workspace_bytes;
    hipStream_t stream;
    bool allow_overlap = true;   // false: never the overlapped prefill (creates no stream)
};

// Process-wide choice of the prefill order (kda_set_prefill_overlap): 0 serial,
// 1 overlapped where it applies, 2 overlapped with every record refused, 3
// overlapped with no wait for the first records (2 and 3 test the repair pass).
int prefill_overlap_mode();

// Upper bound on the number of chunks over all sequences: each sequence of
// L tokens has ceil(L / C) <= L / C + 1 chunks.
// One kernel launch holds at most 2^32 - 1 threads; launchers whose grid would
// exceed that return hipErrorInvalidConfiguration before launching.
inline bool launch_fits(int64_t blocks, int64_t threads) {
    return blocks >= 0 && blocks * threads <= (int64_t)0xFFFFFFFF;
}

inline int64_t max_chunks(int64_t total_tokens, int64_t n_seqs, int64_t chunk) {
    return total_tokens / chunk + n_seqs;
}

// The device address of the no-allocation workspace (KDA_NOALLOC_SCRATCH_BYTES)
// on `device`, which must be the current device; looked up on the first call
// per device and kept.
hipError_t noalloc_scratch(int device, void **ptr);

// MFMA path: (128, 128, 64) with bf16 storage.
bool mfma_path_supported(int dk, int dv, int chunk, bool bf16);
size_t mfma_workspace_bytes(int64_t total_tokens, int64_t n_seqs, int heads, int chunk);
hipError_t launch_chunk_fwd_mfma(const ChunkProblem &p);

// fp32 path: d_k == d_v in {16, 32, 64, 128}, C in {16, 32, 64}, fp32 storage.
bool f32_path_supported(int dk, int dv, int chunk, bool bf16);
size_t f32_workspace_bytes(int64_t total_tokens, int64_t n_seqs, int heads, int chunk);
hipError_t launch_chunk_fwd_f32(const ChunkProblem &p);
// fp32 storage at d_k = d_v = 128 (any gate layout and input form):
// 16-token chunks whatever p.chunk says (the chunk size changes only the
// rounding order), the per-chunk factors on fp32 MFMA, then a chain kernel.
bool f32_mfma_applies(int dk, int dv, bool bf16, Gate gate, InputForm form);
size_t f32_mfma_workspace_bytes(int64_t total_tokens, int64_t n_seqs, int heads);
hipError_t launch_chunk_fwd_f32_mfma(const ChunkProblem &p);

// Gradients of the chunked prefill, fp32 storage, d_k = d_v = d.
struct ChunkBwdProblem {
    int n_seqs, seqlen, heads, d, chunk;   // as ChunkProblem (seqlen = row length)
    bool bf16;                             // q, k, v, dout in bf16 (else fp32)
    const void *q, *k, *v;                 // plain inputs
    const float *g, *beta;                 // per-channel log-decays, write strengths
    float scale;
    const float *s0;        // may be null (zeros)
    const int32_t *cu;      // may be null (equal rows)
    const float *dfinal;    // gradient of the final states; may be null (zeros)
    const void *dout;       // gradient of o, dtype of v
    float *dq, *dk, *dv, *dg, *dbeta;
    float *ds0;             // may be null (not written)
    float *work;            // workspace: per chunk states, gradients and factors
    hipStream_t stream;
};
bool bwd_supported(int dk, int dv, int chunk);
size_t bwd_workspace_bytes(int64_t total_tokens, int n_seqs, int heads, int d, int chunk);
hipError_t launch_chunk_bwd(const ChunkBwdProblem &p);

}  // namespace kda
