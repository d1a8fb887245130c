/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention forward library.
 *
 * The operator, per head, with key-by-value state S (d_k x d_v, row r = key
 * channel r), per-token log-decay g_t = log a_t (<= 0), write strength beta_t
 * and query scale s:
 *
 *   S_bar = Diag(exp(g_t)) S_{t-1}                 (retain)
 *   S_t   = S_bar + beta_t k_t (v_t - S_bar^T k_t)^T (predict, correct)
 *   o_t   = S_t^T (s q_t)                          (read the updated state)
 *
 * Defined in "Understanding Kimi Delta Attention" (A. Flores), section
 * "Learning what to forget", box "KDA: retain, predict, correct"; the query
 * scale d_k^{-1/2} in the read is from "Demystifying Kimi Delta Attention"
 * (J. Dborin), section "The Complexity of Modern Linear Attention".
 *
 * kda_chunk_fwd evaluates a whole sequence chunk by chunk in the WY / UT form
 * of "Understanding Kimi Delta Attention", sections "The triangular system"
 * and "Putting the chunks together" (one triangular system per chunk, one
 * state crossing each chunk boundary).  kda_decode_step applies the recurrence
 * once to each (session, head) pair.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller, dense,
 *     row-major and contiguous in the layouts stated below; the library never
 *     allocates, frees or retains them.  They must stay valid until the work
 *     enqueued on `stream` has completed.
 *   - `stream` is a hipStream_t, declared here by its underlying type
 *     `struct ihipStream_t *` so that this header needs no HIP header
 *     (NULL = the null stream).  All work is enqueued on it in order; calls
 *     return without synchronising.  (The overlapped prefill of
 *     kda_chunk_fwd also runs one kernel on a side stream of the library's,
 *     which waits for `stream` and which `stream` waits for, so the call
 *     still starts and completes in order on `stream`.)
 *   - Arguments are validated on the host before anything is enqueued.  On any
 *     error nothing is enqueued, no output is touched, and a status other than
 *     KDA_OK is returned; kda_last_error() then describes the cause (the text
 *     is thread-local and valid until the next call on the same thread).
 *   - A problem whose kernel grid would exceed 2^32 - 1 threads in one launch
 *     returns KDA_ERR_HIP (hipErrorInvalidConfiguration) before anything is
 *     enqueued.  The prefill's chunk chain is launched in batches of (sequence,
 *     head) pairs, so it never reaches that limit.  Any other KDA_ERR_HIP may
 *     leave kernels of the same call enqueued before the one that failed.
 *   - Device-side faults, if any, surface at the caller's next
 *     synchronisation, as for any HIP kernel.
 *   - No C++ exception crosses this boundary.  The library's only global
 *     state is the prefill order (kda_set_prefill_overlap) and, per device,
 *     the side stream and two events of the overlapped prefill, created by
 *     its first use on the device and kept until the process ends;
 *     concurrent calls on different streams are safe.
 *   - Values are not checked: NaN / Inf in, NaN / Inf out.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP stream type: hipStream_t is a pointer to this (opaque) struct. */
struct ihipStream_t;

#define KDA_ABI_VERSION 6

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1,    /* NULL / misaligned pointer, bad size   */
    KDA_ERR_UNSUPPORTED = 2,         /* (d_k, d_v, chunk, dtype) not built    */
    KDA_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below the query        */
    KDA_ERR_HIP = 4                  /* a HIP launch or runtime call failed   */
} kda_status;

/* Storage type of q, k, v and o.  g, beta and every state are always fp32. */
typedef enum kda_dtype { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/*
 * Problem description for kda_chunk_fwd.
 *   batch      rows B of the q/k/v/g/beta/o tensors (must be 1 with cu_seqlens)
 *   seqlen     tokens per row T; with cu_seqlens, the packed total cu_seqlens[N]
 *   num_heads  H
 *   d_k, d_v   key and value widths
 *   chunk_size C, tokens per chunk
 *   num_seqs   N: number of sequences (== batch without cu_seqlens)
 *   dtype      storage type of q, k, v, o
 * Built combinations (d_k, d_v, C, dtype):
 *   (128, 128, 64, KDA_BF16)  MFMA path (fp16 operands, fp32 accumulation)
 *   (d, d, C, KDA_F32) with d in {16, 32, 64, 128}, C in {16, 32, 64}: fp32
 *                             path (fp32 arithmetic throughout).  At d = 128
 *                             (any gate layout and input form) it
 *                             forms the chunk factors and carries the state
 *                             on fp32 MFMA in 16-token chunks whatever C is
 *                             (C changes only the rounding order).
 * Everything else returns KDA_ERR_UNSUPPORTED.
 */
typedef struct kda_shape {
    int32_t batch;
    int32_t seqlen;
    int32_t num_heads;
    int32_t d_k;
    int32_t d_v;
    int32_t chunk_size;
    int32_t num_seqs;
    kda_dtype dtype;
} kda_shape;

/*
 * How the inputs of the *_ex entry points are given.  A KDA layer produces q,
 * k, the decay and beta from learned projections; normalising q and k and
 * squashing the decay and write-strength logits are the last elementwise steps
 * before the recurrence ("Kimi Delta Attention: How It Works, Step by Step",
 * question 16; "Kimi Delta Attention: a half-life per channel", section
 * "Promote the scalar to a diagonal", a_t = sigmoid(x_t W_a)).  The *_ex entry
 * points apply them inside the kernels as the inputs are read, so no separate
 * pass over q, k, g or beta is needed.
 *   gate_layout    KDA_GATE_PER_CHANNEL: g is [.., d_k] (KDA);
 *                  KDA_GATE_SCALAR: g is [..] (one per token and head);
 *                  KDA_GATE_NONE: no decay, g must be NULL.
 *   gate_is_logit  0: g holds log a (<= 0).  1: g holds logits x and
 *                  log a = log sigmoid(x), evaluated as min(x, 0) - log1p(e^-|x|).
 *   beta_is_logit  0: beta holds the write strength.  1: beta = sigmoid(x).
 *   l2norm_qk      1: q and k are each divided by sqrt(sum of squares + eps)
 *                  over their d_k channels, per (token, head).
 *   eps            the epsilon of l2norm_qk (for example 1e-6); must be > 0
 *                  when l2norm_qk is set.
 * {KDA_GATE_PER_CHANNEL, 0, 0, 0, 0} is exactly kda_chunk_fwd / kda_decode_step.
 */
typedef enum kda_gate_layout {
    KDA_GATE_PER_CHANNEL = 0,
    KDA_GATE_SCALAR = 1,
    KDA_GATE_NONE = 2
} kda_gate_layout;

typedef struct kda_inputs_form {
    int32_t gate_layout;
    int32_t gate_is_logit;
    int32_t beta_is_logit;
    int32_t l2norm_qk;
    float eps;
} kda_inputs_form;

/* ABI version of the loaded library (KDA_ABI_VERSION it was built with). */
int kda_abi_version(void);

/*
 * Chooses, for the whole process, the order in which kda_chunk_fwd (and the
 * scalar-gate and _ex prefills) run their two bf16 kernels, and returns the
 * previous choice, or -1 for an unknown mode (nothing changes then).
 *   1  overlapped where it applies (the default; see kda_chunk_fwd)
 *   0  always one after the other
 *   2  overlapped, but the chain accepts no chunk's factors and runs on
 *      whatever the workspace holds, so every overlapped call ends with the
 *      repair pass: for testing that pass.
 *   3  overlapped, but a chain whose first chunks' factors are not already
 *      published gives up at once (as it does after 250 us in mode 1, when
 *      the intra-chunk kernel is queued behind it), and the repair pass runs:
 *      for testing that path.
 * Calls already enqueued keep the order they were enqueued with.
 */
int kda_set_prefill_overlap(int mode);

/* Static text for a status code. */
const char *kda_status_string(kda_status status);

/* Detail of the last failed call on this thread ("" if none). */
const char *kda_last_error(void);

/*
 * Bytes of device workspace kda_chunk_fwd needs for `shape`, or 0 if the
 * shape is invalid or unsupported (kda_chunk_fwd then reports why).  The
 * workspace holds the per-chunk WY factors between the intra-chunk and the
 * inter-chunk kernels, the chunk table of packed sequences, and one flag per
 * (chunk, head) for the overlapped order.  With fp32 storage it is 0 below
 * d = 128; at d = 128 it holds the fp32 chunk factors (27.5 KB per 16-token
 * chunk slot and head).
 */
size_t kda_chunk_fwd_workspace_bytes(const kda_shape *shape);

/*
 * Chunkwise KDA prefill ("Understanding Kimi Delta Attention", sections "The
 * triangular system" and "Putting the chunks together").
 *
 *   q, k          [B, T, H, d_k]  dtype          (q, k not normalised here)
 *   v             [B, T, H, d_v]  dtype
 *   g_log_decay   [B, T, H, d_k]  fp32: per-token log a_t (<= 0), NOT a
 *                 cumulative sum; the kernel accumulates it per chunk.
 *   beta          [B, T, H]       fp32
 *   scale         query scale s, usually d_k^{-1/2}
 *   initial_state [N, H, d_k, d_v] fp32, or NULL for zeros
 *   cu_seqlens    [N+1] int32 on the device, or NULL.  With it, B must be 1,
 *                 T = cu_seqlens[N] and sequence n owns packed tokens
 *                 [cu_seqlens[n], cu_seqlens[n+1]).  It must start at 0 and be
 *                 non-decreasing (not checked on the device).  Zero-length
 *                 sequences are allowed: their final state is their initial
 *                 state.  Without it, row b is sequence b.
 *   o             [B, T, H, d_v]  dtype (written for every token); must not
 *                 alias any input.
 *   final_state   [N, H, d_k, d_v] fp32, or NULL (not written).  May equal
 *                 initial_state (in-place continuation).
 *   workspace     device buffer of at least
 *                 kda_chunk_fwd_workspace_bytes(shape) bytes, 256-byte aligned.
 * Each sequence is cut into chunks of C tokens from its first token; the last
 * chunk may be shorter.  Chunks never straddle sequences.
 * Decay range: any cumulative decay and any per-token log-decay, -inf
 * included.  The MFMA path (bf16 storage) splits each 64-token chunk into
 * 16-token sub-chunks ("Kimi Delta Attention: a half-life per channel",
 * section "What changes in the kernel") and floors each per-token log-decay at
 * -10: a channel told to keep less than e^-10 (4.5e-5) of its state over one
 * token keeps e^-10 of it, which moves o and the state by at most that
 * fraction of the forgotten state (far inside the bf16 tolerance) and keeps
 * every decay-scaled operand inside the fp32 / bf16 range.  The fp32 path
 * uses the exact factors and takes any finite value.  Keys
 * and queries are expected L2-normalised (|k|, |q| <= 1) and |v| well below
 * the fp16 range, as the layer that calls this operator produces them.
 * Pointers to q, k, v, o, g and the states must be 16-byte aligned; beta and
 * cu_seqlens 4-byte aligned.
 * Order of the two kernels (bf16 storage).  The intra-chunk kernel computes
 * every chunk's factors independently and the chain kernel carries the state
 * across chunks.  By default the two run side by side for equal rows (no
 * cu_seqlens) of at least 128 chunks (8192 tokens at C = 64) with H a
 * multiple of 8, at most n_cu / 8 (sequence, head) pairs (32 on MI355X), an
 * initial state that final_state does not overwrite, and (through
 * kda_chunk_fwd_ex) neither the logit gate nor the in-kernel L2 norms, whose
 * intra-chunk work is as long as the chain.  The chain then starts at once
 * and takes each chunk's factors as soon as they are published, through the
 * L2 of the XCD (accelerator die) on which both kernels place the head.
 * Should the chain fail to accept a chunk's factors (they came through
 * another XCD, or did not arrive within about 10 ms plus 20 us per chunk), a
 * repair pass reruns the chain after both kernels have ended.  A chain that
 * finds its first chunks' factors missing for 250 us gives up at once: the
 * intra-chunk kernel is then queued behind it, as when the library's side
 * stream shares a hardware queue with `stream`.  Every other call, every call
 * under stream capture and every call whose `stream` belongs to another
 * device than the current one runs the kernels one after the other.  Both
 * orders give the same bits.  An overlapped call leaves the first 32-bit word
 * of the workspace nonzero if it needed its repair pass and 0 if not (a
 * diagnostic, valid once the call has completed); a call run in the serial
 * order does not write it.
 */
kda_status kda_chunk_fwd(const kda_shape *shape, const void *q, const void *k,
                         const void *v, const float *g_log_decay,
                         const float *beta, float scale,
                         const float *initial_state, const int32_t *cu_seqlens,
                         void *o, float *final_state, void *workspace,
                         size_t workspace_bytes, struct ihipStream_t *stream);

/*
 * Size of the device buffer behind kda_chunk_fwd_noalloc (256 MiB per device).
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/*
 * kda_chunk_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, hosts that forbid hipMalloc.  Same
 * arguments, semantics and results (bit for bit) as kda_chunk_fwd, without the
 * workspace: the workspace is a buffer of KDA_NOALLOC_SCRATCH_BYTES that the
 * library holds in device memory from the moment it is loaded onto a device
 * until the process ends (each device has its own).  Nothing is allocated or
 * freed by this call.
 *   - Problems whose kda_chunk_fwd_workspace_bytes exceeds
 *     KDA_NOALLOC_SCRATCH_BYTES return KDA_ERR_WORKSPACE_TOO_SMALL before
 *     anything is enqueued; at d_k = d_v = 128 with bf16 storage the buffer
 *     holds about 4,300 (chunk, head) records (for example H = 32 heads over
 *     about 8,600 tokens).  With fp32 storage at d = 128 a problem whose
 *     factors fit (about 9,500 16-token chunk slots x heads) takes the same
 *     path as kda_chunk_fwd; a larger one takes the fp32 kernel that needs no
 *     workspace, whose results agree with kda_chunk_fwd's to within the fp32
 *     tolerance rather than bit for bit.  Below d = 128 the fp32 path needs no
 *     workspace.
 *   - The buffer belongs to the CURRENT device; `stream` must be a stream of
 *     that device (NULL = its null stream), else KDA_ERR_INVALID_ARGUMENT.
 *   - All calls on one device share the buffer, and it keeps the last call's
 *     contents.  Calls that may overlap on one device (different streams,
 *     different host threads) race on it; serialise them, for example on one
 *     stream.  Each call writes every part of the buffer it later reads, so
 *     nothing needs clearing between calls.
 *   - The two kernels always run one after the other (no side stream).
 */
kda_status kda_chunk_fwd_noalloc(const kda_shape *shape, const void *q, const void *k,
                                 const void *v, const float *g_log_decay, const float *beta,
                                 float scale, const float *initial_state,
                                 const int32_t *cu_seqlens, void *o, float *final_state,
                                 struct ihipStream_t *stream);

/*
 * The same prefill with a scalar gate: one log-decay per (token, head), shared
 * by every key channel of the head, i.e. Diag(a_t) = a_t I.  This is the
 * coarser gate that "Understanding Kimi Delta Attention", section "Learning
 * what to forget", contrasts with KDA's per-channel one (the gate of Gated
 * DeltaNet); with no gate at all (a_t = 1) the operator is the plain delta
 * rule of the sections before it (DeltaNet).
 *
 *   g_log_decay   [B, T, H] fp32 per-token log a_t (<= 0), not cumulative, or
 *                 NULL for a_t = 1.  4-byte aligned.
 * Every other argument, the workspace (kda_chunk_fwd_workspace_bytes, same
 * shape), the built combinations, the decay range and the alignment rules are
 * those of kda_chunk_fwd.  With bf16 storage the intra-chunk work has a kernel
 * of its own: with one decay per token, the pairwise factor e^{G_i - G_j}
 * leaves the sum over key channels, so K K^T and (s Q) K^T are plain MFMA
 * products and the decay is a chunk x chunk mask (every factor <= 1) applied
 * to them ("Kimi Delta Attention: a half-life per channel", section "What
 * changes in the kernel"); the chunk chain is shared.  Its results agree with
 * kda_chunk_fwd fed g on every channel to within the bf16 tolerance, not bit
 * for bit.  With fp32 storage one path serves both gate layouts and the
 * results are bit for bit those of kda_chunk_fwd with g repeated.
 */
kda_status kda_chunk_fwd_scalar_gate(const kda_shape *shape, const void *q,
                                     const void *k, const void *v,
                                     const float *g_log_decay,
                                     const float *beta, float scale,
                                     const float *initial_state,
                                     const int32_t *cu_seqlens, void *o,
                                     float *final_state, void *workspace,
                                     size_t workspace_bytes, struct ihipStream_t *stream);

/*
 * One recurrent decode step for num_sessions x num_heads independent pairs
 * ("Understanding Kimi Delta Attention", box "KDA: retain, predict, correct";
 * the fixed-size state is what a decode step reads and rewrites).
 *
 *   q, k          [N, H, d_k]  dtype      v, o  [N, H, d_v]  dtype
 *   g             [N, H, d_k]  fp32 log a (<= 0)
 *   beta          [N, H]       fp32
 *   state_inout   [N, H, d_k, d_v] fp32, read and overwritten in place with
 *                 the state after this token; must not alias o.
 * Built combinations (d_k, d_v): (128, 128) for KDA_BF16 and KDA_F32, and
 * (d, d) with d in {16, 32, 64} for both dtypes.
 * Pointers must be 16-byte aligned, except beta (4-byte aligned).
 */
kda_status kda_decode_step(int32_t num_sessions, int32_t num_heads, int32_t d_k,
                           int32_t d_v, kda_dtype dtype, const void *q,
                           const void *k, const void *v, const float *g,
                           const float *beta, float scale, float *state_inout,
                           void *o, struct ihipStream_t *stream);

/*
 * kda_decode_step with a scalar gate (see kda_chunk_fwd_scalar_gate):
 *   g             [N, H] fp32 log a (<= 0), one per pair, or NULL for a = 1.
 *                 4-byte aligned.
 * Everything else as kda_decode_step.
 */
kda_status kda_decode_step_scalar_gate(int32_t num_sessions, int32_t num_heads,
                                       int32_t d_k, int32_t d_v, kda_dtype dtype,
                                       const void *q, const void *k,
                                       const void *v, const float *g,
                                       const float *beta, float scale,
                                       float *state_inout, void *o,
                                       struct ihipStream_t *stream);

/*
 * kda_chunk_fwd with the inputs in the form `form` describes (see
 * kda_inputs_form).  g_log_decay is [B, T, H, d_k] or [B, T, H] by
 * form->gate_layout (NULL for KDA_GATE_NONE); beta is [B, T, H] either way.
 * Everything else, including the workspace query, is as kda_chunk_fwd.
 */
kda_status kda_chunk_fwd_ex(const kda_shape *shape, const kda_inputs_form *form,
                            const void *q, const void *k, const void *v,
                            const float *g_log_decay, const float *beta,
                            float scale, const float *initial_state,
                            const int32_t *cu_seqlens, void *o,
                            float *final_state, void *workspace,
                            size_t workspace_bytes, struct ihipStream_t *stream);

/*
 * kda_decode_step with the inputs in the form `form` describes; g is
 * [N, H, d_k] or [N, H] by form->gate_layout (NULL for KDA_GATE_NONE).
 */
kda_status kda_decode_step_ex(int32_t num_sessions, int32_t num_heads,
                              int32_t d_k, int32_t d_v, kda_dtype dtype,
                              const kda_inputs_form *form, const void *q,
                              const void *k, const void *v, const float *g,
                              const float *beta, float scale,
                              float *state_inout, void *o, struct ihipStream_t *stream);

/*
 * Output stage of a KDA layer after the recurrence: RMS normalisation of each
 * (token, head) output row over its d_v channels, a learned per-channel
 * weight, and a sigmoid output gate ("Understanding Kimi Delta Attention",
 * section "From mathematics to the GPU", lists output gating and RMS
 * normalisation among the layer's steps around the core):
 *
 *   out[r, c] = o[r, c] / sqrt(mean_c' o[r, c']^2 + eps) * weight[c]
 *               * sigmoid(gate[r, c])
 *
 *   o, gate, out  [rows, d_v] in dtype (rows = tokens x heads, or sessions x
 *                 heads); out may equal o (in place) but not gate.
 *   weight        [d_v] fp32.
 *   eps           > 0.
 * d_v in {16, 32, 64, 128, 256}; rows >= 0 (0 enqueues nothing).  o, gate and
 * out 16-byte aligned for fp32 and 8-byte for bf16; weight 16-byte aligned.
 */
kda_status kda_output_rmsnorm_gate(int64_t rows, int32_t d_v, kda_dtype dtype,
                                   const void *o, const void *gate,
                                   const float *weight, float eps, void *out,
                                   struct ihipStream_t *stream);

/*
 * Gradients of kda_chunk_fwd (per-channel log-decays, plain inputs) for the
 * loss L = <o, d_o> + <final states, d_final_state>.  The pages derive no
 * gradients ("Kimi Delta Attention: How It Works, Step by Step" motivates the
 * chunkwise form by training); this reverses the chunk algebra of
 * "Understanding Kimi Delta Attention", sections "The triangular system" and
 * "Putting the chunks together", step by step.  A first kernel (one
 * workgroup per chunk and head) stores every per-chunk factor that does not
 * depend on the values.  A chain kernel (one workgroup per sequence, head and
 * 16 value columns) walks the chunks forward storing each chunk's start
 * state and Z = U - R S, then in reverse carrying dL/dS across chunk
 * boundaries and storing each chunk's end-state gradient and dZ (at d = 128
 * only every other state and end-state gradient); a last kernel (one
 * workgroup per chunk and head) forms every other gradient from one chunk's
 * inputs and those stored quantities, rebuilding a state or gradient that
 * was not stored with one chunk step from its neighbour's.
 *
 *   shape         as kda_chunk_fwd; dtype KDA_F32 or KDA_BF16 (the storage of
 *                 q, k, v and d_o), d_k = d_v = d with (d, chunk) in
 *                 {(16, 16|32|64), (32, 16|32), (64, 16|32), (128, 16|32|64)};
 *                 at d = 128 the gradients are formed over 16-token chunks
 *                 whatever the chunk (the chunkwise form is exact for any
 *                 chunk, so it changes only the rounding order).
 *   q, k, g_log_decay, v, beta, scale, initial_state, cu_seqlens
 *                 the forward's inputs, same layouts (initial_state may be NULL).
 *   d_o           [B, T, H, d_v], dtype as v: dL/do.
 *   All arithmetic is fp32 (bf16 inputs widen exactly); every gradient is
 *   written in fp32.
 *   d_final_state [N, H, d_k, d_v] fp32 or NULL (zeros).
 *   dq, dk, dv, dg, dbeta
 *                 fp32 outputs with the layouts of q, k, v, g_log_decay, beta.
 *   d_initial_state [N, H, d_k, d_v] fp32 or NULL (not written).
 *   workspace     at least kda_chunk_bwd_workspace_bytes(shape) bytes (0 for
 *                 an invalid or unsupported shape), 256-byte aligned: per
 *                 chunk slot and head (16-token slots at d = 128), fp32, the
 *                 chunk-start state and end-state gradient (d x d); Z, dZ
 *                 and the factors R, Kbar, Qbar (chunk x d); T, K~, H
 *                 (chunk x chunk); e^{G_C} (d); with T_total / chunk + N + 1
 *                 slots.  Its contents are scratch between calls.
 * Tensors 16-byte aligned (beta, dbeta, cu_seqlens 4-byte); outputs must not
 * alias inputs.  Log-decays must be finite.  Asynchronous on `stream`; the
 * library enqueues kernels only.
 */
size_t kda_chunk_bwd_workspace_bytes(const kda_shape *shape);
kda_status kda_chunk_bwd(const kda_shape *shape, const void *q, const void *k,
                         const void *v, const float *g_log_decay,
                         const float *beta, float scale,
                         const float *initial_state,
                         const int32_t *cu_seqlens, const void *d_o,
                         const float *d_final_state, float *dq, float *dk,
                         float *dv, float *dg, float *dbeta,
                         float *d_initial_state, void *workspace,
                         size_t workspace_bytes, struct ihipStream_t *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
