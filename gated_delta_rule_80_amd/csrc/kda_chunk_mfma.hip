// kda_chunk_mfma.hip -- chunkwise KDA prefill on gfx950 MFMA, d_k = d_v = 128,
// C = 64, bf16 storage, fp16 MFMA operands with fp32 accumulation.
//
// The chunk algebra is that of "Understanding Kimi Delta Attention"
// (A. Flores), sections "The triangular system" and "Putting the chunks
// together", written with the opposite sign for the coupling matrix
// (A here = -A there, so the solve is (I + A) T = I):
//   G_i    = sum_{r <= i} g_r                     (inclusive, per channel)
//   A_ij   = beta_i k_i^T Diag(e^{G_i - G_j}) k_j  (j < i)
//   T      = (I + A)^{-1}
//   W      = T Diag(beta) (K . e^{G})    U = T Diag(beta) V
//   H_ij   = s q_i^T Diag(e^{G_i - G_j}) k_j     (j <= i)
//   Qbar   = s Q . e^{G}                          Ktil = K . e^{G_C - G}
// and, carried across chunks with the state S (d_k x d_v, fp32):
//   Z = U - W S,   O = Qbar S + H Z,   S <- Diag(e^{G_C}) S + Ktil^T Z.
// The decay is folded into the vectors ("Kimi Delta Attention: a half-life
// per channel", section "What changes in the kernel") with secondary
// chunking: A and H are built from 16-token sub-chunk blocks, each with its
// own reference point, so no factor ever divides by the decay of more than
// half a sub-chunk.  Qbar, L and Ktil only ever scale by e^{x} with x <= 0.
// Exponents are differences of cumulative logs, as the derivation
// recommends.  Per-token log-decays below MIN_LOG_DECAY = -10 (down to -inf)
// are taken as -10: a retention of e^-10 = 4.5e-5 instead of less, which
// keeps every factor in range and changes o and S by at most that fraction of
// the state being forgotten.
//
// Kernels
//   kda_chunk_index  packed sequences -> chunk table (device side, no sync)
//   kda_intra        one workgroup per (chunk, head), fully parallel: the
//                    cumulative decay, A and H on MFMA (fp16 for the blocks
//                    between sub-chunks, fp16 or split bf16 inside them),
//                    (I + A)^{-1} (diagonal 16x16 blocks as the product
//                    (I - A)(I + A^2)(I + A^4)(I + A^8), off-diagonal blocks by
//                    block substitution, all on fp32 MFMA), then W on MFMA.
//                    Its outputs, with the fragments of T Diag(beta), go to
//                    the workspace already in the register-fragment order the
//                    inter kernel consumes.  It does not read v.
//   kda_inter        one workgroup per (sequence, head, 16- or 32-column value
//                    tile): the sequential chunk loop with the fp32 state
//                    resident in registers; it forms U = T Diag(beta) V from
//                    v one chunk ahead.  Columns of the value space evolve
//                    independently, so value tiles need no communication.
//
// MFMA fragments (v_mfma_f32_16x16x32_f16): lane l gives row/column l % 16
// and 8 reduction values for group l / 16; it receives output column l % 16,
// rows 4 (l / 16) .. +3.  The reduction index inside a fragment may be any
// permutation as long as both operands use the same one.  All fragments here
// that contract over 32 channels or 32 tokens use the permutation
//   slot s < 4  -> index 4 (l/16) + s,   slot s >= 4 -> index 16 + 4 (l/16) + s - 4
// which is exactly what two vertically adjacent 16x16 accumulator tiles hold,
// so an MFMA result feeds the next MFMA without leaving registers.
#include <mutex>

#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace mfma_path {

constexpr int C = 64, DK = 128, DV = 128;
// Floor of the per-token log-decay (natural log) on this path.  Within a
// 16-token sub-chunk the mid-point split factors then stay below e^{8 * 10},
// and a sub-chunk's whole decay below e^{160}: inside the fp32 / bf16 range.
constexpr float MIN_LOG_DECAY = -10.f;
#ifndef KDA_INTER_PF
#define KDA_INTER_PF 2
#endif
#ifndef KDA_INTER_PF_WIDE
#define KDA_INTER_PF_WIDE 2
#endif
#ifndef KDA_INTER_L2D
#define KDA_INTER_L2D 4
#endif
#ifndef KDA_INTER_L2R
#define KDA_INTER_L2R 4
#endif
#ifndef KDA_INTER_TOUCH
#define KDA_INTER_TOUCH 128
#endif
// Chunk records in flight per inter wave, for 16- and 32-column value tiles.
template <int NCT>
constexpr int ring_depth() { return NCT == 1 ? KDA_INTER_PF : KDA_INTER_PF_WIDE; }
constexpr int L2D = KDA_INTER_L2D;    // L2 prefetch distance in chunks (0: no prefetch wave)
constexpr int L2R = KDA_INTER_L2R;    // chunks a prefetch load may stay in flight
constexpr int TOUCH = KDA_INTER_TOUCH;  // bytes of a record between two prefetch touches
constexpr int INTER_THREADS = L2D > 0 ? 576 : 512;   // 4 state + 4 output (+ 1 prefetch) waves
constexpr int INTER_MAX_PAIRS = 1 << 19;               // (sequence, head) pairs per chain launch

// One chunk-head record in the workspace (bytes).  Fragment index -> 1 KB
// (64 lanes x 16 B) unless noted.
// U = T Diag(beta) V is not stored: the chain forms it from v and the T
// fragments, so the intra-chunk kernel neither reads v nor writes U.
constexpr int REC_W = 0;        // W   A-frags [token tile 4][channel block 4]
constexpr int REC_Q = 16384;    // Qbar A-frags [token tile 4][channel block 4]
constexpr int REC_K = 32768;    // Ktil^T A-frags [channel tile 8][token block 2]
constexpr int REC_H = 49152;    // H A-frags, 6 nonzero (token tile, token block) pairs
constexpr int REC_T = 55296;    // T Diag(beta) A-frags, the same 6 pairs
constexpr int REC_GE = 61440;   // e^{G_C} fp32 [128]
constexpr int REC_BYTES = 61952;
static_assert(REC_BYTES % 256 == 0, "record alignment");

// H and T fragment slot of (token tile it, token block kb), kb <= it / 2.
__device__ __forceinline__ int h_slot(int it, int kb) { return it < 2 ? it : 2 * it - 2 + kb; }

// ---- Record handoff between the two kernels when they run side by side ------------
// In the overlapped prefill the chain kernel starts beside the intra-chunk
// kernel and reads each record as soon as it is published, instead of after
// the whole intra-chunk launch.  The records are handed over through the L2 of
// one XCD (accelerator die), with no cache write-back or invalidation: the
// producer's stores of a record are acknowledged by L2 (the vector L1 writes
// through) before it stores the record's flag, and the chain reads flags and
// records through its own XCD's L2.  That holds only when producer and chain
// share an XCD.  Workgroups are dispatched to the 8 XCDs round-robin by id and
// both kernels place head h on XCD h mod 8 when H is a multiple of 8, but the
// flag carries the XCD the producer actually ran on, and the chain accepts a
// record only from its own XCD; anything else (another XCD, or a flag not seen
// in time) marks the call for a repair pass, which reruns the chain after both
// kernels have ended, as the serial order would.

// Flag value of a published record: nonzero, with the producer's XCD.
constexpr uint32_t REC_READY = 0x100u;

// The XCD this wave runs on (the XCC_ID hardware register).
__device__ __forceinline__ uint32_t xcc_id() {
    return __builtin_amdgcn_s_getreg((3 << 11) | 20) & 15u;   // HW_REG_XCC_ID, bits 3:0
}

// Work placement by XCD.  A dispatch does not always start on XCD 0, so two
// kernels on different queues cannot agree on a placement by workgroup id.  In
// the overlapped order every workgroup reads the XCD it runs on and claims the
// next item of that XCD's pool instead: n_items items, pool x holding those
// whose head is x mod 8, `per` consecutive pool items (the heads x, x + 8, ...
// of one position) at a time.  A workgroup whose pool is empty takes the next
// item of the following pools; there are exactly as many workgroups as items,
// so every item is taken once.  ctr: 8 zeroed counters.  Returns the pool and
// the rank of the item in it.  Called by one thread.
__device__ __forceinline__ void claim_item(uint32_t *ctr, int n_items, int *pool, int *rank) {
    const int x0 = (int)xcc_id() & 7, cap = n_items / 8;
    for (int d = 0; d < 8; ++d) {
        const int x = (x0 + d) & 7;
        const uint32_t k = __hip_atomic_fetch_add(ctr + x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((int)k < cap) {
            *pool = x;
            *rank = (int)k;
            return;
        }
    }
    *pool = x0;   // unreachable while the grid has n_items workgroups
    *rank = cap;
}

// Producer side, after the workgroup's last record store: every wave waits
// until its stores are acknowledged, then one thread stores the flag.
__device__ __forceinline__ void publish_record(uint32_t *flag, int tid) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt and lgkmcnt left at their maxima
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (tid == 0)
        __hip_atomic_store(flag, REC_READY | xcc_id(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Chunk {
    int seq, t0, len;
};

// Chunk c of the problem: equal rows (table == nullptr) or the device table.
__device__ __forceinline__ Chunk chunk_at(int c, const int4 *table, int row_len, int ncr) {
    if (!table) {
        const int b = c / ncr, j = c - b * ncr;
        return {b, b * row_len + j * C, min(C, row_len - j * C)};
    }
    const int4 e = table[c];
    return {e.x, e.y, e.z};
}

__device__ __forceinline__ float bf(uint16_t x) { return bf16_to_f32(x); }

// Value j of 8 bf16 packed two per word (low half first).
__device__ __forceinline__ float bf_at(const uint32_t (&w)[4], int j) {
    return (j & 1) ? __uint_as_float(w[j >> 1] & 0xffff0000u) : __uint_as_float(w[j >> 1] << 16);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): about 16 significant
// bits in two bf16 values, with the range of fp32.
__device__ __forceinline__ void split_bf16(float x, bf16x8 &hi, bf16x8 &lo, int j) {
    const __bf16 h = (__bf16)x;
    hi[j] = h;
    lo[j] = (__bf16)(x - (float)h);
}

// D = A * B + C for one 16x16 fp32 tile, K = 32 bf16, same lane layout as mfma16.
__device__ __forceinline__ float4v mfma16_bf16(bf16x8 a, bf16x8 b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Inclusive prefix sum across the 16 lanes of each DPP row.
__device__ __forceinline__ float row_scan16(float x) {
#define KDA_SHR(N)                                                                              \
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + (N), 0xf, 0xf, \
                                                    true));
    KDA_SHR(1) KDA_SHR(2) KDA_SHR(4) KDA_SHR(8)
#undef KDA_SHR
    return x;
}

// ------------------------------------------------------------------------------------
// Chunk table for packed sequences.  One workgroup; writes off[0..N] (chunk
// offsets, off[N] = number of chunks) and table[c] = {seq, first token, len}.
// Boundaries are sanitised first -- b'_0 = 0, b'_n = max(b'_{n-1}, clamp(cu[n],
// 0, T)) -- so that even a malformed cu_seqlens yields disjoint in-range
// sequences and at most T / C + N chunks: every later access stays in bounds.
// For a valid cu_seqlens (starting at 0, non-decreasing, ending at T) b' = cu.
// It also writes order[0..N): the sequences by chunk count, longest first (ties
// by index), so that the chain kernel starts the longest chains first and the
// short ones fill in behind them.  Beyond ORDER_MAX sequences the order is the
// identity (ranking costs O(N) per sequence).
// ------------------------------------------------------------------------------------
constexpr int ORDER_MAX = 1024;
// Exclusive scan over the 1024 threads of the workgroup, by sum or by max
// (inputs >= 0, so 0 is the identity of both); also returns the total.
template <bool MAX>
__device__ __forceinline__ int block_exclusive_scan(int x, int *s_wave, int &total) {
    auto op = [](int a, int b) { return MAX ? max(a, b) : a + b; };
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    int incl = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl = op(incl, y);
    }
    const int prev = __shfl_up(incl, 1, 64);
    if (lane == 63) s_wave[w] = incl;
    __syncthreads();
    if (w == 0) {
        int v = lane < 16 ? s_wave[lane] : 0;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const int y = __shfl_up(v, o, 64);
            if (lane >= o) v = op(v, y);
        }
        if (lane < 16) s_wave[16 + lane] = v;   // inclusive over waves 0..lane
    }
    __syncthreads();
    total = s_wave[31];
    const int before = w == 0 ? 0 : s_wave[16 + w - 1];
    const int r = op(before, lane == 0 ? 0 : prev);
    __syncthreads();   // s_wave is reused by the next scan
    return r;
}

__global__ __launch_bounds__(1024) void kda_chunk_index_kernel(const int32_t *__restrict__ cu,
                                                               int n_seqs, int total_tokens,
                                                               int32_t *__restrict__ off,
                                                               int32_t *__restrict__ order,
                                                               int4 *__restrict__ table) {
    __shared__ int s_wave[32];
    __shared__ int s_cnt[ORDER_MAX];
    const int t = threadIdx.x;
    const int per = (n_seqs + 1023) / 1024;
    const int s0 = min(n_seqs, t * per), s1 = min(n_seqs, s0 + per);
    auto clampT = [&](int x) { return min(total_tokens, max(0, x)); };
    int mx = 0;
    for (int n = s0; n < s1; ++n) mx = max(mx, clampT(cu[n + 1]));
    int tot;
    const int start = block_exclusive_scan<true>(mx, s_wave, tot);   // b'_{s0}
    int a = start, cnt = 0;
    for (int n = s0; n < s1; ++n) {
        const int b = max(a, clampT(cu[n + 1]));
        cnt += (b - a + C - 1) / C;
        a = b;
    }
    int run = block_exclusive_scan<false>(cnt, s_wave, tot);
    if (t == 0) off[n_seqs] = tot;
    a = start;
    for (int n = s0; n < s1; ++n) {
        const int b = max(a, clampT(cu[n + 1])), L = b - a;
        off[n] = run;
        for (int j = 0; j * C < L; ++j) table[run + j] = make_int4(n, a + j * C, min(C, L - j * C), 0);
        run += (L + C - 1) / C;
        a = b;
    }
    if (n_seqs > ORDER_MAX) {
        for (int n = s0; n < s1; ++n) order[n] = n;
        return;
    }
    // One sequence per thread here (per == 1): its rank among all counts.
    if (t < n_seqs) s_cnt[t] = cnt;
    __syncthreads();
    if (t < n_seqs) {
        int rank = 0;
        for (int m = 0; m < n_seqs; ++m) {
            const int cm = s_cnt[m];
            rank += (cm > cnt) || (cm == cnt && m < t);
        }
        order[rank] = t;
    }
}

// ------------------------------------------------------------------------------------
// Intra-chunk kernel.
// ------------------------------------------------------------------------------------
// LDS map (bytes).  Stages 1-2: fp16 fragments [row tile][channel block][lane]
// of the off-diagonal sub-chunk blocks, and the transposed Ktil.
constexpr int L_LK = 0;           // K e^{G - E_a}      sub-chunks 1..3   12288
constexpr int L_LQ = 12288;       // s Q e^{G - E_a}    sub-chunks 1..3   12288
constexpr int L_RB = 24576;       // K e^{E_{b+1} - G}  sub-chunks 0..2   12288
constexpr int L_RD = 36864;       // the same times e^{E_a - E_{b+1}}, blocks (2,0), (3,0), (3,1)
constexpr int L_KT = 49152;       // Ktil^T fp16 [128][TP]  18432 -> 67584
constexpr int L_NRM = 67584;      // fp32 [4 waves][64 rows][2]: partial |k|^2, |q|^2 (stage 1)
// Stage 2b-2c: per-wave partial sums of the 8 diagonal blocks, float4 [wave][block][lane].
constexpr int L_DP = 16640;       // 32768 -> 49408, over dead fragment buffers, clear of sA
// Stages 3-6 (the fragment buffers are dead by then).
constexpr int L_A = 0;            // fp32 [64][65]   16640
constexpr int L_BL = 16640;       // fp16 [128][72]  18432  L^T = (K e^{G})^T
constexpr int L_TF = 53504;       // fp32 [64][65]   16640  T
constexpr int L_T16 = 0;          // fp16 [64][72]    9216  T (after A is dead)
constexpr int L_BETA = 70144;     // fp32 [64]
constexpr int L_BYTES = 70400;
constexpr int TP = 72;            // fp16 pitch of transposed [channel][token] buffers
constexpr int AP = 65;            // fp32 pitch of A and T
static_assert(L_KT == L_RD + 12288 && L_KT + 128 * TP * 2 == L_NRM && L_NRM + 2048 <= L_BETA,
              "stage 1 LDS map");
static_assert(L_DP >= L_A + 64 * AP * 4 && L_DP + 32768 <= L_TF && L_BL + 128 * TP * 2 <= L_TF,
              "diagonal partials sit clear of sA and sTf; L^T clear of sTf");

// Block column J of T = (I + A)^{-1} below the diagonal, by one wave:
//   X_J = T_JJ;  X_b = -T_bb sum_{k=J}^{b-1} A_bk X_k  for b > J.
// X_k stays in accumulator registers (rows 4 (l/16) .. +3 of column l % 16)
// and is fed back as the B operand of v_mfma_f32_16x16x4f32 with the
// reduction index permuted accordingly (step s uses rows 4 (l/16) + s).
template <int J>
__device__ __forceinline__ void offdiag_column(const float *sA, float *sTf, int g4, int i16) {
    float4v X[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) X[J][e] = sTf[(16 * J + 4 * g4 + e) * AP + 16 * J + i16];
#pragma unroll
    for (int b = J + 1; b < 4; ++b) {
        float4v Y = {0, 0, 0, 0};
#pragma unroll
        for (int kk = J; kk < b; ++kk) {
            const float *arow = sA + (16 * b + i16) * AP + 16 * kk + 4 * g4;
#pragma unroll
            for (int s = 0; s < 4; ++s)
                Y = __builtin_amdgcn_mfma_f32_16x16x4f32(arow[s], X[kk][s], Y, 0, 0, 0);
        }
        float4v Xb = {0, 0, 0, 0};
        const float *trow = sTf + (16 * b + i16) * AP + 16 * b + 4 * g4;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            Xb = __builtin_amdgcn_mfma_f32_16x16x4f32(trow[s], Y[s], Xb, 0, 0, 0);
        X[b] = -Xb;
#pragma unroll
        for (int e = 0; e < 4; ++e) sTf[(16 * b + 4 * g4 + e) * AP + 16 * J + i16] = X[b][e];
    }
}

// Diagonal block w of T = (I + A)^{-1} by one wave, into the same block of
// sTf.  Ad holds the block of A in accumulator layout (rows 4 (l/16) + e,
// column l % 16); sA holds it too (row-major, pitch AP).
__device__ __forceinline__ void diag_inverse(const float *sA, float *sTf, int w, int g4, int i16,
                                             float4v Ad) {
    // A is strictly lower triangular, so A^16 = 0 and
    //   (I + A)^{-1} = (I - A)(I + A^2)(I + A^4)(I + A^8),
    // factors that commute.  On fp32 MFMA: the running product Y stays in
    // accumulator layout and is the B operand of each step (Y <- Y + P Y);
    // each power P is read as the A operand (row l % 16, column 4 (l/16) + s)
    // from LDS, A from sA and the higher powers from this wave's diagonal
    // block of sTf, which T overwrites at the end.  Every entry of A is at
    // most beta_i |k_i| |k_j| in size (its decay factor is <= 1), so the
    // powers stay small.  The reads follow writes by other lanes of this
    // wave: LDS executes a wave's operations in order; the waits keep the
    // compiler from moving the reads above the writes.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    float *blk = sTf + (16 * w) * AP + 16 * w;
    const float *arow = sA + (16 * w + i16) * AP + 16 * w + 4 * g4;
    const float *prow = blk + i16 * AP + 4 * g4;
    float4v Y, P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) Y[e] = (4 * g4 + e == i16 ? 1.f : 0.f) - Ad[e];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2)
        P = __builtin_amdgcn_mfma_f32_16x16x4f32(arow[s2], Ad[s2], P, 0, 0, 0);   // A^2
#pragma unroll
    for (int q2 = 0; q2 < 3; ++q2) {   // P = A^2, A^4, A^8
#pragma unroll
        for (int e = 0; e < 4; ++e) blk[(4 * g4 + e) * AP + i16] = P[e];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        float pa[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) pa[s2] = prow[s2];
        float4v Yn = Y, Pn = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            Yn = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[s2], Y[s2], Yn, 0, 0, 0);
            if (q2 < 2) Pn = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[s2], P[s2], Pn, 0, 0, 0);
        }
        Y = Yn;
        P = Pn;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) blk[(4 * g4 + e) * AP + i16] = Y[e];
}

// Stages 5, 3 and 6 of the intra-chunk kernels, after the diagonal inverses:
// the off-diagonal blocks of T and L^T transposed into LDS, then T Diag(beta)
// in fp16 and the WY factor W^T = L^T (T B)^T into the record, with the
// fragments of T B from which the chain forms U = (T B) V.  hL holds
// L = K e^{G} in fp16 for this lane's rows 16 r + l % 16 and channels ca.., cb...
__device__ __forceinline__ void finish_wy(uint8_t *smem, uint8_t *__restrict__ rec, int tid, int l,
                                          int w, int g4, int i16, int ca, int cb,
                                          const half8 (&hL)[4], const float *sA, float *sTf,
                                          const float *sBeta) {
    // ---- stage 5: off-diagonal blocks of T, block column j by wave j (fp32 MFMA); ----
    // ---- stage 3 alongside: L^T transposed into LDS (over the dead partials) ------
    // beta is applied to the columns of T in stage 6 (W = (T Diag(beta)) L), so L
    // goes to LDS unscaled.
    switch (w) {
    case 0: offdiag_column<0>(sA, sTf, g4, i16); break;
    case 1: offdiag_column<1>(sA, sTf, g4, i16); break;
    case 2: offdiag_column<2>(sA, sTf, g4, i16); break;
    default: break;
    }
    _Float16 *sBL = reinterpret_cast<_Float16 *>(smem + L_BL);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = 16 * r + i16;   // rows past the end hold zeros (masked loads)
#pragma unroll
        for (int j = 0; j < 8; ++j) sBL[(j < 4 ? ca + j : cb + j - 4) * TP + i] = hL[r][j];
    }
    lds_barrier();

    // ---- stage 6: T Diag(beta) to fp16, then W^T = L^T (T B)^T ------------------------
    _Float16 *sT16 = reinterpret_cast<_Float16 *>(smem + L_T16);
    {
        // thread: row i, columns j0 .. j0+15; all reads before the two 16-byte writes
        const int i = tid >> 2, j0 = 16 * (tid & 3);
        float tv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) tv[j] = sTf[i * AP + j0 + j];
        half8 h0, h1;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            h0[j] = (_Float16)((j0 + j <= i) ? tv[j] * sBeta[j0 + j] : 0.f);
            h1[j] = (_Float16)((j0 + 8 + j <= i) ? tv[8 + j] * sBeta[j0 + 8 + j] : 0.f);
        }
        *reinterpret_cast<half8 *>(sT16 + i * TP + j0) = h0;
        *reinterpret_cast<half8 *>(sT16 + i * TP + j0 + 8) = h1;
    }
    lds_barrier();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        float4v aw[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb > (it >> 1)) continue;
            const half8 tfrag =
                *reinterpret_cast<const half8 *>(sT16 + (16 * it + i16) * TP + 32 * kb + 8 * g4);
#pragma unroll
            for (int cl = 0; cl < 2; ++cl) {   // channel tiles 2w, 2w + 1 of W^T
                const half8 lfrag = *reinterpret_cast<const half8 *>(
                    sBL + (16 * (2 * w + cl) + i16) * TP + 32 * kb + 8 * g4);
                aw[cl] = mfma16(lfrag, tfrag, aw[cl]);   // rows: channels, cols: tokens
            }
            // Wave w stores the T B fragments of token tile w.
            if (it == w) reinterpret_cast<half8 *>(rec + REC_T)[h_slot(it, kb) * 64 + l] = tfrag;
        }
        // W A-frag (token tile it, channel block w): channel tile 2w in bytes
        // 0..7, channel tile 2w+1 in bytes 8..15.
        half8 hw;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            hw[e] = (_Float16)aw[0][e];
            hw[4 + e] = (_Float16)aw[1][e];
        }
        reinterpret_cast<half8 *>(rec + REC_W)[(it * 4 + w) * 64 + l] = hw;
    }
}

// Grid: one workgroup per (head, chunk).  With a chunk table (packed sequences)
// block b covers global chunk b / H.  Without one (B equal rows of ncr chunks)
// it covers local chunk jlo + (b / H) % jn of row (b / H) / jn, so a launch can
// produce one segment [jlo, jlo + jn) of every row.  Heads vary fastest, so the
// 32 heads of one chunk -- which share every token row of q, k, v, g -- are
// read together.  GATE says how g is laid out: [tokens, H, d_k] (one log-decay
// per channel), [tokens, H] (one per token and head, shared by its channels) or
// absent (no decay).
template <Gate GATE>
__global__ __launch_bounds__(256, 2) void kda_intra_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, float scale, int form, float eps, int H, int row_len,
    int ncr, const int4 *__restrict__ table, const int32_t *__restrict__ n_chunks, int nc_max,
    int jlo, int jn, uint8_t *__restrict__ recs, uint32_t *__restrict__ ready,
    uint32_t *__restrict__ claim) {
    // No FMA contraction in this kernel: the compiler would fuse differently in
    // each gate layout's instantiation, and a scalar gate would then no longer
    // give the bits of the same gate repeated over the channels.
#pragma clang fp contract(off)
    __shared__ __attribute__((aligned(16))) uint8_t smem[L_BYTES];
    int item = blockIdx.x;   // b H + h
    if (claim) {
        // Overlapped order: the item comes from this XCD's pool (heads = XCD mod 8).
        __shared__ int s_item;
        if (threadIdx.x == 0) {
            int x, k;
            claim_item(claim, (int)gridDim.x, &x, &k);
            const int per = H / 8;
            s_item = (k / per) * H + x + 8 * (k % per);
        }
        __syncthreads();
        item = s_item;
    }
    const int h = item % H, b = item / H;
    int c;
    if (table) {
        c = b;
        if (c >= *n_chunks) return;
    } else {
        const int row = b / jn, j = jlo + (b - row * jn);
        if (j >= ncr) return;
        c = row * ncr + j;
    }
    const Chunk ch = chunk_at(c, table, row_len, ncr);
    uint8_t *rec = recs + ((size_t)h * nc_max + c) * REC_BYTES;

    const int tid = threadIdx.x, l = tid & 63, g4 = l >> 4, i16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
    const int len = ch.len;
    const int ca = 32 * w + 4 * g4, cb = ca + 16;   // this lane's 8 channels: ca..ca+3, cb..cb+3

    half8 *sLK = reinterpret_cast<half8 *>(smem + L_LK);
    half8 *sLQ = reinterpret_cast<half8 *>(smem + L_LQ);
    half8 *sRB = reinterpret_cast<half8 *>(smem + L_RB);
    half8 *sRD = reinterpret_cast<half8 *>(smem + L_RD);
    _Float16 *sKt = reinterpret_cast<_Float16 *>(smem + L_KT);
    float *sBeta = reinterpret_cast<float *>(smem + L_BETA);

    // ---- stage 1: cumulative decay and the decay-scaled operands -------------------
    // k and q stay packed (two bf16 per word, channels in slot order) and are
    // expanded where they are used; nk, nq are the per-row L2-norm factors
    // (nq also carries the query scale s).
    float G[4][8], nk[4], nq[4];
    uint32_t kw[4][4], qw[4][4];
    // All loads are issued before any of them is used, so the four row tiles
    // cost one memory round trip; the gate's elementwise form is applied after.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = 16 * r + i16;
        const bool ok = i < len;
        const size_t base = ((size_t)(ch.t0 + (ok ? i : 0)) * H + h) * DK;
        float4v ga = {0, 0, 0, 0}, gb = {0, 0, 0, 0};
        uint2 ka = {0, 0}, kb2 = {0, 0}, qa = {0, 0}, qb = {0, 0};
        if (ok) {
            if constexpr (GATE == Gate::PerChannel) {
                ga = *reinterpret_cast<const float4v *>(g + base + ca);
                gb = *reinterpret_cast<const float4v *>(g + base + cb);
            } else if constexpr (GATE == Gate::Scalar) {
                ga[0] = g[(size_t)(ch.t0 + i) * H + h];
            }
            ka = *reinterpret_cast<const uint2 *>(k + base + ca);
            kb2 = *reinterpret_cast<const uint2 *>(k + base + cb);
            qa = *reinterpret_cast<const uint2 *>(q + base + ca);
            qb = *reinterpret_cast<const uint2 *>(q + base + cb);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            G[r][e] = ga[e];
            G[r][4 + e] = gb[e];
        }
        kw[r][0] = ka.x, kw[r][1] = ka.y, kw[r][2] = kb2.x, kw[r][3] = kb2.y;
        qw[r][0] = qa.x, qw[r][1] = qa.y, qw[r][2] = qb.x, qw[r][3] = qb.y;
        nk[r] = 1.f;
        nq[r] = scale;   // the query scale rides on the per-row factor
    }
    // Gate as a logit: log a = log sigmoid(x) on the valid rows (padding rows
    // keep log a = 0).  A scalar gate is broadcast over the channels.  Each
    // per-token log-decay is then floored at MIN_LOG_DECAY (NaN passes through):
    // a channel that keeps less than e^-10 of its state over one token keeps
    // e^-10 instead, which bounds every split factor below (see the secondary
    // chunking comment) whatever the gate, -inf included.  Log-decays are then
    // kept in base 2 (g log2 e), so every factor below is one exp2.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const bool ok = 16 * r + i16 < len;
        if constexpr (GATE == Gate::Scalar) {
            float gs = G[r][0];
            if ((form & kFormGateLogit) && ok) gs = log_sigmoid(gs);
#pragma unroll
            for (int j = 0; j < 8; ++j) G[r][j] = gs;
        } else if constexpr (GATE == Gate::PerChannel) {
            if ((form & kFormGateLogit) && ok) {
#pragma unroll
                for (int j = 0; j < 8; ++j) G[r][j] = log_sigmoid(G[r][j]);
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = G[r][j];
            G[r][j] = (x < MIN_LOG_DECAY ? MIN_LOG_DECAY : x) * 1.4426950408889634f;
        }
    }
    if (tid < C) {
        const int i = tid;
        float b = i < len ? beta[(size_t)(ch.t0 + i) * H + h] : 0.f;
        if ((form & kFormBetaLogit) && i < len) b = sigmoid(b);
        sBeta[i] = b;
    }
    // Optional L2 normalisation of q and k over their d_k channels: each lane
    // holds 8 channels of 4 rows; the 4 lanes of a row in a wave, then the 4
    // waves through LDS, complete the sums of squares.
    if (form & kFormL2Norm) {
        float *sNrm = reinterpret_cast<float *>(smem + L_NRM);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float a = 0.f, b = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float kx = bf_at(kw[r], j), qx = bf_at(qw[r], j);
                a += kx * kx;
                b += qx * qx;
            }
            a += __shfl_xor(a, 16, 64);
            a += __shfl_xor(a, 32, 64);
            b += __shfl_xor(b, 16, 64);
            b += __shfl_xor(b, 32, 64);
            if (g4 == 0) {
                sNrm[(w * 64 + 16 * r + i16) * 2 + 0] = a;
                sNrm[(w * 64 + 16 * r + i16) * 2 + 1] = b;
            }
        }
        lds_barrier();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * r + i16;
            float a = 0.f, b = 0.f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                a += sNrm[(ww * 64 + i) * 2 + 0];
                b += sNrm[(ww * 64 + i) * 2 + 1];
            }
            nk[r] = rsqrtf(a + eps);
            nq[r] = scale * rsqrtf(b + eps);
        }
    }
    // Secondary chunking ("Kimi Delta Attention: a half-life per channel",
    // section "What changes in the kernel"): the decay is folded into the
    // vectors relative to a point inside the chunk, never across the whole
    // chunk.  With E_a the cumulative log-decay before 16-token sub-chunk a
    // (E_0 = 0, E_4 = G_C), for sub-chunks a > b the factor e^{G_i - G_j}
    // (i in a, j in b) splits at the boundary before sub-chunk a:
    //   e^{G_i - E_a} * e^{E_{b+1} - G_j} * e^{E_a - E_{b+1}},
    // three factors that are all <= 1, so the fp16 operands cannot overflow
    // whatever the decay.  Inside a sub-chunk the split is taken at the
    // mid-point M_a = (E_a + E_{a+1}) / 2, so each factor lies within
    // e^{+-(E_a - E_{a+1}) / 2}: in range for fp32 and bf16 while the decay of
    // 16 tokens stays above about -175, which the floor of -10 per token
    // guarantees (-160 at most).
    float E[5][8];
    float gcmin = 0.f;   // the strongest whole-chunk decay (log2) among this lane's channels
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float carry = 0.f;   // inclusive cumsum: scan inside each sub-chunk, carry across
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float x = row_scan16(G[r][j]);
            E[r][j] = carry;
            G[r][j] = carry + x;
            carry += __shfl(x, (l & 48) | 15, 64);
        }
        E[4][j] = carry;
        gcmin = fminf(gcmin, carry);
        // e^{G_C} for the state decay, written by one lane per channel group
        if (i16 == 0) {
            float *ge = reinterpret_cast<float *>(rec + REC_GE);
            ge[(j < 4 ? ca + j : cb + j - 4)] = __builtin_amdgcn_exp2f(carry);
        }
    }
    half8 hL[4];         // L = K e^{G} in fp16, kept for stage 3
    float4v accD[8];     // diagonal blocks over this wave's 32 channels: A(r, r), then H^T(r, r)
    // Each wave picks the split for its own 32 channels; the fragments have the
    // same meaning either way (their products over a channel are the exact
    // pairwise factors), so stage 2 sums waves that chose differently.
    if (__all(gcmin >= -16.f)) {
        // Weak decay: the whole chunk decays by at most 2^-16 on every channel
        // of this wave.  One split point per channel, the chunk's mid-decay
        // M = G_C / 2, serves every block: e^{+-(G_i - M)} lies within 2^{+-8},
        // and e^{M} = e^{G_C - M} turns the split operands into Qbar, L, Ktil.
        float Mw[8], Em[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            Mw[j] = 0.5f * E[4][j];
            Em[j] = __builtin_amdgcn_exp2f(Mw[j]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            half8 hp, hm, hq, hqb;
            const int i = 16 * r + i16;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float e1 = __builtin_amdgcn_exp2f(G[r][j] - Mw[j]);
                const float e2 = __builtin_amdgcn_exp2f(Mw[j] - G[r][j]);
                const float kk = bf_at(kw[r], j) * nk[r], qq = bf_at(qw[r], j) * nq[r];
                const float kp = kk * e1, km = kk * e2, qp = qq * e1;
                hp[j] = (_Float16)kp;
                hm[j] = (_Float16)km;
                hq[j] = (_Float16)qp;
                hL[r][j] = (_Float16)(kp * Em[j]);                 // L = K e^{G}
                hqb[j] = (_Float16)(qp * Em[j]);                   // Qbar = s Q e^{G}
                const int cc = j < 4 ? ca + j : cb + j - 4;
                sKt[cc * TP + i] = (_Float16)(km * Em[j]);        // Ktil = K e^{G_C - G}
            }
            if (r >= 1) {
                sLK[((r - 1) * 4 + w) * 64 + l] = hp;
                sLQ[((r - 1) * 4 + w) * 64 + l] = hq;
            }
            if (r <= 2) sRB[(r * 4 + w) * 64 + l] = hm;
            if (r == 0) {
                sRD[(0 * 4 + w) * 64 + l] = hm;
                sRD[(1 * 4 + w) * 64 + l] = hm;
            }
            if (r == 1) sRD[(2 * 4 + w) * 64 + l] = hm;
            reinterpret_cast<half8 *>(rec + REC_Q)[(r * 4 + w) * 64 + l] = hqb;
            float4v a = {0, 0, 0, 0}, hh = {0, 0, 0, 0};
            accD[r] = mfma16(hp, hm, a);
            accD[4 + r] = mfma16(hm, hq, hh);
        }
    } else {
        // Sub-chunk splits.  Kept per (sub-chunk, channel): M_a and the
        // half-decay h_a = e^{(E_{a+1} - E_a) / 2}; s_a = h_a^2 is the sub-chunk's
        // whole decay, and the other factors are products of those: e^{E_a} =
        // s_0 .. s_{a-1}, e^{G_C - E_{a+1}} = s_{a+1} .. s_3, e^{E_a - E_{b+1}} =
        // s_{b+1} .. s_{a-1}.  Products of factors <= 1 only underflow where the
        // exact value is below the fp32 range.
        float M[4][8], hf[4][8];
        float dmax = 0.f;   // largest sub-chunk decay (log2) among this lane's channels
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                M[r][j] = 0.5f * (E[r][j] + E[r + 1][j]);
                hf[r][j] = __builtin_amdgcn_exp2f(0.5f * (E[r + 1][j] - E[r][j]));
                dmax = fmaxf(dmax, E[r][j] - E[r + 1][j]);
            }
        // Where no sub-chunk of this wave's channels decays by more than 2^-8,
        // the mid-point factors stay within 2^{+-4} and the diagonal blocks use
        // plain fp16 operands like the others; stronger decays take bf16 MFMA
        // with each operand split into a high and a low bf16 part (three
        // products, about 16 significant bits).
        const bool diag_fp16 = __all(dmax <= 8.f);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            half8 hlk, hlq, hrb, hrd0, hrd1, hqb;
            float dlk[8], dlq[8], drk[8];   // diagonal-block operands before rounding
            const int i = 16 * r + i16;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                // DL = e^{G_i - M_a}, DR = e^{M_a - G_i} lie within 1 / h_a and h_a;
                // X = e^{G_i - E_a} = DL h_a and Y = e^{E_{a+1} - G_i} = DR h_a are <= 1.
                const float DL = __builtin_amdgcn_exp2f(G[r][j] - M[r][j]);
                const float DR = __builtin_amdgcn_exp2f(M[r][j] - G[r][j]);
                const float X = DL * hf[r][j], Y = DR * hf[r][j];
                float sd[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) sd[t] = hf[t][j] * hf[t][j];
                float P = 1.f, Qf = 1.f;                           // e^{E_a}, e^{G_C - E_{a+1}}
#pragma unroll
                for (int t = 0; t < r; ++t) P *= sd[t];
#pragma unroll
                for (int t = 3; t > r; --t) Qf *= sd[t];
                const float kk = bf_at(kw[r], j) * nk[r], qq = bf_at(qw[r], j) * nq[r];
                const float kX = kk * X, qX = qq * X;
                hL[r][j] = (_Float16)(kX * P);                     // L = K e^{G}
                hqb[j] = (_Float16)(qX * P);                       // Qbar = s Q e^{G}
                hlk[j] = (_Float16)kX;
                hlq[j] = (_Float16)qX;
                const float ky = kk * Y;
                hrb[j] = (_Float16)ky;
                // blocks (2, 0) and (3, 1) scale by the sub-chunk between them, (3, 0) by two
                hrd0[j] = (_Float16)(ky * (r == 0 ? sd[1] : sd[2]));
                hrd1[j] = (_Float16)(ky * (sd[1] * sd[2]));
                const int cc = j < 4 ? ca + j : cb + j - 4;
                sKt[cc * TP + i] = (_Float16)(ky * Qf);           // Ktil = K e^{G_C - G}
                dlk[j] = kk * DL;
                dlq[j] = qq * DL;
                drk[j] = kk * DR;
            }
            if (r >= 1) {
                sLK[((r - 1) * 4 + w) * 64 + l] = hlk;
                sLQ[((r - 1) * 4 + w) * 64 + l] = hlq;
            }
            if (r <= 2) sRB[(r * 4 + w) * 64 + l] = hrb;
            if (r == 0) {
                sRD[(0 * 4 + w) * 64 + l] = hrd0;   // block (2, 0)
                sRD[(1 * 4 + w) * 64 + l] = hrd1;   // block (3, 0)
            }
            if (r == 1) sRD[(2 * 4 + w) * 64 + l] = hrd0;   // block (3, 1)
            reinterpret_cast<half8 *>(rec + REC_Q)[(r * 4 + w) * 64 + l] = hqb;
            // Diagonal block r: A rows i / columns j, H^T rows j / columns i.
            float4v a = {0, 0, 0, 0}, hh = {0, 0, 0, 0};
            if (diag_fp16) {
                half8 fk, fq, fr;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    fk[j] = (_Float16)dlk[j];
                    fq[j] = (_Float16)dlq[j];
                    fr[j] = (_Float16)drk[j];
                }
                a = mfma16(fk, fr, a);
                hh = mfma16(fr, fq, hh);
            } else {
                bf16x8 lk_hi, lk_lo, lq_hi, lq_lo, rk_hi, rk_lo;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    split_bf16(dlk[j], lk_hi, lk_lo, j);
                    split_bf16(dlq[j], lq_hi, lq_lo, j);
                    split_bf16(drk[j], rk_hi, rk_lo, j);
                }
                a = mfma16_bf16(lk_hi, rk_hi, a);
                a = mfma16_bf16(lk_hi, rk_lo, a);
                a = mfma16_bf16(lk_lo, rk_hi, a);
                hh = mfma16_bf16(rk_hi, lq_hi, hh);
                hh = mfma16_bf16(rk_lo, lq_hi, hh);
                hh = mfma16_bf16(rk_hi, lq_lo, hh);
            }
            accD[r] = a;
            accD[4 + r] = hh;
        }
    }
    lds_barrier();

    // ---- stage 2: off-diagonal blocks of A and H^T on MFMA; Ktil^T fragments out ----
    // Block u = 0..5 is the sub-chunk pair (a, b) = (1,0), (2,0), (2,1), (3,0),
    // (3,1), (3,2); list entries 0..5 are A(a, b), 6..11 are H^T(b, a).  Wave w
    // takes entries w, w+4, w+8: slot 0 is always an A block, slot 1 is an A
    // block for w < 2, slot 2 is always an H^T block.
    float4v accA[2];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        const int t = w + 4 * s;
        const bool is_a = t < 6;
        const int u = is_a ? t : t - 6;
        const int a = u >= 3 ? 3 : (u >= 1 ? 2 : 1);
        const int b = u - (a * (a - 1)) / 2;
        const half8 *right = (a == b + 1) ? sRB + b * 256 : sRD + (u == 1 ? 0 : (u == 3 ? 1 : 2)) * 256;
        const half8 *lk = sLK + (a - 1) * 256, *lq = sLQ + (a - 1) * 256;
        float4v acc = {0, 0, 0, 0};
        if (is_a) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) acc = mfma16(lk[kb * 64 + l], right[kb * 64 + l], acc);
            // A_ij = beta_i * acc (rows i = 16a + 4 g4 + e, all columns j < i)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] *= sBeta[16 * a + 4 * g4 + e];
            if (s < 2) accA[s] = acc;
        } else {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) acc = mfma16(right[kb * 64 + l], lq[kb * 64 + l], acc);
            half4 hv;
#pragma unroll
            for (int e = 0; e < 4; ++e) hv[e] = (_Float16)acc[e];
            uint8_t *dst = rec + REC_H + (h_slot(a, b >> 1) * 64 + l) * 16;
            *reinterpret_cast<half4 *>(dst + (b & 1) * 8) = hv;
        }
    }
    // Ktil^T fragments: channel tiles 2w, 2w+1, token blocks 0, 1.
#pragma unroll
    for (int cl = 0; cl < 2; ++cl) {
        const int ct = 2 * w + cl;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const _Float16 *row = sKt + (16 * ct + i16) * TP + 32 * kb + 4 * g4;
            const half4 lo = *reinterpret_cast<const half4 *>(row);
            const half4 hi = *reinterpret_cast<const half4 *>(row + 16);
            half8 f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[e] = lo[e];
                f[4 + e] = hi[e];
            }
            reinterpret_cast<half8 *>(rec + REC_K)[(ct * 2 + kb) * 64 + l] = f;
        }
    }
    lds_barrier();

    // ---- stage 2b: diagonal partial sums to LDS; off-diagonal A blocks into sA ------
    float *sA = reinterpret_cast<float *>(smem + L_A);
    float4v *sDP = reinterpret_cast<float4v *>(smem + L_DP);
#pragma unroll
    for (int d = 0; d < 8; ++d) sDP[(w * 8 + d) * 64 + l] = accD[d];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int t = w + 4 * s;
        if (t < 6) {
            const int a = t >= 3 ? 3 : (t >= 1 ? 2 : 1);
            const int b = t - (a * (a - 1)) / 2;
#pragma unroll
            for (int e = 0; e < 4; ++e) sA[(16 * a + 4 * g4 + e) * AP + 16 * b + i16] = accA[s][e];
        }
    }
    lds_barrier();

    // ---- stage 4: diagonal blocks summed in wave order; their inverses -------------
    // Wave w sums diagonal block w of A (into sA) and of H^T (into the record),
    // then inverts diagonal block w of (I + A).  It reads only what it wrote,
    // so no barrier is needed in between.
    float *sTf = reinterpret_cast<float *>(smem + L_TF);
    {
        float4v a = sDP[(0 * 8 + w) * 64 + l], hs = sDP[(0 * 8 + 4 + w) * 64 + l];
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) {
            a += sDP[(ww * 8 + w) * 64 + l];
            hs += sDP[(ww * 8 + 4 + w) * 64 + l];
        }
        half4 hv;
        float4v Ad;   // diagonal block w of A, rows 4 (l/16) + e, column l % 16
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int rr = 16 * w + 4 * g4 + e, cc = 16 * w + i16;
            // A(rr, cc) for cc < rr; H^T(rr, cc) = H(cc, rr) for rr <= cc
            Ad[e] = (cc < rr) ? a[e] * sBeta[rr] : 0.f;
            sA[rr * AP + cc] = Ad[e];
            hv[e] = (_Float16)((rr <= cc) ? hs[e] : 0.f);
        }
        uint8_t *dst = rec + REC_H + (h_slot(w, w >> 1) * 64 + l) * 16;
        *reinterpret_cast<half4 *>(dst + (w & 1) * 8) = hv;
        if (!(w & 1)) {
            const half4 z = {0, 0, 0, 0};
            *reinterpret_cast<half4 *>(dst + 8) = z;
        }
        diag_inverse(sA, sTf, w, g4, i16, Ad);
    }
    lds_barrier();

    finish_wy(smem, rec, tid, l, w, g4, i16, ca, cb, hL, sA, sTf, sBeta);
    if (ready) publish_record(ready + (size_t)h * nc_max + c, tid);
}

// ------------------------------------------------------------------------------------
// Intra-chunk kernel for a scalar gate (one log-decay per token and head, Gated
// DeltaNet's gate) or none (DeltaNet).  With the same decay on every key channel
// the factor e^{G_i - G_j} leaves the sum over channels:
//   A_ij = beta_i e^{G_i - G_j} (k_i . k_j)   (j < i)
//   H_ij = e^{G_i - G_j} (s q_i . k_j)        (j <= i)
// so K K^T and (s Q) K^T are plain MFMA products of fp16 k and q, and the decay
// is a C x C mask applied in fp32 to the accumulators, every factor <= 1 ("Kimi
// Delta Attention: a half-life per channel", section "What changes in the
// kernel": the scalar gate's C x C mask).  No split points and no per-element
// exponentials: L = K e^{G}, Qbar = s Q e^{G} and Ktil = K e^{G_C - G} scale
// whole rows by one factor each.  The record written is the one kda_intra_kernel
// writes, so the chunk chain is shared.  Per-token log-decays are floored at
// MIN_LOG_DECAY as there, so cumulative logs stay finite (-inf included).
// ------------------------------------------------------------------------------------
constexpr int LS_K = 0;        // K fp16 A/B-fragments [row tile 4][channel block 4][lane]  16384
constexpr int LS_Q = 16384;    // s Q fp16 fragments, same layout                            16384
constexpr int LS_G = 32768;    // G (log2 units) fp32 [64]                                   256
static_assert(LS_G + 256 <= L_KT && L_NRM + 2048 <= L_BETA, "scalar-gate stage 1 LDS map");

// Lower-triangle tile u = 0..9 of a 4 x 4 tile grid: (a, b) with b <= a.
__device__ __forceinline__ void lower_tile(int u, int &a, int &b) {
    a = u >= 6 ? 3 : (u >= 3 ? 2 : (u >= 1 ? 1 : 0));
    b = u - (a * (a + 1)) / 2;
}
// Strictly-lower tile t = 0..5: (1,0), (2,0), (2,1), (3,0), (3,1), (3,2).
__device__ __forceinline__ void offdiag_tile(int t, int &a, int &b) {
    a = t >= 3 ? 3 : (t >= 1 ? 2 : 1);
    b = t - (a * (a - 1)) / 2;
}

template <bool HAS_GATE>
__global__ __launch_bounds__(256, 2) void kda_intra_scalar_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, float scale, int form, float eps, int H, int row_len,
    int ncr, const int4 *__restrict__ table, const int32_t *__restrict__ n_chunks, int nc_max,
    int jlo, int jn, uint8_t *__restrict__ recs, uint32_t *__restrict__ ready,
    uint32_t *__restrict__ claim) {
#pragma clang fp contract(off)
    __shared__ __attribute__((aligned(16))) uint8_t smem[L_BYTES];
    int item = blockIdx.x;   // b H + h
    if (claim) {
        // Overlapped order: the item comes from this XCD's pool (heads = XCD mod 8).
        __shared__ int s_item;
        if (threadIdx.x == 0) {
            int x, k;
            claim_item(claim, (int)gridDim.x, &x, &k);
            const int per = H / 8;
            s_item = (k / per) * H + x + 8 * (k % per);
        }
        __syncthreads();
        item = s_item;
    }
    const int h = item % H, b = item / H;
    int c;
    if (table) {
        c = b;
        if (c >= *n_chunks) return;
    } else {
        const int row = b / jn, j = jlo + (b - row * jn);
        if (j >= ncr) return;
        c = row * ncr + j;
    }
    const Chunk ch = chunk_at(c, table, row_len, ncr);
    uint8_t *rec = recs + ((size_t)h * nc_max + c) * REC_BYTES;

    const int tid = threadIdx.x, l = tid & 63, g4 = l >> 4, i16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int len = ch.len;
    const int ca = 32 * w + 4 * g4, cb = ca + 16;   // this lane's 8 channels

    half8 *sK = reinterpret_cast<half8 *>(smem + LS_K);
    half8 *sQ = reinterpret_cast<half8 *>(smem + LS_Q);
    float *sG = reinterpret_cast<float *>(smem + LS_G);
    _Float16 *sKt = reinterpret_cast<_Float16 *>(smem + L_KT);
    float *sBeta = reinterpret_cast<float *>(smem + L_BETA);

    // ---- stage 1: loads, cumulative decay, fp16 operands ------------------------------
    float gr[4], nk[4], nq[4];
    uint32_t kw[4][4], qw[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = 16 * r + i16;
        const bool ok = i < len;
        const size_t row = (size_t)(ch.t0 + (ok ? i : 0)) * H + h;
        uint2 ka = {0, 0}, kb2 = {0, 0}, qa = {0, 0}, qb = {0, 0};
        gr[r] = 0.f;
        if (ok) {
            if constexpr (HAS_GATE) gr[r] = g[row];
            ka = *reinterpret_cast<const uint2 *>(k + row * DK + ca);
            kb2 = *reinterpret_cast<const uint2 *>(k + row * DK + cb);
            qa = *reinterpret_cast<const uint2 *>(q + row * DK + ca);
            qb = *reinterpret_cast<const uint2 *>(q + row * DK + cb);
        }
        kw[r][0] = ka.x, kw[r][1] = ka.y, kw[r][2] = kb2.x, kw[r][3] = kb2.y;
        qw[r][0] = qa.x, qw[r][1] = qa.y, qw[r][2] = qb.x, qw[r][3] = qb.y;
        nk[r] = 1.f;
        nq[r] = scale;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float x = gr[r];
        if (HAS_GATE && (form & kFormGateLogit) && 16 * r + i16 < len) x = log_sigmoid(x);
        gr[r] = (x < MIN_LOG_DECAY ? MIN_LOG_DECAY : x) * 1.4426950408889634f;
    }
    if (tid < C) {
        const int i = tid;
        float bt = i < len ? beta[(size_t)(ch.t0 + i) * H + h] : 0.f;
        if ((form & kFormBetaLogit) && i < len) bt = sigmoid(bt);
        sBeta[i] = bt;
    }
    if (form & kFormL2Norm) {
        float *sNrm = reinterpret_cast<float *>(smem + L_NRM);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float a = 0.f, bb = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float kx = bf_at(kw[r], j), qx = bf_at(qw[r], j);
                a += kx * kx;
                bb += qx * qx;
            }
            a += __shfl_xor(a, 16, 64);
            a += __shfl_xor(a, 32, 64);
            bb += __shfl_xor(bb, 16, 64);
            bb += __shfl_xor(bb, 32, 64);
            if (g4 == 0) {
                sNrm[(w * 64 + 16 * r + i16) * 2 + 0] = a;
                sNrm[(w * 64 + 16 * r + i16) * 2 + 1] = bb;
            }
        }
        lds_barrier();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * r + i16;
            float a = 0.f, bb = 0.f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                a += sNrm[(ww * 64 + i) * 2 + 0];
                bb += sNrm[(ww * 64 + i) * 2 + 1];
            }
            nk[r] = rsqrtf(a + eps);
            nq[r] = scale * rsqrtf(bb + eps);
        }
    }
    // Inclusive cumulative log-decay of the token rows (log2 units): a scan over
    // the 16 lanes of each row tile, carried across the tiles.
    float G2[4], carry = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float x = row_scan16(gr[r]);
        G2[r] = carry + x;
        carry += __shfl(x, (l & 48) | 15, 64);
    }
    const float G2C = carry;   // G at the chunk's last row (padding rows add 0)
    if (w == 0 && g4 == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sG[16 * r + i16] = G2[r];
    }
    if (i16 == 0) {
        float *ge = reinterpret_cast<float *>(rec + REC_GE);
        const float eC = __builtin_amdgcn_exp2f(G2C);
        const float4v e4 = {eC, eC, eC, eC};
        *reinterpret_cast<float4v *>(ge + ca) = e4;
        *reinterpret_cast<float4v *>(ge + cb) = e4;
    }
    half8 hL[4];   // L = K e^{G} in fp16, for stage 3
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = 16 * r + i16;
        const float eG = __builtin_amdgcn_exp2f(G2[r]), eK = __builtin_amdgcn_exp2f(G2C - G2[r]);
        half8 hk, hq, hqb;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float kk = bf_at(kw[r], j) * nk[r], qq = bf_at(qw[r], j) * nq[r];
            hk[j] = (_Float16)kk;
            hq[j] = (_Float16)qq;
            hL[r][j] = (_Float16)(kk * eG);    // L = K e^{G}
            hqb[j] = (_Float16)(qq * eG);      // Qbar = s Q e^{G}
            const int cc = j < 4 ? ca + j : cb + j - 4;
            sKt[cc * TP + i] = (_Float16)(kk * eK);   // Ktil = K e^{G_C - G}
        }
        sK[(r * 4 + w) * 64 + l] = hk;
        sQ[(r * 4 + w) * 64 + l] = hq;
        reinterpret_cast<half8 *>(rec + REC_Q)[(r * 4 + w) * 64 + l] = hqb;
    }
    lds_barrier();

    // ---- stage 2: K K^T and (s Q) K^T tiles on MFMA, masked by the decay --------------
    // Wave w takes diagonal tile (w, w) of A, then 4 of the other 16 tiles: the 6
    // off-diagonal A tiles and the 10 lower H^T tiles (list entries 0..5 and 6..15).
    float4v accA[2];   // this wave's off-diagonal A tiles (waves 0, 1 have two, 2, 3 one)
    float4v Ad;        // diagonal tile (w, w) of A
    {
        float4v acc = {0, 0, 0, 0};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            acc = mfma16(sK[(w * 4 + kb) * 64 + l], sK[(w * 4 + kb) * 64 + l], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * w + 4 * g4 + e, j = 16 * w + i16;
            Ad[e] = (j < i) ? acc[e] * sBeta[i] * __builtin_amdgcn_exp2f(sG[i] - sG[j]) : 0.f;
        }
    }
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
        const int t = w + 4 * s2;
        int a, bt;
        if (t < 6) {
            // off-diagonal A tile t of (1,0), (2,0), (2,1), (3,0), (3,1), (3,2)
            offdiag_tile(t, a, bt);
            float4v acc = {0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                acc = mfma16(sK[(a * 4 + kb) * 64 + l], sK[(bt * 4 + kb) * 64 + l], acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * a + 4 * g4 + e, j = 16 * bt + i16;
                acc[e] = acc[e] * sBeta[i] * __builtin_amdgcn_exp2f(sG[i] - sG[j]);
            }
            accA[s2] = acc;   // s2 is 0 or 1 here (t < 6)
        } else {
            // H^T tile (bt, a) of lower tile u = t - 6: rows tokens j, columns tokens i
            lower_tile(t - 6, a, bt);
            float4v acc = {0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                acc = mfma16(sK[(bt * 4 + kb) * 64 + l], sQ[(a * 4 + kb) * 64 + l], acc);
            half4 hv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 16 * bt + 4 * g4 + e, i = 16 * a + i16;
                hv[e] = (_Float16)((j <= i) ? acc[e] * __builtin_amdgcn_exp2f(sG[i] - sG[j]) : 0.f);
            }
            uint8_t *dst = rec + REC_H + (h_slot(a, bt >> 1) * 64 + l) * 16;
            *reinterpret_cast<half4 *>(dst + (bt & 1) * 8) = hv;
            if (a == bt && !(a & 1)) {   // tile (a, a + 1) above the diagonal shares the slot
                const half4 z = {0, 0, 0, 0};
                *reinterpret_cast<half4 *>(dst + 8) = z;
            }
        }
    }
    // Ktil^T fragments: channel tiles 2w, 2w+1, token blocks 0, 1.
#pragma unroll
    for (int cl = 0; cl < 2; ++cl) {
        const int ct = 2 * w + cl;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const _Float16 *rowp = sKt + (16 * ct + i16) * TP + 32 * kb + 4 * g4;
            const half4 lo = *reinterpret_cast<const half4 *>(rowp);
            const half4 hi = *reinterpret_cast<const half4 *>(rowp + 16);
            half8 f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[e] = lo[e];
                f[4 + e] = hi[e];
            }
            reinterpret_cast<half8 *>(rec + REC_K)[(ct * 2 + kb) * 64 + l] = f;
        }
    }
    lds_barrier();

    // ---- stage 2b and 4: A tiles into sA; each wave inverts its diagonal block --------
    float *sA = reinterpret_cast<float *>(smem + L_A);
    float *sTf = reinterpret_cast<float *>(smem + L_TF);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
        const int t = w + 4 * s2;
        if (t < 6) {
            int a, bt;
            offdiag_tile(t, a, bt);
#pragma unroll
            for (int e = 0; e < 4; ++e) sA[(16 * a + 4 * g4 + e) * AP + 16 * bt + i16] = accA[s2][e];
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) sA[(16 * w + 4 * g4 + e) * AP + 16 * w + i16] = Ad[e];
    diag_inverse(sA, sTf, w, g4, i16, Ad);
    lds_barrier();

    finish_wy(smem, rec, tid, l, w, g4, i16, ca, cb, hL, sA, sTf, sBeta);
    if (ready) publish_record(ready + (size_t)h * nc_max + c, tid);
}

// ------------------------------------------------------------------------------------
// Inter-chunk kernel: the sequential chunk loop for one (sequence, head, value tile).
// ------------------------------------------------------------------------------------
// Eight waves, two per SIMD, in two roles that share no operand:
//   state wave t (0..3)   owns channel rows 32t..32t+31 of the state (fp32, in
//                         registers) and, for token tile t, Z = U - W S; it then
//                         applies S <- Diag(e^{G_C}) S + Ktil^T Z.  This is the
//                         serial chain from chunk to chunk.
//   output wave t (0..3)  computes token tile t of O = Qbar S + H Z and stores it,
//                         off the chain.  It also forms token tile t of
//                         U = (T Diag(beta)) V one chunk ahead, from the value
//                         rows it staged in LDS (transposed, fp16) the step before.
// S and Z (fp16) and U (fp32) are exchanged through LDS with two barriers per
// chunk.  Each operand fragment is reused for the NCT 16-column tiles of the
// workgroup, and each byte of a chunk record is loaded by exactly one wave of
// the CU.
template <int NCT>
struct StateOps {
    half8 W[4], K[4];
    float4v ge[2];
};
// Ring slot of an output wave for chunk x: Qbar and H of x, T Diag(beta) of
// x + 1 and the value rows of x + 2 (each is used that many steps earlier).
template <int NCT>
struct OutOps {
    half8 Q[4], H[2], T[2];
    uint32_t V[2 * NCT];   // bf16 pairs: row 16 t + l / 4, columns 4 NCT (l % 4) .. of the tile
};

// Value rows of one (sequence, head, value tile) as this lane loads them: local
// chunk x - first covers rows (x - first) C .. of the sequence's len rows.
struct VRows {
    const uint16_t *p;   // row 0 of the sequence, at this lane's columns
    size_t stride;       // elements from one row to the next
    int first, len;
};

constexpr int VTP = 72;   // fp16 pitch (tokens) of the transposed value rows in LDS

// Refills are split by the step that consumes each piece, so a buffer is
// reloaded for the chunk PF ahead right after each piece's last use.
template <int NCT>
__device__ __forceinline__ void load_w(StateOps<NCT> &op, const uint8_t *rec, int t, int l) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
        op.W[kb] = reinterpret_cast<const half8 *>(rec + REC_W)[(t * 4 + kb) * 64 + l];
}
template <int NCT>
__device__ __forceinline__ void load_kg(StateOps<NCT> &op, const uint8_t *rec, int t, int l) {
#pragma unroll
    for (int cl = 0; cl < 2; ++cl)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            op.K[cl * 2 + kb] =
                reinterpret_cast<const half8 *>(rec + REC_K)[((2 * t + cl) * 2 + kb) * 64 + l];
    const float *ge = reinterpret_cast<const float *>(rec + REC_GE);
#pragma unroll
    for (int cl = 0; cl < 2; ++cl)
        op.ge[cl] = *reinterpret_cast<const float4v *>(ge + 16 * (2 * t + cl) + 4 * (l >> 4));
}
// Fragments of token tile t in the 6-slot layout of H and T B (zero above the diagonal).
__device__ __forceinline__ void load_tri(half8 (&f)[2], const uint8_t *src, int t, int l) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
        f[kb] = (kb <= (t >> 1)) ? reinterpret_cast<const half8 *>(src)[h_slot(t, kb) * 64 + l]
                                 : half8{0, 0, 0, 0, 0, 0, 0, 0};
}
template <int NCT>
__device__ __forceinline__ void load_v(uint32_t (&V)[2 * NCT], const VRows &vr, int x, int t, int l) {
    const int rel = (x - vr.first) * C + 16 * t + (l >> 2);
    const bool ok = rel < vr.len;   // rows past the sequence's end are zeros
    const uint16_t *src = vr.p + (size_t)(ok ? rel : 0) * vr.stride;
    if constexpr (NCT == 1) {
        const uint2 u = ok ? *reinterpret_cast<const uint2 *>(src) : uint2{0, 0};
        V[0] = u.x, V[1] = u.y;
    } else {
#pragma unroll
        for (int i = 0; i < NCT / 2; ++i) {   // 8 columns per 16-byte load
            const uint4 u = ok ? reinterpret_cast<const uint4 *>(src)[i] : uint4{0, 0, 0, 0};
            V[4 * i] = u.x, V[4 * i + 1] = u.y, V[4 * i + 2] = u.z, V[4 * i + 3] = u.w;
        }
    }
}
// Value rows 16 t .. 16 t + 15 of one chunk into LDS as fp16 [column][token].
template <int NCT>
__device__ __forceinline__ void stage_v(const uint32_t (&V)[2 * NCT], _Float16 *sVt, int t, int l) {
    const int tok = 16 * t + (l >> 2), col0 = 4 * NCT * (l & 3);
#pragma unroll
    for (int j = 0; j < 4 * NCT; ++j)
        sVt[(col0 + j) * VTP + tok] = (_Float16)bf((j & 1) ? (V[j >> 1] >> 16) : (V[j >> 1] & 0xffff));
}
// Token tile t of U = (T B) V for one chunk, from its staged value rows, into
// sU in the accumulator layout of Z (rows 16 t + 4 (l/16) + e, column l % 16).
template <int NCT>
__device__ __forceinline__ void form_u(const half8 (&T)[2], const _Float16 *sVt, float4v *sU, int t,
                                       int l) {
    const int g4 = l >> 4, i16 = l & 15;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        float4v u = {0, 0, 0, 0};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            if (kb <= (t >> 1))
                u = mfma16(T[kb],
                           *reinterpret_cast<const half8 *>(sVt + (16 * ct + i16) * VTP + 32 * kb + 8 * g4),
                           u);
        sU[(t * NCT + ct) * 64 + l] = u;
    }
}

// Chunk step of a state wave (token tile / channel block t); sU holds this chunk's U.
template <int NCT>
__device__ __forceinline__ void state_step(float4v (&S)[2][NCT], StateOps<NCT> &op, half8 *sS,
                                           half8 *sZ, const float4v *sU, int t, int l,
                                           const uint8_t *next) {
    // S -> fp16 B-fragments of channel block t.
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        half8 f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[e] = (_Float16)S[0][ct][e];
            f[4 + e] = (_Float16)S[1][ct][e];
        }
        sS[(t * NCT + ct) * 64 + l] = f;
    }
    lds_barrier();
    // Z = U - W S for token tile t (rows: tokens).
    float4v u[NCT], p[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        u[ct] = sU[(t * NCT + ct) * 64 + l];
        p[ct] = float4v{0, 0, 0, 0};
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) p[ct] = mfma16(op.W[kb], sS[(kb * NCT + ct) * 64 + l], p[ct]);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        half4 zh;
#pragma unroll
        for (int e = 0; e < 4; ++e) zh[e] = (_Float16)(u[ct][e] - p[ct][e]);
        *reinterpret_cast<half4 *>(reinterpret_cast<uint8_t *>(&sZ[((t >> 1) * NCT + ct) * 64 + l]) +
                                   (t & 1) * 8) = zh;
    }
    load_w(op, next, t, l);
    lds_barrier();
    // S <- Diag(e^{G_C}) S + Ktil^T Z for channel rows 32t .. 32t+31.
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        const half8 z0 = sZ[(0 * NCT + ct) * 64 + l], z1 = sZ[(1 * NCT + ct) * 64 + l];
#pragma unroll
        for (int cl = 0; cl < 2; ++cl) {
            float4v acc = S[cl][ct] * op.ge[cl];
            acc = mfma16(op.K[cl * 2 + 0], z0, acc);
            acc = mfma16(op.K[cl * 2 + 1], z1, acc);
            S[cl][ct] = acc;
        }
    }
    load_kg(op, next, t, l);
}

// Chunk step of an output wave (token tile t) for chunk c: O^T = S^T Qbar^T +
// Z^T H^T; after the second barrier also U of chunk c + 1 into sU1 from the
// value rows in sVt1, and the value rows of chunk c + 2 into sVt2.  The ring
// slot is refilled for chunk c + PF (x below).
template <int NCT>
__device__ __forceinline__ void output_step(OutOps<NCT> &op, const half8 *sS, const half8 *sZ,
                                            const _Float16 *sVt1, float4v *sU1, _Float16 *sVt2,
                                            const Chunk &ch, int H, int h, int t, int l, int vt0,
                                            const uint8_t *rbase, int x, int clast,
                                            const VRows &vr, uint16_t *__restrict__ o) {
    const int g4 = l >> 4, i16 = l & 15;
    lds_barrier();
    float4v O[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) O[ct] = float4v{0, 0, 0, 0};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) O[ct] = mfma16(sS[(kb * NCT + ct) * 64 + l], op.Q[kb], O[ct]);
    {
        const uint8_t *rq = rbase + (size_t)min(x, clast) * REC_BYTES;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            op.Q[kb] = reinterpret_cast<const half8 *>(rq + REC_Q)[(t * 4 + kb) * 64 + l];
    }
    lds_barrier();
    const int tok = 16 * t + i16;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            if (kb <= (t >> 1)) O[ct] = mfma16(sZ[(kb * NCT + ct) * 64 + l], op.H[kb], O[ct]);
        if (tok < ch.len) {
            const size_t ob = ((size_t)(ch.t0 + tok) * H + h) * DV + 16 * (vt0 + ct) + 4 * g4;
            uint2 pk;
            pk.x = pack_bf16x2(O[ct][0], O[ct][1]);
            pk.y = pack_bf16x2(O[ct][2], O[ct][3]);
            *reinterpret_cast<uint2 *>(o + ob) = pk;
        }
    }
    form_u<NCT>(op.T, sVt1, sU1, t, l);
    stage_v<NCT>(op.V, sVt2, t, l);
    load_tri(op.H, rbase + (size_t)min(x, clast) * REC_BYTES + REC_H, t, l);
    load_tri(op.T, rbase + (size_t)min(x + 1, clast) * REC_BYTES + REC_T, t, l);
    load_v<NCT>(op.V, vr, min(x + 2, clast), t, l);
}

// The chain's side of the record handoff in the overlapped order, run by the
// ninth wave of the workgroup.  The other waves load record x at step x - PF
// (the T Diag(beta) fragments at step x - PF - 1, after that step's second
// barrier), and the first PF + 1 records before the loop; the handoff wave
// accepts each record before the barrier that precedes its first load.  A record's flag is
// read one step before it is needed, so a record already published costs no
// wait.  A flag from another XCD, or none within the limits, marks the call
// for the repair pass and ends every later wait (the chain then runs on
// whatever the records hold, in bounds, and its results are overwritten).
struct Handoff {
    const uint32_t *fl;   // the head's record flags
    uint32_t *status;
    uint32_t me, spin_limit, next;
    uint64_t t_start, deadline, max_ticks;
    int cs, ce, h, l;
    bool bad;

    __device__ void init(const uint32_t *ready, int nc_max_, uint32_t *status_, uint32_t spin,
                         uint64_t max_t, uint64_t start_t, int cs_, int ce_, int h_, int l_) {
        fl = ready + (size_t)h_ * nc_max_;
        status = status_;
        me = xcc_id();
        spin_limit = spin;
        t_start = (uint64_t)wall_clock64();
        deadline = t_start + start_t;   // for the first records; then t_start + max_t
        max_ticks = max_t;
        cs = cs_;
        ce = ce_;
        h = h_;
        l = l_;
        bad = false;
        next = 0;
        if (spin_limit == 0) mark(3u, 0u, cs);   // accept nothing: the repair pass recomputes
    }
    // Marks the call for the repair pass.  The first refusal of the call also
    // leaves its details in status[1..5]: why (1 not seen in time, 2 from
    // another XCD, 3 refused by request), the flag seen, this XCD, the chunk
    // and the head.
    __device__ void mark(uint32_t why, uint32_t seen, int cc) {
        bad = true;
        if (l == 0) {
            __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (atomicCAS(status + 1, 0u, why) == 0u) {
                status[2] = seen;
                status[3] = me;
                status[4] = (uint32_t)cc;
                status[5] = (uint32_t)h;
            }
        }
    }
    __device__ uint32_t peek(int cc) const {
        return (bad || cc >= ce) ? 0u
                                 : __hip_atomic_load(fl + cc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ void accept(int cc, uint32_t x) {
        if (bad || cc >= ce) return;
        x = __builtin_amdgcn_readfirstlane(x);
        for (uint32_t it = 0; x == 0u; ++it) {
            if (it >= spin_limit || (uint64_t)wall_clock64() > deadline) break;
            __builtin_amdgcn_s_sleep(1);
            x = __builtin_amdgcn_readfirstlane(
                __hip_atomic_load(fl + cc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        }
        if (x != (REC_READY | me)) mark(x == 0u ? 1u : 2u, x, cc);
    }
    // With rings PF records deep, step c accepts chunk c + A, A = PF + 1, and
    // the records before the loop are cs .. cs + A - 1.
    // Before the first barrier: the records of chunks cs .. cs + A - 1.
    // Returns true when the workgroup must end at once: they did not come in
    // time (the intra-chunk kernel is then queued behind this one) or not from
    // this XCD.
    template <int A>
    __device__ bool begin() {
#pragma unroll 1
        for (int j = 0; j < A; ++j) accept(cs + j, peek(cs + j));
        const bool quit = bad && spin_limit != 0;
        deadline = t_start + max_ticks;
        next = peek(cs + A);
        return quit;
    }
    // Between the two barriers of step c: the record of chunk c + A.
    template <int A>
    __device__ void step(int c) {
        accept(c + A, next);
        next = peek(c + A + 1);
    }
};

// Processes local chunks [jlo, jhi) of every (sequence, head, value tile): the
// state is read from s_in (NULL = zeros) and written to s_out (NULL = not
// written).  s_out may equal s_in: each lane reads its state elements before
// it writes them, and no other lane touches them.
// With `ready` the records are still being produced by an intra-chunk kernel
// running beside this one: the prefetch wave waits for each record's flag
// (at most `spin_limit` polls each, and until `max_ticks` of the wall clock
// from the workgroup's start in all) instead of touching records, and notes in
// *status any record it could not accept.  If the first records are not there
// within `start_ticks`, the intra-chunk kernel is taken to be queued behind
// this one and the whole workgroup ends at once.  With `run_if` the launch is
// the repair pass: every workgroup ends at once unless *run_if is nonzero.
template <int NCT>
__global__ __launch_bounds__(INTER_THREADS, 1) void kda_inter_kernel(
    const int32_t *__restrict__ off, const int32_t *__restrict__ order, int pair0, int n_pairs,
    int H, int row_len, int ncr,
    const int4 *__restrict__ table, int nc_max, const uint8_t *__restrict__ recs, int jlo,
    int jhi, const uint16_t *__restrict__ v, const float *s_in, float *s_out,
    uint16_t *__restrict__ o, const uint32_t *ready, uint32_t *status, uint32_t spin_limit,
    uint64_t max_ticks, uint64_t start_ticks, const uint32_t *run_if, uint32_t *claim) {
    constexpr int NTILES = DV / (16 * NCT);   // workgroups per (sequence, head)
    constexpr int PF = ring_depth<NCT>();
    constexpr int ACC = PF + 1;   // the handoff accepts record c + ACC at step c
    constexpr int U_SLOT = 4 * NCT * 64, VT_SLOT = 16 * NCT * VTP;
    __shared__ half8 sS[4 * NCT * 64];   // S as fp16 B-fragments [channel block][column tile]
    __shared__ half8 sZ[2 * NCT * 64];   // Z as fp16 B-fragments [token block][column tile]
    // By chunk parity: U [token tile][column tile] in accumulator layout, and
    // value rows transposed, fp16 [column][token].
    __shared__ float4v sU[2 * U_SLOT];
    __shared__ __attribute__((aligned(16))) _Float16 sVt[2 * VT_SLOT];
    __shared__ int s_quit;   // overlapped order: the first records never came

    // Block id -> (pair, tile) so the value tiles of one (sequence, head) run on one XCD
    // (consecutive ids go round-robin over the 8 XCDs) and share its L2.  In the
    // overlapped order the pair comes from this XCD's pool instead (pairs, and
    // so heads, = XCD mod 8), the XCD the intra-chunk kernel produces its
    // records on.
    int lane8 = blockIdx.x & 7, rest = blockIdx.x >> 3;
    if (claim) {
        __shared__ int s_slot;
        if (threadIdx.x == 0) {
            int x, k;
            claim_item(claim, (int)gridDim.x, &x, &k);
            s_slot = k * 8 + x;
        }
        __syncthreads();
        lane8 = s_slot & 7;
        rest = s_slot >> 3;
    }
    const int tile = rest % NTILES, grp = rest / NTILES;
    const int pair = pair0 + grp * 8 + lane8;
    if (pair >= n_pairs) return;
    // The repair pass runs only when the overlapped launch marked the call.
    if (run_if && __hip_atomic_load(run_if, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u)
        return;
    // Launch position -> sequence: longest chains first for packed sequences.
    const int pos = pair / H, h = pair - pos * H;
    const int n = table ? order[pos] : pos;

    const int tid = threadIdx.x, l = tid & 63, g4 = l >> 4, i16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
    const int t = w & 3;
    const bool state_role = w < 4;
    const int vt0 = tile * NCT;

    int cs, ce;
    if (table) {
        cs = off[n];
        ce = off[n + 1];
    } else {
        cs = n * ncr;
        ce = cs + ncr;
    }
    const int first = cs, n_chunks = ce - cs;
    ce = min(ce, cs + jhi);
    cs = min(ce, cs + jlo);
    const uint8_t *rbase = recs + (size_t)h * nc_max * REC_BYTES;
    const int clast = max(cs, ce - 1);
    const size_t sbase = ((size_t)n * H + h) * DK * DV;

    // The loads are unconditional -- past the last chunk they re-read the last
    // record (in bounds, unused) -- so the compiler's wait-count tracking stays
    // exact across the loop.  Each ring slot is refilled for the chunk PF ahead.
    if (state_role) {
        // The state waves carry the chain from chunk to chunk: let them win
        // instruction issue on their SIMD over the output and prefetch waves
        // (priority 2 measured best of 0-3).
        __builtin_amdgcn_s_setprio(2);
        // State rows (channels) 32t + 16 cl + 4 g4 + e, columns 16 (vt0 + ct) + i16.
        float4v S[2][NCT];
#pragma unroll
        for (int cl = 0; cl < 2; ++cl)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    S[cl][ct][e] = s_in ? s_in[sbase + (size_t)(32 * t + 16 * cl + 4 * g4 + e) * DV +
                                               16 * (vt0 + ct) + i16]
                                        : 0.f;
        if (ready) {
            lds_barrier();   // the records of the first chunks are published (or never will be)
            if (s_quit) return;
        }
        StateOps<NCT> buf[PF];
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            const uint8_t *rec = rbase + (size_t)min(cs + j, clast) * REC_BYTES;
            load_w(buf[j], rec, t, l);
            load_kg(buf[j], rec, t, l);
        }
        lds_barrier();   // the output waves' U of the first chunk
        // Whole groups of PF chunks run without per-step conditions, so the
        // compiler's wait counts see the same load sequence on every path and
        // wait only for the ring slot in use; the last < PF chunks follow.
        int c = cs;
        for (; c + PF <= ce; c += PF) {
#pragma unroll
            for (int j = 0; j < PF; ++j)
                state_step(S, buf[j], sS, sZ, sU + ((c + j) & 1) * U_SLOT, t, l,
                           rbase + (size_t)min(c + j + PF, clast) * REC_BYTES);
        }
#pragma unroll
        for (int j = 0; j < PF - 1; ++j)
            if (c + j < ce)
                state_step(S, buf[j], sS, sZ, sU + ((c + j) & 1) * U_SLOT, t, l,
                           rbase + (size_t)min(c + j + PF, clast) * REC_BYTES);
        if (s_out) {
#pragma unroll
            for (int cl = 0; cl < 2; ++cl)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        s_out[sbase + (size_t)(32 * t + 16 * cl + 4 * g4 + e) * DV +
                              16 * (vt0 + ct) + i16] = S[cl][ct][e];
        }
    } else if (w < 8) {
        // The sequence's value rows at this lane's columns (row 16 t + l / 4 of
        // each chunk, 4 NCT columns from 16 vt0 + 4 NCT (l % 4)).
        VRows vr;
        vr.stride = (size_t)H * DV;
        vr.first = first;
        vr.len = 0;
        size_t tok0 = 0;
        if (n_chunks > 0) {
            if (table) {
                const int4 e0 = table[first], e1 = table[first + n_chunks - 1];
                tok0 = (size_t)e0.y;
                vr.len = e1.y + e1.z - e0.y;
            } else {
                tok0 = (size_t)n * row_len;
                vr.len = row_len;
            }
        }
        vr.p = v + (tok0 * H + h) * DV + 16 * vt0 + 4 * NCT * (l & 3);
        OutOps<NCT> buf[PF];
        if (ready) {
            lds_barrier();   // the records of the first chunks are published (or never will be)
            if (s_quit) return;
        }
        if (cs < ce) {
            // U of the first chunk needs its rows and T B now; the rows of the
            // second go to LDS for the first step.
            half8 T0[2];
            uint32_t V0[2 * NCT], V1[2 * NCT];
            load_v<NCT>(V0, vr, cs, t, l);
            load_v<NCT>(V1, vr, min(cs + 1, clast), t, l);
            load_tri(T0, rbase + (size_t)cs * REC_BYTES + REC_T, t, l);
#pragma unroll
            for (int j = 0; j < PF; ++j) {
                const uint8_t *rec = rbase + (size_t)min(cs + j, clast) * REC_BYTES;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    buf[j].Q[kb] = reinterpret_cast<const half8 *>(rec + REC_Q)[(t * 4 + kb) * 64 + l];
                load_tri(buf[j].H, rec + REC_H, t, l);
                load_tri(buf[j].T, rbase + (size_t)min(cs + j + 1, clast) * REC_BYTES + REC_T, t, l);
                load_v<NCT>(buf[j].V, vr, min(cs + j + 2, clast), t, l);
            }
            stage_v<NCT>(V0, sVt + (cs & 1) * VT_SLOT, t, l);
            stage_v<NCT>(V1, sVt + ((cs + 1) & 1) * VT_SLOT, t, l);
            lds_barrier();
            form_u<NCT>(T0, sVt + (cs & 1) * VT_SLOT, sU + (cs & 1) * U_SLOT, t, l);
        } else {
            lds_barrier();
        }
        int c = cs;
        for (; c + PF <= ce; c += PF) {
#pragma unroll
            for (int j = 0; j < PF; ++j) {
                const int cc = c + j;
                output_step<NCT>(buf[j], sS, sZ, sVt + ((cc + 1) & 1) * VT_SLOT,
                                 sU + ((cc + 1) & 1) * U_SLOT, sVt + (cc & 1) * VT_SLOT,
                                 chunk_at(cc, table, row_len, ncr), H, h, t, l, vt0, rbase,
                                 cc + PF, clast, vr, o);
            }
        }
#pragma unroll
        for (int j = 0; j < PF - 1; ++j) {
            const int cc = c + j;
            if (cc < ce)
                output_step<NCT>(buf[j], sS, sZ, sVt + ((cc + 1) & 1) * VT_SLOT,
                                 sU + ((cc + 1) & 1) * U_SLOT, sVt + (cc & 1) * VT_SLOT,
                                 chunk_at(cc, table, row_len, ncr), H, h, t, l, vt0, rbase,
                                 cc + PF, clast, vr, o);
        }
    } else if (ready) {
        // Handoff wave: the records come from an intra-chunk kernel running
        // beside this one, through this XCD's L2, so nothing is touched ahead.
        static_assert(L2D > 0, "the overlapped chain needs its ninth wave");
        Handoff hand;
        hand.init(ready, nc_max, status, spin_limit, max_ticks, start_ticks, cs, ce, h, l);
        const bool quit = hand.begin<ACC>();
        if (l == 0) s_quit = quit ? 1 : 0;
        lds_barrier();   // the records of the first chunks are published (or never will be)
        if (quit) return;
        lds_barrier();   // the output waves' U of the first chunk
#pragma unroll 1
        for (int c = cs; c < ce; ++c) {
            lds_barrier();
            hand.step<ACC>(c);
            lds_barrier();
        }
    } else if (L2D > 0) {
        // Prefetch wave: touches this tile's share of the record L2D chunks
        // ahead, one 4-byte load every TOUCH bytes, so that the record sits in
        // L2 when the other waves' register rings load it (the value tiles of a
        // pair share that L2).  A touch is consumed -- waited for -- L2R chunks
        // after it was issued, so this wave never stalls the chunk barriers on
        // memory.
        static_assert(REC_BYTES % TOUCH == 0 && TOUCH >= 4, "touch stride");
        constexpr int LINES = REC_BYTES / TOUCH;
#ifdef KDA_INTER_L2ALL
        constexpr int SHARE = LINES;
        const int tile0 = 0;
#else
        constexpr int SHARE = (LINES + NTILES - 1) / NTILES;
        const int tile0 = tile;
#endif
        constexpr int NLD = (SHARE + 63) / 64;
        int lofs[NLD];
#pragma unroll
        for (int i = 0; i < NLD; ++i)
            lofs[i] = min(tile0 * SHARE + min(64 * i + l, SHARE - 1), LINES - 1) * TOUCH;
        uint32_t ring[L2R][NLD];
#pragma unroll
        for (int j = 0; j < L2R; ++j)
#pragma unroll
            for (int i = 0; i < NLD; ++i) ring[j][i] = 0;
        auto touch = [&](int j, int cc) {
            lds_barrier();
            const uint8_t *rec = rbase + (size_t)min(cc + L2D, clast) * REC_BYTES;
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                asm volatile("" ::"v"(ring[j][i]));
                ring[j][i] = *reinterpret_cast<const uint32_t *>(rec + lofs[i]);
            }
            lds_barrier();
        };
        lds_barrier();   // the output waves' U of the first chunk
        int c = cs;
        for (; c + L2R <= ce; c += L2R) {
#pragma unroll
            for (int j = 0; j < L2R; ++j) touch(j, c + j);
        }
#pragma unroll
        for (int j = 0; j < L2R - 1; ++j)
            if (c + j < ce) touch(j, c + j);
#pragma unroll
        for (int j = 0; j < L2R; ++j)
#pragma unroll
            for (int i = 0; i < NLD; ++i) asm volatile("" ::"v"(ring[j][i]));
    }
}

// Zeroes n words (the overlapped prefill's status word and record flags).
__global__ __launch_bounds__(256) void kda_clear_words_kernel(uint32_t *__restrict__ p, int64_t n) {
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += step) p[i] = 0u;
}

// Workspace: [status word, 256 B][off int32 (N+1)][order int32 N][chunk table
// int4 x nc_max][record flags uint32 x H x nc_max][records], each region
// 256-byte aligned.  The status word (nonzero after an overlapped call that
// needed its repair pass) and the flags serve the overlapped prefill.
struct WsLayout {
    size_t off, order, table, status, flags, recs, total;
    int64_t nc_max;
};

static WsLayout ws_layout(int64_t total_tokens, int64_t n_seqs, int heads) {
    WsLayout L;
    L.nc_max = max_chunks(total_tokens, n_seqs, C);
    auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
    L.status = 0;
    L.off = 256;
    L.order = L.off + up((size_t)(n_seqs + 1) * 4);
    L.table = L.order + up((size_t)n_seqs * 4);
    L.flags = L.table + up((size_t)L.nc_max * 16);
    L.recs = L.flags + up((size_t)heads * L.nc_max * 4);
    L.total = L.recs + (size_t)heads * L.nc_max * REC_BYTES;
    return L;
}

// The side stream and the two events of the overlapped prefill, one set per
// device, created on first use and kept until the process ends.  The mutex
// also keeps the fork / join of one call from interleaving with another
// thread's.
struct SideStream {
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
static std::mutex g_side_mu;
static SideStream g_side[64];

static hipError_t side_stream(int dev, SideStream **out) {
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    SideStream &s = g_side[dev];
    hipError_t e;
    if (!s.stream) {
        hipStream_t st = nullptr;
        hipEvent_t f = nullptr, j = nullptr;
        if ((e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking)) != hipSuccess) return e;
        if ((e = hipEventCreateWithFlags(&f, hipEventDisableTiming)) != hipSuccess ||
            (e = hipEventCreateWithFlags(&j, hipEventDisableTiming)) != hipSuccess) {
            if (f) (void)hipEventDestroy(f);
            (void)hipStreamDestroy(st);
            return e;
        }
        s.stream = st;
        s.fork = f;
        s.join = j;
    }
    *out = &s;
    return hipSuccess;
}

}  // namespace mfma_path

bool mfma_path_supported(int dk, int dv, int chunk, bool bf16) {
    return bf16 && dk == mfma_path::DK && dv == mfma_path::DV && chunk == mfma_path::C;
}

size_t mfma_workspace_bytes(int64_t total_tokens, int64_t n_seqs, int heads, int /*chunk*/) {
    return mfma_path::ws_layout(total_tokens, n_seqs, heads).total;
}

hipError_t launch_chunk_fwd_mfma(const ChunkProblem &p) {
    using namespace mfma_path;
    const bool varlen = p.cu != nullptr;
    const int64_t total = (int64_t)p.batch * p.seqlen;
    const WsLayout L = ws_layout(total, p.n_seqs, p.heads);
    hipError_t e;
    uint8_t *ws = static_cast<uint8_t *>(p.workspace);
    int32_t *off = reinterpret_cast<int32_t *>(ws + L.off);
    int32_t *order = reinterpret_cast<int32_t *>(ws + L.order);
    int4 *table = varlen ? reinterpret_cast<int4 *>(ws + L.table) : nullptr;
    uint8_t *recs = ws + L.recs;
    const int ncr = (p.seqlen + C - 1) / C;
    const int n_pairs = p.n_seqs * p.heads;
    // One chain workgroup per CU is resident at a time (its nine waves hold
    // nearly every VGPR of a SIMD), so chains beyond the CU count wait for whole
    // earlier chains to finish.  When 16-column tiles would give more chains
    // than CUs, 32-column tiles halve their number; each step is then slower
    // (about 1.4 against 1.2 us per chunk), but twice as many (sequence, head)
    // pairs advance at once.
    int dev = 0, n_cu = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev)) !=
        hipSuccess)
        return e;
    const bool wide = (int64_t)n_pairs * (DV / 16) > n_cu;
    // A launch holds at most 2^32 threads, so the chains go out in launches of
    // at most INTER_MAX_PAIRS (sequence, head) pairs (a multiple of 8, so the
    // XCD placement is the same in every launch).
    static_assert((uint64_t)INTER_MAX_PAIRS * (DV / 16) * INTER_THREADS <= 0xFFFFFFFFull, "");
    uint16_t *o = static_cast<uint16_t *>(p.o);

    // Status region: [0] repair needed, [1..5] the first refusal, [8..15] and
    // [16..23] the intra-chunk and chain kernels' XCD pool counters.
    uint32_t *status = reinterpret_cast<uint32_t *>(ws + L.status);
    uint32_t *flags = reinterpret_cast<uint32_t *>(ws + L.flags);

    auto intra = [&](hipStream_t st, int jlo, int jn, int grid, uint32_t *ready, uint32_t *claim) {
        auto kern = p.gate == Gate::PerChannel ? kda_intra_kernel<Gate::PerChannel>
                    : p.gate == Gate::Scalar   ? kda_intra_scalar_kernel<true>
                                               : kda_intra_scalar_kernel<false>;
        hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, st,
                           static_cast<const uint16_t *>(p.q), static_cast<const uint16_t *>(p.k),
                           p.g, p.beta, p.scale,
                           p.form.flags(), p.form.eps, p.heads, p.seqlen, ncr, table,
                           off + p.n_seqs, (int)L.nc_max, jlo, jn, recs, ready, claim);
        return hipGetLastError();
    };
    // The chunk chain over local chunks [jlo, jhi), with 32-column tiles when
    // `wide_tiles`.  `ready` etc.: the overlapped launch and its repair pass.
    auto inter = [&](int nct, int jlo, int jhi, const float *s_in, float *s_out,
                     const uint32_t *ready, uint32_t spin_limit, uint64_t max_ticks,
                     uint64_t start_ticks, const uint32_t *run_if, uint32_t *claim) {
        auto kern = nct == 2 ? kda_inter_kernel<2> : kda_inter_kernel<1>;
        const int n_tiles = DV / (16 * nct);
        hipError_t err = hipSuccess;
        for (int p0 = 0; p0 < n_pairs && err == hipSuccess; p0 += INTER_MAX_PAIRS) {
            const int np = min(INTER_MAX_PAIRS, n_pairs - p0);
            hipLaunchKernelGGL(kern, dim3((np + 7) / 8 * 8 * n_tiles), dim3(INTER_THREADS), 0,
                               p.stream, off, order, p0, n_pairs, p.heads, p.seqlen, ncr, table,
                               (int)L.nc_max, recs, jlo, jhi, static_cast<const uint16_t *>(p.v),
                               s_in, s_out, o, ready, status, spin_limit, max_ticks,
                               start_ticks, run_if, claim);
            err = hipGetLastError();
        }
        return err;
    };
    auto serial_inter = [&](int jlo, int jhi, const float *s_in, float *s_out) {
        return inter(wide ? 2 : 1, jlo, jhi, s_in, s_out, nullptr, 0u, 0, 0, nullptr, nullptr);
    };

    if (varlen || total == 0) {
        // Packed sequences: chunk table, all intra-chunk work, then the chunk chain.
        if (varlen) {
            if (!launch_fits((int64_t)p.heads * L.nc_max, 256)) return hipErrorInvalidConfiguration;
            hipLaunchKernelGGL(kda_chunk_index_kernel, dim3(1), dim3(1024), 0, p.stream, p.cu,
                               p.n_seqs, (int)total, off, order, table);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            if (L.nc_max > 0 &&
                (e = intra(p.stream, 0, 0, p.heads * (int)L.nc_max, nullptr, nullptr)) != hipSuccess)
                return e;
        }
        return serial_inter(0, INT32_MAX / 2, p.s0, p.s_final);
    }

    if (!launch_fits((int64_t)p.heads * p.batch * ncr, 256)) return hipErrorInvalidConfiguration;
    // Overlapped order, for equal rows of at least OVERLAP_MIN_CHUNKS chunks
    // whose chains fit on half the CUs as 32-column tiles: the chain kernel
    // starts at once on the caller's stream and reads each record as the
    // intra-chunk kernel, on a side stream, publishes it (both kernels take
    // the heads of their own XCD, h mod 8, so H must be a multiple of 8).  The
    // intra-chunk work then shares the device with the chains instead of
    // preceding them, and the records are read from L2 instead of HBM.  Left
    // out: calls that cannot create a stream (the no-allocation entry point,
    // stream capture), an initial state that the chain overwrites (the repair
    // pass needs it), and a mode set to serial.  Measured at H = 32: 7% faster
    // from 32768 tokens per row up, even at 8192, 10% slower at 4096 (the
    // side stream's fork and join and the extra launches cost about 30 us).
    // Side by side, the intra-chunk work has about half the CUs and bounds the
    // call, so the overlap pays only while that work is lighter than the chain:
    // with the logit gate and the in-kernel L2 norms it is not (4.43 against
    // 4.36 ms at T = 131072), and those forms keep the serial order.
    constexpr int OVERLAP_MIN_CHUNKS = 128;
    const int mode = prefill_overlap_mode();
    const bool light_intra = (p.form.flags() & (kFormGateLogit | kFormL2Norm)) == 0;
    bool overlap = mode != 0 && p.allow_overlap && light_intra && p.heads % 8 == 0 &&
                   (int64_t)n_pairs * (DV / 32) * 2 <= n_cu &&
                   ncr >= OVERLAP_MIN_CHUNKS && !(p.s_final && p.s_final == p.s0);
    if (overlap) {
        // The side stream is the current device's: a caller's stream of another
        // device keeps the serial order (its kernels run on the stream's device).
        int sdev = dev;
        if (p.stream && (e = hipStreamGetDevice(p.stream, &sdev)) != hipSuccess) return e;
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        if ((e = hipStreamIsCapturing(p.stream, &cap)) != hipSuccess) return e;
        overlap = sdev == dev && cap == hipStreamCaptureStatusNone;
    }
    if (!overlap) {
        // Serial order: all intra-chunk work, then the chunk chain, on the caller's stream.
        if ((e = intra(p.stream, 0, ncr, p.heads * p.batch * ncr, nullptr, nullptr)) != hipSuccess)
            return e;
        return serial_inter(0, ncr, p.s0, p.s_final);
    }
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStream *side = nullptr;
    if ((e = side_stream(dev, &side)) != hipSuccess) return e;
    int khz = 0;
    if ((e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev)) != hipSuccess)
        return e;
    // A chain waits at most 10 ms plus 20 us per chunk in all (a chunk row of
    // the intra-chunk kernel takes about 2 us beside the chains), then stops
    // waiting and leaves the call to the repair pass.
    const uint64_t max_ticks = (uint64_t)((10.0 + 0.02 * ncr) * (double)(khz > 0 ? khz : 100000));
    const uint32_t spin_limit = mode == 2 ? 0u : 0xFFFFFFFFu;
    // Clear the status words (repair flag, refusal details, work counters) and
    // every record flag.
    const int64_t n_flags = (int64_t)(L.recs - L.flags) / 4;
    const int64_t clear_blocks = (n_flags + 255) / 256;
    hipLaunchKernelGGL(kda_clear_words_kernel, dim3(1), dim3(256), 0, p.stream, status, (int64_t)64);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(kda_clear_words_kernel,
                       dim3((unsigned)(clear_blocks < 1024 ? clear_blocks : 1024)), dim3(256), 0,
                       p.stream, flags, n_flags);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // The chain is enqueued first, so that its workgroups find whole CUs free
    // (enqueued second, they wait for the intra-chunk workgroups to drain a
    // CU: 3% slower).  Should the side stream share a hardware queue with the
    // caller's stream (a process has a few, and streams beyond that share
    // them), the intra-chunk kernel cannot start before the chain ends: each
    // chain workgroup then gives up within START_US and the repair pass runs.
    constexpr double START_US = 250.0;
    const uint64_t start_ticks =
        mode == 3 ? 0 : (uint64_t)(START_US * 1e-3 * (double)(khz > 0 ? khz : 100000));
    if ((e = hipEventRecord(side->fork, p.stream)) != hipSuccess) return e;
    if ((e = inter(2, 0, ncr, p.s0, p.s_final, flags, spin_limit, max_ticks, start_ticks, nullptr,
                   status + 16)) != hipSuccess)
        return e;
    if ((e = hipStreamWaitEvent(side->stream, side->fork, 0)) != hipSuccess) return e;
    if ((e = intra(side->stream, 0, ncr, p.heads * p.batch * ncr, flags, status + 8)) !=
        hipSuccess)
        return e;
    if ((e = hipEventRecord(side->join, side->stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(p.stream, side->join, 0)) != hipSuccess) return e;
    // Repair pass: reruns the chain in the serial order if any record was not accepted.
    return inter(wide ? 2 : 1, 0, ncr, p.s0, p.s_final, nullptr, 0u, 0, 0, status, nullptr);
}

}  // namespace kda
