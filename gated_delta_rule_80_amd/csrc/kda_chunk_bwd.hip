// kda_chunk_bwd.hip -- gradients of the chunkwise KDA prefill in fp32, for
// fp32 storage and d_k = d_v = d in {16, 32, 64, 128}; and, sharing the prep
// kernel's chunk factors, the fp32 prefill itself at d = 128 (near the end).
//
// The pages derive no gradients.  These kernels reverse the chunk algebra of
// "Understanding Kimi Delta Attention" (A. Flores), sections "The triangular
// system" and "Putting the chunks together" (written here with A = -A_page,
// so T = (I + A)^{-1}):
//   R = T Diag(beta) L,  U = T Diag(beta) V,  Z = U - R S,
//   O = Qbar S + H Z,    S' = Diag(e^{G_C}) S + Kbar^T Z,
// one step at a time, last step first.  With dS' the gradient reaching the
// end of a chunk:
//   dZ = Kbar dS' + H^T dO,   dS = Diag(e^{G_C}) dS' + Qbar^T dO - R^T dZ,
//   dR = -dZ S^T,  dT = dZ (BV)^T + dR (BL)^T,  dA = T^T dT T^T (strictly lower),
// and the decay-weighted products behind A and H hand their gradients to k, q
// and the cumulative log-decay G, whose reverse cumulative sum is dg.
//
// Three kernels.  Every per-chunk factor that does not depend on the value
// columns (K~, T, H, R, Kbar, Qbar, e^{G_C}) comes from a prep kernel, one
// workgroup per (chunk, head), into the workspace.  Only S and dS are carried
// from chunk to chunk, and each of their value columns evolves on its own (Z
// and dZ are column-wise too), so the chain kernel runs one workgroup per
// (sequence, head, 16 value columns) and streams those factors: a forward
// sweep stores each chunk's start state and Z, a reverse sweep stores each
// chunk's end-state gradient dS' and dZ and leaves dS_0.  Every other
// gradient is a function of one chunk's inputs and the stored quantities, so
// the gradient kernel runs one workgroup per (chunk, head), all in parallel.
// fp32 on the vector ALUs, decay factors as e^{G_i - G_j} with exponents <= 0
// (and e^{G_i}, e^{G_C - G_i} <= 1), so any finite log-decay is in range.
//
// At d = 128, C = 16 the contractions run on fp32 MFMA (16 x 16 x 4), so the
// arithmetic stays fp32: the chain kernel keeps its state tiles in
// accumulators and has a fifth wave that prefetches each chunk's operands
// into L2 a few steps ahead; it stores S only at even chunks and dS' only at
// odd chunks and the last one, and the gradient kernel rebuilds the other
// with one chunk step from its neighbour's.  The decay-weighted sums of the
// prep kernel (K~, H) and of the gradient kernel (P1-P4) become products
// between row scalings, e^{G_i - G_j} = e^{G_i - G_r} e^{G_r - G_j}, where
// every channel decays by at most 40 over the chunk (both factors then stay
// within e^{+-40}); elsewhere the pairwise factors above are kept.  T is the
// nilpotent product (I - N)(I + N^2)(I + N^4)(I + N^8), N = Diag(beta) K~.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace bwd {

constexpr int THREADS = 256;   // prep kernel
constexpr int CT = 512;        // chain kernel: two waves per SIMD
constexpr int GT = 512;        // gradient kernel
constexpr int TV = 16;         // value columns per chain workgroup

// ---- workspace ------------------------------------------------------------------
// Per (chunk slot, head), fp32, row-major, one region per quantity:
//   S at the chunk start and dS' at the chunk end [d][d] (at d = 128, C = 16
//   only S of even and dS' of odd and last chunks are written); Z, dZ, R,
//   Kbar, Qbar [C][d]; T, K~, H [C][C]; e^{G_C} [d].
__host__ __device__ inline size_t n_slots(int64_t total_tokens, int n_seqs, int chunk) {
    return (size_t)(total_tokens / chunk + n_seqs + 1);
}
__host__ __device__ inline size_t ws_floats_per_slot(int d, int C) {
    return 2 * (size_t)d * d + 5 * (size_t)C * d + 3 * (size_t)C * C + d;
}
struct Ws {
    float *S, *dS, *Z, *dZ, *R, *Kb, *Qb, *T, *Kt, *Hm, *gC;
};
__host__ __device__ inline Ws ws_layout(float *base, size_t slots, int heads, int d, int C) {
    const size_t n = slots * heads, dd = n * d * d, cd = n * C * d, cc = n * C * C;
    Ws w;
    w.S = base;
    w.dS = w.S + dd;
    w.Z = w.dS + dd;
    w.dZ = w.Z + cd;
    w.R = w.dZ + cd;
    w.Kb = w.R + cd;
    w.Qb = w.Kb + cd;
    w.T = w.Qb + cd;
    w.Kt = w.T + cc;
    w.Hm = w.Kt + cc;
    w.gC = w.Hm + cc;
    return w;
}

// First chunk slot of sequence n: floor(start / C) + n.  Strictly increasing in
// n, and a sequence's slots stay below the next one's first slot.
__device__ __forceinline__ int chunk_base(int ts, int n, int C) { return ts / C + n; }

__device__ __forceinline__ void seq_range(const int32_t *cu, int row_len, int n, int &ts,
                                          int &te) {
    if (cu) {
        const int T = row_len;   // clamped: a malformed cu_seqlens stays inside [0, T)
        ts = min(T, max(0, cu[n]));
        te = min(T, max(ts, cu[n + 1]));
    } else {
        ts = n * row_len;
        te = ts + row_len;
    }
}

// The chunk held by slot `slot`: its first token and length, its index c
// within its sequence and the sequence's end te.  False for a gap slot
// (uniform over a workgroup).
template <int C>
__device__ __forceinline__ bool slot_chunk(const int32_t *cu, int row_len, int n_seqs, int slot,
                                           int &t0, int &len, int &c, int &te) {
    // the sequence owning the slot: the last n with chunk_base(n) <= slot
    int lo = 0, hi = n_seqs - 1, ts;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        seq_range(cu, row_len, mid, ts, te);
        if (chunk_base(ts, mid, C) <= slot) lo = mid;
        else hi = mid - 1;
    }
    seq_range(cu, row_len, lo, ts, te);
    c = slot - chunk_base(ts, lo, C);
    if (c >= (te - ts + C - 1) / C) return false;
    t0 = ts + c * C;
    len = min(C, te - t0);
    return true;
}
template <int C>
__device__ __forceinline__ bool slot_chunk(const int32_t *cu, int row_len, int n_seqs, int slot,
                                           int &t0, int &len) {
    int c, te;
    return slot_chunk<C>(cu, row_len, n_seqs, slot, t0, len, c, te);
}

// ---- shared chunk steps (one workgroup, THREADS threads, operands in LDS) ----------
// [C][d] operands sit in LDS with row stride d + 1, so that lanes walking the
// rows of one column hit distinct banks.
__host__ __device__ inline int row_stride(int d) { return d + 1; }

// A [rows][d] block (rows * d <= 2048) moves from global memory to LDS in two
// steps: fetch_rows issues 16-byte loads into registers, commit_rows stores
// them, so a chunk's loads can be in flight while the previous chunk computes.
constexpr int MAX_BLOCK = 2048;   // floats in one fetched [rows][d] block
template <int NT> struct Rows {
    static constexpr int NV = (MAX_BLOCK / 4 + NT - 1) / NT;   // float4 per thread
    float4 x[NV];
};
// Four consecutive elements as fp32 (bf16 widens exactly).
__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ float4 ld4(const bf16_t *p) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
// Row i (< len) of the block starts at src + i * pitch; rows >= len read as 0.
template <int NT, typename E>
__device__ __forceinline__ void fetch_rows(Rows<NT> &r, const E *src, size_t pitch, int rows,
                                           int len, int d, int tid) {
#pragma unroll
    for (int u = 0; u < Rows<NT>::NV; ++u) {
        const int e = 4 * (tid + u * NT), i = e / d;
        float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i < rows && i < len)
            val = ld4(src + (size_t)i * pitch + (e - i * d));
        r.x[u] = val;
    }
}
template <int NT>
__device__ __forceinline__ void commit_rows(float *dst, const Rows<NT> &r, int rows, int d,
                                            int tid) {
    const int dp = row_stride(d);
#pragma unroll
    for (int u = 0; u < Rows<NT>::NV; ++u) {
        const int e = 4 * (tid + u * NT), i = e / d;
        if (i < rows) {
            float *p = dst + i * dp + (e - i * d);
            p[0] = r.x[u].x;
            p[1] = r.x[u].y;
            p[2] = r.x[u].z;
            p[3] = r.x[u].w;
        }
    }
}
// In place: G[i][c] <- sum_{r <= i} g[r][c] (padding rows add zero).
template <int C, int NT> __device__ __forceinline__ void cumsum_rows(float *G, int d, int tid) {
    const int dp = row_stride(d);
    for (int c = tid; c < d; c += NT) {
        float run = 0.f;
#pragma unroll 4
        for (int i = 0; i < C; ++i) {
            run += G[i * dp + c];
            G[i * dp + c] = run;
        }
    }
}
// Pairwise decay-weighted products, with E_ijc = e^{G_ic - G_jc} (exponent <= 0):
//   K~_ij = sum_c k_ic k_jc E_ijc (j < i, else 0),
//   H_ij  = s sum_c q_ic k_jc E_ijc (j <= i, else 0; only when Hm is given).
template <int C>
__device__ __forceinline__ void pair_products(float *Kt, float *Hm, const float *k,
                                              const float *q, const float *G, float scale, int d,
                                              int tid) {
    const int dp = row_stride(d);
    for (int e = tid; e < C * C; e += THREADS) {
        const int i = e / C, j = e - i * C;
        float a = 0.f, hh = 0.f;
        if (j <= i) {
            if (Hm) {
#pragma unroll 8
                for (int c = 0; c < d; ++c) {
                    const float E = fast_exp(G[i * dp + c] - G[j * dp + c]) * k[j * dp + c];
                    a += k[i * dp + c] * E;
                    hh += q[i * dp + c] * E;
                }
            } else if (j < i) {
#pragma unroll 8
                for (int c = 0; c < d; ++c)
                    a += k[i * dp + c] * fast_exp(G[i * dp + c] - G[j * dp + c]) * k[j * dp + c];
            }
        }
        Kt[e] = (j < i) ? a : 0.f;
        if (Hm) Hm[e] = scale * hh;
    }
}
// T = (I + Diag(beta) K~)^{-1}, unit lower triangular.  Thread j < C solves
// column j by forward substitution, keeping the column in registers:
//   T_ij = delta_ij - beta_i sum_{j <= m < i} K~_im T_mj.
template <int C>
__device__ __forceinline__ void solve_T(float *T, const float *Kt, const float *b, int tid) {
    if (tid < C) {
        const int j = tid;
        float col[C];
#pragma unroll
        for (int i = 0; i < C; ++i) {
            float s = 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) s += Kt[i * C + m] * col[m];
            col[i] = (i < j) ? 0.f : ((i == j) ? 1.f : -b[i] * s);
        }
#pragma unroll
        for (int i = 0; i < C; ++i) T[i * C + j] = col[i];
    }
}

// One fp32 MFMA step, 16 x 16 x 4: lane l gives A[l % 16][l / 16] and
// B[l / 16][l % 16]; accumulator element e is D[4 (l / 16) + e][l % 16].
__device__ __forceinline__ float4v mfma4(float a, float b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4v as4v(float4 x) { return float4v{x.x, x.y, x.z, x.w}; }

// ---- prep kernel ----------------------------------------------------------------
struct PrepLds {
    int k, G, q, L, beta, Kt, T, Hm, total;
};
__host__ __device__ inline PrepLds prep_layout(int d, int C) {
    PrepLds L;
    int o = 0;
    const int cd = C * row_stride(d), cc = C * C;
    L.k = o; o += cd;
    L.G = o; o += cd;
    L.q = o; o += cd;
    L.L = o; o += cd;
    L.beta = o; o += C;
    L.Kt = o; o += cc;
    L.T = o; o += cc;
    L.Hm = o; o += cc;
    L.total = o;
    return L;
}

// One chunk of one head: K~, T, H, R = T Diag(beta) L, Kbar, Qbar and e^{G_C}
// into the workspace (padding rows come out zero, T's padding block identity).
// GL is the layout of g (Gate): per channel [T, H, d], one log-decay per
// (token, head) [T, H] broadcast over the channels, or none (g unused).
// `form` (fp32 prefill only; 0 for the backward) applies the layer's input
// steps as the rows are read: log a = log sigmoid(g), beta = sigmoid(beta)
// and q, k divided by sqrt(sum of squares + eps), on the valid rows.
template <int C, int D, typename In, int GL = 0>
__global__ __launch_bounds__(THREADS) void kda_bwd_prep_kernel(
    const In *__restrict__ q, const In *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, float scale, int H, int row_len,
    const int32_t *__restrict__ cu, int n_seqs, Ws ws, int form = 0, float eps = 0.f) {
    constexpr int d = D;
    extern __shared__ float sm[];
    const PrepLds L = prep_layout(d, C);
    float *sk = sm + L.k, *sG = sm + L.G, *sq = sm + L.q, *sL = sm + L.L, *sb = sm + L.beta;
    float *sKt = sm + L.Kt, *sT = sm + L.T, *sHm = sm + L.Hm;
    const int slot = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H, tid = threadIdx.x;
    int t0, len;
    if (!slot_chunk<C>(cu, row_len, n_seqs, slot, t0, len)) return;
    const int dp = row_stride(d), cd = C * d, cc = C * C;
    const size_t wslot = (size_t)slot * H + h;
    {
        const size_t off = ((size_t)t0 * H + h) * d, pitch = (size_t)H * d;
        Rows<THREADS> rk, rg, rq;
        fetch_rows(rk, k + off, pitch, C, len, d, tid);
        if constexpr (GL == 0) {
            fetch_rows(rg, g + off, pitch, C, len, d, tid);
        } else {
#pragma unroll
            for (int u = 0; u < Rows<THREADS>::NV; ++u) {
                const int i = 4 * (tid + u * THREADS) / d;
                const float gi = (GL == 1 && i < C && i < len) ? g[(size_t)(t0 + i) * H + h] : 0.f;
                rg.x[u] = make_float4(gi, gi, gi, gi);
            }
        }
        fetch_rows(rq, q + off, pitch, C, len, d, tid);
        float rb = tid < len ? beta[(size_t)(t0 + tid) * H + h] : 0.f;
        if (GL != 2 && (form & kFormGateLogit)) {
#pragma unroll
            for (int u = 0; u < Rows<THREADS>::NV; ++u)
                if (4 * (tid + u * THREADS) / d < len) {
                    float4 &x = rg.x[u];
                    x = make_float4(log_sigmoid(x.x), log_sigmoid(x.y), log_sigmoid(x.z),
                                    log_sigmoid(x.w));
                }
        }
        if ((form & kFormBetaLogit) && tid < len) rb = sigmoid(rb);
        commit_rows(sk, rk, C, d, tid);
        commit_rows(sG, rg, C, d, tid);
        commit_rows(sq, rq, C, d, tid);
        if (tid < C) sb[tid] = rb;
    }
    __syncthreads();
    if (form & kFormL2Norm) {
        // one k or q row per THREADS / (2 C) lanes of a wave, reduced by shuffles
        constexpr int LPR = THREADS / (2 * C);
        static_assert(LPR <= 64 && 64 % LPR == 0 && D % LPR == 0, "a row within one wave");
        const int x = tid / LPR, part = tid % LPR;
        float *row = (x < C ? sk : sq) + (x % C) * dp;
        float ss = 0.f;
        for (int c2 = part; c2 < d; c2 += LPR) ss += row[c2] * row[c2];
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
        const float inv = 1.f / sqrtf(ss + eps);
        for (int c2 = part; c2 < d; c2 += LPR) row[c2] *= inv;
    }
    cumsum_rows<C, THREADS>(sG, d, tid);
    __syncthreads();
    bool products = false;   // K~ and H formed on MFMA
    if constexpr (C == 16 && D == 128) {
        // With row r = 7 of the cumulative decays as reference,
        // e^{G_i - G_j} = e^{G_i - G_r} e^{G_r - G_j} in each channel, so
        //   K~ = (k e^{G - G_r}) (k e^{G_r - G})^T,  H = s (q e^{G - G_r}) (k e^{G_r - G})^T
        // are plain products over the channels (then masked to j < i and
        // j <= i).  Every channel must decay by at most 40 over the chunk so
        // that both factors stay within e^{+-40}; else the pairwise factors.
        // Wave w takes channels 32w .. 32w+31, channel 32w + 4s + l/16 in step
        // s from lane l (row l % 16 for both operands); the four waves' parts
        // meet in L's storage, written only afterwards.
        static_assert(THREADS == C * C, "one K~ and H entry per thread");
        const int wide = tid < d && !(sG[tid] - sG[(C - 1) * dp + tid] <= 40.f);
        if (!__syncthreads_or(wide)) {
            products = true;
            const int l = tid & 63, g4 = l >> 4, i16 = l & 15, w = tid >> 6;
            float4v ak = {0.f, 0.f, 0.f, 0.f}, ah = ak;
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2) {
                const int c2 = 32 * w + 4 * s2 + g4, a = i16 * dp + c2;
                const float Gr = sG[7 * dp + c2], G = sG[a], kk = sk[a];
                const float up = fast_exp(G - Gr), dn = kk * fast_exp(Gr - G);
                ak = mfma4(kk * up, dn, ak);
                ah = mfma4(sq[a] * up, dn, ah);
            }
            // accumulator element e: row i = 4 (l/16) + e, column j = l % 16
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sL[w * 2 * cc + (4 * g4 + e) * C + i16] = ak[e];
                sL[w * 2 * cc + cc + (4 * g4 + e) * C + i16] = ah[e];
            }
            __syncthreads();
            {
                const int e = tid, i = e / C, j = e - i * C;   // THREADS == C * C
                float a = 0.f, hh = 0.f;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    a += sL[u * 2 * cc + e];
                    hh += sL[u * 2 * cc + cc + e];
                }
                sKt[e] = j < i ? a : 0.f;
                sHm[e] = j <= i ? scale * hh : 0.f;
            }
            __syncthreads();
        }
    }
    for (int e = tid; e < cd; e += THREADS) {
        const int i = e / d, c2 = e - i * d, a = i * dp + c2;
        const float kk = sk[a], G = sG[a];
        const float eG = fast_exp(G);
        sL[a] = kk * eG;
        ws.Kb[wslot * cd + e] = kk * fast_exp(sG[(C - 1) * dp + c2] - G);
        ws.Qb[wslot * cd + e] = scale * sq[a] * eG;
    }
    for (int c2 = tid; c2 < d; c2 += THREADS) ws.gC[wslot * d + c2] = fast_exp(sG[(C - 1) * dp + c2]);
    if (!products) pair_products<C>(sKt, sHm, sk, sq, sG, scale, d, tid);
    __syncthreads();
    if constexpr (C == 16 && D == 128) {
        // T = (I + N)^{-1} with N = Diag(beta) K~ strictly lower, so N^16 = 0
        // and T = (I - N)(I + N^2)(I + N^4)(I + N^8), on fp32 MFMA in wave 0.
        // A matrix M is held as lane l's element e = M[4 (l/16) + e][l % 16];
        // with token 4 (l/16) + s as the reduction index of step s, a product
        // over held P and Q gives P^T Q, held.  Every factor is a polynomial
        // in N, so each one used on the left is also kept transposed.
        if (tid < 64) {
            const int g4 = tid >> 4, i16 = tid & 15;
            float4v n, nt;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g4 + e;
                n[e] = sb[r] * sKt[r * C + i16];     // N[r][l % 16]
                nt[e] = sb[i16] * sKt[i16 * C + r];  // N^T[r][l % 16]
            }
            auto tmul = [](const float4v &p, const float4v &q) {   // P^T Q
                float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) acc = mfma4(p[s2], q[s2], acc);
                return acc;
            };
            auto eye = [&](const float4v &m, float sign) {   // I + sign M
                float4v x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = sign * m[e] + (4 * g4 + e == i16 ? 1.f : 0.f);
                return x;
            };
            const float4v n2 = tmul(nt, n), n2t = tmul(n, nt);
            const float4v n4 = tmul(n2t, n2), n4t = tmul(n2, n2t);
            const float4v n8 = tmul(n4t, n4);
            const float4v imnt = eye(nt, -1.f), ipn2 = eye(n2, 1.f), ipn4 = eye(n4, 1.f);
            const float4v p1t = tmul(ipn2, imnt);                      // ((I - N)(I + N^2))^T
            const float4v p2t = tmul(ipn4, p1t);                       // (P1 (I + N^4))^T
            const float4v t = tmul(p2t, eye(n8, 1.f));                 // P2 (I + N^8)
#pragma unroll
            for (int e = 0; e < 4; ++e) sT[(4 * g4 + e) * C + i16] = t[e];
        }
    } else {
        solve_T<C>(sT, sKt, sb, tid);
    }
    __syncthreads();
    if constexpr (C == 16 && D == 128) {
        // R = T Diag(beta) L on fp32 MFMA: wave w takes channel tiles 2w and
        // 2w + 1, token 4s + l/16 in step s (T is zero above its diagonal).
        const int l = tid & 63, g4 = l >> 4, i16 = l & 15, w = tid >> 6;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int c0 = 16 * (2 * w + t);
            float4v r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const int j = 4 * s2 + g4;
                r = mfma4(sT[i16 * C + j] * sb[j], sL[j * dp + c0 + i16], r);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) ws.R[wslot * cd + (4 * g4 + e) * d + c0 + i16] = r[e];
        }
    } else {
        for (int e = tid; e < cd; e += THREADS) {
            const int i = e / d, c2 = e - i * d;
            float r = 0.f;
            for (int j = 0; j <= i; ++j) r += sT[i * C + j] * sb[j] * sL[j * dp + c2];
            ws.R[wslot * cd + e] = r;
        }
    }
    for (int e = tid; e < cc; e += THREADS) {
        ws.T[wslot * cc + e] = sT[e];
        ws.Kt[wslot * cc + e] = sKt[e];
        ws.Hm[wslot * cc + e] = sHm[e];
    }
}

// ---- chain kernel ---------------------------------------------------------------
struct ChainLds {
    int R, Kb, Qb, T, Hm, beta, gC, vt, zt, A, total;
};
__host__ __device__ inline ChainLds chain_layout(int d, int C) {
    ChainLds L;
    int o = 0;
    const int cd = C * row_stride(d), cc = C * C, ct = C * TV, dt = d * TV;
    L.R = o; o += cd;
    L.Kb = o; o += cd;
    L.Qb = o; o += cd;
    L.T = o; o += cc;
    L.Hm = o; o += cc;
    L.beta = o; o += C;
    L.gC = o; o += d;
    L.vt = o; o += ct;   // v tile (forward sweep) or dO tile (reverse sweep)
    L.zt = o; o += ct;   // Z tile or dZ tile
    L.A = o; o += dt;    // S tile or dS tile
    L.total = o;
    return L;
}

template <int C, int D, typename In>
__global__ __launch_bounds__(CT) void kda_bwd_chain_kernel(
    const In *__restrict__ v, const float *__restrict__ beta, int H, int row_len,
    const int32_t *__restrict__ cu, int n_pairs, const float *__restrict__ s0,
    const float *__restrict__ dfinal, const In *__restrict__ dout, float *__restrict__ ds0,
    Ws ws) {
    constexpr int d = D;
    constexpr int NCC = (C * C + CT - 1) / CT;       // T / H entries per thread
    constexpr int NVT = (C * TV + CT - 1) / CT;      // v or dO tile entries per thread
    constexpr int RS = CT / TV, RPT = (D + RS - 1) / RS;   // state rows: stride, per thread
    constexpr int ZS = (C * TV < CT) ? CT / (C * TV) : 1;  // lanes sharing one Z / dZ entry
    static_assert(ZS == 1 || ZS == 2, "Z entries are split over at most a lane pair");
    extern __shared__ float sm[];
    const ChainLds L = chain_layout(d, C);
    float *sR = sm + L.R, *sKb = sm + L.Kb, *sQb = sm + L.Qb, *sT = sm + L.T, *sHm = sm + L.Hm;
    float *sb = sm + L.beta, *sgC = sm + L.gC, *svt = sm + L.vt, *szt = sm + L.zt, *sA = sm + L.A;

    // Block id -> (pair, value tile) with the tiles of a pair on one XCD
    // (consecutive ids go round-robin over the 8 XCDs), so they share its L2.
    const int nt = d / TV;
    const int lane8 = blockIdx.x & 7, rest = blockIdx.x >> 3;
    const int tile = rest % nt, pid = (rest / nt) * 8 + lane8;
    if (pid >= n_pairs) return;
    const int n = pid / H, h = pid - n * H;
    const int v0 = tile * TV, tid = threadIdx.x;
    const int dd = d * d, dt = d * TV, ct = C * TV, cd = C * d, dp = row_stride(d);
    const int jc = tid % TV, rb0 = tid / TV;   // this thread's column and first row in S updates
    int ts, te;
    seq_range(cu, row_len, n, ts, te);
    const size_t pair = (size_t)n * H + h;
    const int nck = (te - ts + C - 1) / C;
    const int base = chunk_base(ts, n, C);

    // One chunk's factors and a 16-column tile of v (forward) or dO (reverse),
    // fetched into registers a chunk ahead of their use.
    Rows<CT> rR, rKb, rQb;
    float rT[NCC], rH[NCC], rv[NVT], rb = 0.f, rg = 0.f;
    auto fetch_chunk = [&](int c, bool reverse) {
        const int t0 = ts + c * C, len = min(C, te - t0);
        const size_t w = (size_t)(base + c) * H + h;
        fetch_rows(rR, ws.R + w * cd, d, C, C, d, tid);
        fetch_rows(rKb, ws.Kb + w * cd, d, C, C, d, tid);
        if (reverse) fetch_rows(rQb, ws.Qb + w * cd, d, C, C, d, tid);
#pragma unroll
        for (int u = 0; u < NCC; ++u) {
            const int e = tid + u * CT;
            if (e < C * C) {
                rT[u] = ws.T[w * C * C + e];
                if (reverse) rH[u] = ws.Hm[w * C * C + e];
            }
        }
        const size_t off = ((size_t)t0 * H + h) * d, pitch = (size_t)H * d;
        const In *src = reverse ? dout : v;
#pragma unroll
        for (int u = 0; u < NVT; ++u) {
            const int e = tid + u * CT, i = e / TV;
            rv[u] = (i < C && i < len) ? io<In>::load(src, off + (size_t)i * pitch + v0 + (e - i * TV))
                                       : 0.f;
        }
        if (tid < C) rb = tid < len ? beta[(size_t)(t0 + tid) * H + h] : 0.f;
        if (tid < d) rg = ws.gC[w * d + tid];
    };
    // The fetched chunk into LDS, then the next chunk's fetch is issued.
    auto commit_chunk = [&](bool reverse, int next) {
        commit_rows(sR, rR, C, d, tid);
        commit_rows(sKb, rKb, C, d, tid);
        if (reverse) commit_rows(sQb, rQb, C, d, tid);
#pragma unroll
        for (int u = 0; u < NCC; ++u) {
            const int e = tid + u * CT;
            if (e < C * C) {
                sT[e] = rT[u];
                if (reverse) sHm[e] = rH[u];
            }
        }
#pragma unroll
        for (int u = 0; u < NVT; ++u)
            if (tid + u * CT < C * TV) svt[tid + u * CT] = rv[u];
        if (tid < C) sb[tid] = rb;
        if (tid < d) sgC[tid] = rg;
        __syncthreads();
        if (next >= 0) fetch_chunk(next, reverse);
    };

    // ---- forward sweep: S at each chunk start, and Z --------------------------
    for (int e = tid; e < dt; e += CT) {
        const int r = e / TV;
        sA[e] = s0 ? s0[pair * dd + (size_t)r * d + v0 + (e - r * TV)] : 0.f;
    }
    if (nck > 0) fetch_chunk(0, false);
    __syncthreads();
    for (int c = 0; c < nck; ++c) {
        const size_t slot = (size_t)(base + c) * H + h;
        float *Sd = ws.S + slot * dd;
        for (int e = tid; e < dt; e += CT) {
            const int r = e / TV;
            Sd[(size_t)r * d + v0 + (e - r * TV)] = sA[e];
        }
        commit_chunk(false, c + 1 < nck ? c + 1 : -1);
        // Z = T Diag(beta) V - R S on this tile
        float *Zd = ws.Z + slot * cd;
        for (int e = tid / ZS; e < ct; e += CT / ZS) {
            const int i = e / TV, j = e - i * TV, part = tid % ZS;
            float z = 0.f;
            if (part == 0)
                for (int m = 0; m <= i; ++m) z += sT[i * C + m] * sb[m] * svt[m * TV + j];
#pragma unroll 8
            for (int r = part * (d / ZS); r < (part + 1) * (d / ZS); ++r)
                z -= sR[i * dp + r] * sA[r * TV + j];
            if (ZS == 2) z += __shfl_xor(z, 1);
            if (part == 0) {
                szt[e] = z;
                Zd[(size_t)i * d + v0 + j] = z;
            }
        }
        __syncthreads();
        // S <- Diag(e^{G_C}) S + Kbar^T Z, in place: each thread owns its entries
        if (rb0 < d) {   // rows rb0 + RS u of column jc (RS >= d leaves some threads idle)
            float acc[RPT];
#pragma unroll
            for (int u = 0; u < RPT; ++u) {
                const int r = min(rb0 + RS * u, d - 1);
                acc[u] = sgC[r] * sA[r * TV + jc];
            }
#pragma unroll 4
            for (int i = 0; i < C; ++i) {
                const float z = szt[i * TV + jc];
#pragma unroll
                for (int u = 0; u < RPT; ++u) acc[u] += sKb[i * dp + min(rb0 + RS * u, d - 1)] * z;
            }
#pragma unroll
            for (int u = 0; u < RPT; ++u)
                if (rb0 + RS * u < d) sA[(rb0 + RS * u) * TV + jc] = acc[u];
        }
        __syncthreads();
    }

    // ---- reverse sweep: dS' at each chunk end, and dZ; dS_0 at the end -----------
    for (int e = tid; e < dt; e += CT) {
        const int r = e / TV;
        sA[e] = dfinal ? dfinal[pair * dd + (size_t)r * d + v0 + (e - r * TV)] : 0.f;
    }
    if (nck > 0) fetch_chunk(nck - 1, true);
    __syncthreads();
    for (int c = nck - 1; c >= 0; --c) {
        const size_t slot = (size_t)(base + c) * H + h;
        float *dSd = ws.dS + slot * dd;
        for (int e = tid; e < dt; e += CT) {
            const int r = e / TV;
            dSd[(size_t)r * d + v0 + (e - r * TV)] = sA[e];
        }
        commit_chunk(true, c > 0 ? c - 1 : -1);
        // dZ = Kbar dS' + H^T dO on this tile
        float *dZd = ws.dZ + slot * cd;
        for (int e = tid / ZS; e < ct; e += CT / ZS) {
            const int i = e / TV, j = e - i * TV, part = tid % ZS;
            float z = 0.f;
#pragma unroll 8
            for (int r = part * (d / ZS); r < (part + 1) * (d / ZS); ++r)
                z += sKb[i * dp + r] * sA[r * TV + j];
            if (part == 0)
                for (int i2 = i; i2 < C; ++i2) z += sHm[i2 * C + i] * svt[i2 * TV + j];
            if (ZS == 2) z += __shfl_xor(z, 1);
            if (part == 0) {
                szt[e] = z;
                dZd[(size_t)i * d + v0 + j] = z;
            }
        }
        __syncthreads();
        // dS = Diag(e^{G_C}) dS' + Qbar^T dO - R^T dZ, in place
        if (rb0 < d) {
            float acc[RPT];
#pragma unroll
            for (int u = 0; u < RPT; ++u) {
                const int r = min(rb0 + RS * u, d - 1);
                acc[u] = sgC[r] * sA[r * TV + jc];
            }
#pragma unroll 4
            for (int i = 0; i < C; ++i) {
                const float o = svt[i * TV + jc], z = szt[i * TV + jc];
#pragma unroll
                for (int u = 0; u < RPT; ++u) {
                    const int r = min(rb0 + RS * u, d - 1);
                    acc[u] += sQb[i * dp + r] * o - sR[i * dp + r] * z;
                }
            }
#pragma unroll
            for (int u = 0; u < RPT; ++u)
                if (rb0 + RS * u < d) sA[(rb0 + RS * u) * TV + jc] = acc[u];
        }
        __syncthreads();
    }
    if (ds0)
        for (int e = tid; e < dt; e += CT) {
            const int r = e / TV;
            ds0[pair * dd + (size_t)r * d + v0 + (e - r * TV)] = sA[e];
        }
}

// ---- chain kernel on fp32 MFMA (C = 16, d = 128) ------------------------------------
// The same two sweeps with the state tile in MFMA accumulators.  Four waves;
// wave w owns state rows (key channels) 32w .. 32w+31 of the 16 value columns
// as two 16x16 fp32 tiles.  v_mfma_f32_16x16x4f32: lane l gives A[l % 16][k]
// and B[k][l % 16] and holds D rows 4 (l / 16) + e, column l % 16 (e = 0..3).
// Step s of a contraction uses k = 4 (l / 16) + s, so an accumulator tile is
// the B operand of the next product as it stands: S feeds Z = U - R S, Z feeds
// S <- Diag(e^{G_C}) S + Kbar^T Z, and likewise dS', dZ in the reverse sweep.
// Each wave forms the part of Z (dZ) over its own 32 channels; the four parts
// meet in LDS (double-buffered, one barrier per chunk step).  The next chunk's
// operands are loaded into registers during the current step.
constexpr int MT = 256;   // MFMA chain kernel: one compute wave per SIMD
constexpr int MTP = MT + 64;   // and a prefetch wave
constexpr int MC = 16, MD = 128;
#ifndef KDA_BWD_PD
#define KDA_BWD_PD 5
#endif
#ifndef KDA_BWD_PR
#define KDA_BWD_PR 3
#endif
constexpr int BWD_PD = KDA_BWD_PD;   // prefetch distance in chunk steps
constexpr int BWD_PR = KDA_BWD_PR;   // chunk steps between a touch and its wait

// Token-row values are kept as loaded (bf16 bits or fp32) and widened where
// they are used, so that nothing waits on the next chunk's loads early.
template <typename In> struct Raw {
    typedef float type;
    __device__ static float ld(const float *p, size_t i) { return p[i]; }
    __device__ static float f(float x) { return x; }
};
template <> struct Raw<bf16_t> {
    typedef unsigned short type;
    __device__ static unsigned short ld(const bf16_t *p, size_t i) { return p[i].bits; }
    __device__ static float f(unsigned short x) { return bf16_to_f32(x); }
};
template <typename In> struct FwdOps {
    float4 r[2];     // R[i16][32w + 16cl + 4g4 .. +3]        (A of R S)
    float kb[2][4];  // Kbar[4g4 + s][32w + 16cl + i16]      (A of Kbar^T Z)
    float4 gc[2];    // e^{G_C}[32w + 16cl + 4g4 .. +3]
    float t;         // T[i16][4g4 + w]                       (A of T (beta V), step w)
    float b;         // beta[4g4 + w]                          (B of T (beta V): beta V)
    typename Raw<In>::type vr;      // V[4g4 + w][v0 + i16]
    int len;         // tokens in the chunk: rows >= len count as zero
};
template <typename In> struct RevOps {
    float4 kb[2];    // Kbar[i16][32w + 16cl + 4g4 .. +3]     (A of Kbar dS')
    float qb[2][4];  // Qbar[4g4 + s][32w + 16cl + i16]       (A of Qbar^T dO)
    float rr[2][4];  // R[4g4 + s][32w + 16cl + i16]          (A of R^T dZ)
    float4 gc[2];
    float h;         // H[4g4 + w][i16]                        (A of H^T dO, step w)
    typename Raw<In>::type dr[4];   // dO[4g4 + s][v0 + i16]  (B of H^T dO, Qbar^T dO)
    int len;
};


template <typename In>
__global__ __launch_bounds__(MTP) void kda_bwd_chain_mfma_kernel(
    const In *__restrict__ v, const float *__restrict__ beta, int H, int row_len,
    const int32_t *__restrict__ cu, int n_pairs, const float *__restrict__ s0,
    const float *__restrict__ dfinal, const In *__restrict__ dout, float *__restrict__ ds0,
    Ws ws) {
    constexpr int C = MC, d = MD, dd = MD * MD, cd = MC * MD;
    __shared__ float4v sPart[2][4][64];   // [buffer][wave][lane]: one wave's part of Z or dZ

    // Block id -> (pair, value tile) with the 8 tiles of a pair on one XCD.
    const int bid = blockIdx.x, lane8 = bid & 7, rest = bid >> 3;
    const int tile = rest & 7, pid = (rest >> 3) * 8 + lane8;
    if (pid >= n_pairs) return;
    const int n = pid / H, h = pid - n * H;
    const int tid = threadIdx.x, l = tid & 63, g4 = l >> 4, i16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int v0 = tile * TV;
    int ts, te;
    seq_range(cu, row_len, n, ts, te);
    const size_t pair = (size_t)pid;
    const int nck = (te - ts + C - 1) / C;
    const int base = chunk_base(ts, n, C);
    if (w == 4) {
        // Prefetch wave.  Step q of the 2 nck chunk steps (forward, then
        // reverse) touches the operand lines of the step BWD_PD later: one
        // 4-byte load per 128-byte line, every eighth line from this tile's
        // offset, so the eight value tiles of a pair together bring each
        // line into their XCD's L2 before the compute waves' register rings
        // load it.  A touch is waited for BWD_PR steps after it was issued,
        // and this wave meets the compute waves at their one barrier per
        // step, so it never holds that barrier up on memory.
        constexpr int RL = MD * (int)sizeof(In) / 128;   // lines per token row
        static_assert(MD * sizeof(In) % 128 == 0 && (C * MD * 4) % 128 == 0, "whole lines");
        auto line = [&](bool rev, int c, int li) -> const uint32_t * {
            const size_t slot = (size_t)(base + c) * H + h;
            const int t0 = ts + c * C, len = min(C, te - t0);
            const int nb = rev ? 3 : 2, nl = 64 * nb + 4 + 8 + C * RL;
            li = min(li, nl - 1);
            if (li < 64 * nb) {
                const float *blk = rev ? (li < 64 ? ws.Kb : li < 128 ? ws.Qb : ws.R)
                                       : (li < 64 ? ws.R : ws.Kb);
                return reinterpret_cast<const uint32_t *>(blk + slot * cd) + 32 * (li & 63);
            }
            li -= 64 * nb;
            if (li < 4) return reinterpret_cast<const uint32_t *>(ws.gC + slot * d) + 32 * li;
            li -= 4;
            if (li < 8)
                return reinterpret_cast<const uint32_t *>((rev ? ws.Hm : ws.T) + slot * C * C) +
                       32 * li;
            li -= 8;
            const int row = min(li / RL, len - 1);
            const In *src = (rev ? dout : v) + ((size_t)(t0 + row) * H + h) * d;
            return reinterpret_cast<const uint32_t *>(src) + 32 * (li % RL);
        };
        uint32_t ring[BWD_PR];
#pragma unroll
        for (int j = 0; j < BWD_PR; ++j) ring[j] = 0u;
        const int nq = 2 * nck;
        auto touch = [&](int j, int q) {
            const int p = q + BWD_PD;
            const bool rev = p >= nck;
            const int c = !rev ? p : max(nq - 1 - p, 0);
            asm volatile("" ::"v"(ring[j]));
            ring[j] = *line(rev, c, 8 * l + tile);
            lds_barrier();
        };
        int q = 0;
        for (; q + BWD_PR <= nq; q += BWD_PR)
#pragma unroll
            for (int j = 0; j < BWD_PR; ++j) touch(j, q + j);
#pragma unroll
        for (int j = 0; j < BWD_PR - 1; ++j)
            if (q + j < nq) touch(j, q + j);
#pragma unroll
        for (int j = 0; j < BWD_PR; ++j) asm volatile("" ::"v"(ring[j]));
        return;
    }
    // This lane's state entries: rows 32w + 16cl + 4g4 + e, column v0 + i16.
    auto srow = [&](int cl, int e) { return 32 * w + 16 * cl + 4 * g4 + e; };

    // Rows past the chunk's end are read at its last token (in bounds) and
    // zeroed where they are used.
    auto load_fwd = [&](int c, FwdOps<In> &op) {
        const size_t slot = (size_t)(base + c) * H + h;
        const int t0 = ts + c * C, len = min(C, te - t0);
        const float *R = ws.R + slot * cd, *Kb = ws.Kb + slot * cd, *gC = ws.gC + slot * d;
#pragma unroll
        for (int cl = 0; cl < 2; ++cl) {
            op.r[cl] = *reinterpret_cast<const float4 *>(R + i16 * d + srow(cl, 0));
            op.gc[cl] = *reinterpret_cast<const float4 *>(gC + srow(cl, 0));
#pragma unroll
            for (int s = 0; s < 4; ++s) op.kb[cl][s] = Kb[(4 * g4 + s) * d + 32 * w + 16 * cl + i16];
        }
        // T (beta V) is split over the waves by reduction step: wave w takes k = 4g4 + w
        op.t = ws.T[slot * C * C + i16 * C + 4 * g4 + w];
        const size_t row = (size_t)(t0 + min(4 * g4 + w, len - 1)) * H + h;
        op.b = beta[row];
        op.vr = Raw<In>::ld(v, row * d + v0 + i16);
        op.len = len;
    };
    auto load_rev = [&](int c, RevOps<In> &op) {
        const size_t slot = (size_t)(base + c) * H + h;
        const int t0 = ts + c * C, len = min(C, te - t0);
        const float *R = ws.R + slot * cd, *Kb = ws.Kb + slot * cd, *Qb = ws.Qb + slot * cd;
        const float *gC = ws.gC + slot * d;
#pragma unroll
        for (int cl = 0; cl < 2; ++cl) {
            op.kb[cl] = *reinterpret_cast<const float4 *>(Kb + i16 * d + srow(cl, 0));
            op.gc[cl] = *reinterpret_cast<const float4 *>(gC + srow(cl, 0));
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                op.qb[cl][s] = Qb[(4 * g4 + s) * d + 32 * w + 16 * cl + i16];
                op.rr[cl][s] = R[(4 * g4 + s) * d + 32 * w + 16 * cl + i16];
            }
        }
        op.h = ws.Hm[slot * C * C + (4 * g4 + w) * C + i16];
#pragma unroll
        for (int s = 0; s < 4; ++s)
            op.dr[s] = Raw<In>::ld(dout, ((size_t)(t0 + min(4 * g4 + s, len - 1)) * H + h) * d +
                                             v0 + i16);
        op.len = len;
    };
    // This wave's state rows (32w + 16cl + 4g4 + e, column v0 + i16) to dst.
    auto store_tile = [&](const float4v (&x)[2], float *dst) {
#pragma unroll
        for (int cl = 0; cl < 2; ++cl)
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[(size_t)srow(cl, e) * d + v0 + i16] = x[cl][e];
    };
    // Element w of a 4-vector (w is uniform; no register indexing).
    auto pick = [&](const float4v &x) { return w == 0 ? x[0] : w == 1 ? x[1] : w == 2 ? x[2] : x[3]; };
    // The four waves' parts of Z (dZ) summed; buffer b alternates by chunk.
    // The waves share nothing but LDS, so the barrier waits for LDS only and
    // the next chunk's operand loads stay in flight across it.
    auto exchange = [&](float4v part, int b) {
        sPart[b][w][l] = part;
        lds_barrier();
        float4v z = sPart[b][0][l];
#pragma unroll
        for (int u = 1; u < 4; ++u) z += sPart[b][u][l];
        return z;
    };

    float4v St[2];   // S (forward sweep), dS' (reverse sweep)
#pragma unroll
    for (int cl = 0; cl < 2; ++cl)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            St[cl][e] = s0 ? s0[pair * dd + (size_t)srow(cl, e) * d + v0 + i16] : 0.f;

    // ---- forward sweep ----
    // The state is stored at the start of even chunks only, and dS' at the end
    // of odd chunks and of the last one: the gradient kernel rebuilds the
    // other from its neighbour's with one chunk step, which costs less than
    // the stores saved.
    auto fwd_step = [&](int c, const FwdOps<In> &op) {
        const size_t slot = (size_t)(base + c) * H + h;
        if (!(c & 1)) store_tile(St, ws.S + slot * dd);
        // this wave's part of Z: -R[:, rows of w] S[rows of w], plus step w of U
        float4v p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cl = 0; cl < 2; ++cl) {
            p = mfma4(op.r[cl].x, St[cl][0], p);
            p = mfma4(op.r[cl].y, St[cl][1], p);
            p = mfma4(op.r[cl].z, St[cl][2], p);
            p = mfma4(op.r[cl].w, St[cl][3], p);
        }
        p = -p;
        // reduction step w of U = T (beta V)
        p = mfma4(op.t, 4 * g4 + w < op.len ? op.b * Raw<In>::f(op.vr) : 0.f, p);
        const float4v z = exchange(p, c & 1);
        // every wave stores one token row of each lane group: 4g4 + w
        ws.Z[slot * cd + (size_t)(4 * g4 + w) * d + v0 + i16] = pick(z);
        // S <- Diag(e^{G_C}) S + Kbar^T Z on this wave's rows
#pragma unroll
        for (int cl = 0; cl < 2; ++cl) {
            float4v a = St[cl] * as4v(op.gc[cl]);
#pragma unroll
            for (int s = 0; s < 4; ++s) a = mfma4(op.kb[cl][s], z[s], a);
            St[cl] = a;
        }
    };
    // A ring of three chunks' operands, refilled two chunks ahead (a fourth
    // slot measured no faster).  Loads past the last chunk re-read it (in
    // bounds, unused), so the loop has no conditional loads and the wait
    // counts stay exact across it.
    if (nck > 0) {
        const int cl = nck - 1;
        FwdOps<In> A, B, D;
        load_fwd(0, A);
        load_fwd(min(1, cl), B);
        int c = 0;
        for (; c + 3 <= nck; c += 3) {
            load_fwd(min(c + 2, cl), D);
            fwd_step(c, A);
            load_fwd(min(c + 3, cl), A);
            fwd_step(c + 1, B);
            load_fwd(min(c + 4, cl), B);
            fwd_step(c + 2, D);
        }
        if (c < nck) fwd_step(c, A);
        if (c + 1 < nck) fwd_step(c + 1, B);
    }

    // ---- reverse sweep ----
#pragma unroll
    for (int cl = 0; cl < 2; ++cl)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            St[cl][e] = dfinal ? dfinal[pair * dd + (size_t)srow(cl, e) * d + v0 + i16] : 0.f;
    auto rev_step = [&](int c, const RevOps<In> &op) {
        const size_t slot = (size_t)(base + c) * H + h;
        if ((c & 1) || c == nck - 1) store_tile(St, ws.dS + slot * dd);
        float dO[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) dO[s] = 4 * g4 + s < op.len ? Raw<In>::f(op.dr[s]) : 0.f;
        // this wave's part of dZ: Kbar[:, rows of w] dS'[rows of w], plus step w of H^T dO
        float4v p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cl = 0; cl < 2; ++cl) {
            p = mfma4(op.kb[cl].x, St[cl][0], p);
            p = mfma4(op.kb[cl].y, St[cl][1], p);
            p = mfma4(op.kb[cl].z, St[cl][2], p);
            p = mfma4(op.kb[cl].w, St[cl][3], p);
        }
        // reduction step w of H^T dO
        p = mfma4(op.h, w == 0 ? dO[0] : w == 1 ? dO[1] : w == 2 ? dO[2] : dO[3], p);
        // Buffers keep alternating across the two sweeps: the forward sweep's
        // last step (c = nck - 1) used buffer (nck - 1) & 1, so this sweep's
        // first step, also c = nck - 1, takes the other one.
        const float4v z = exchange(p, (c + 1) & 1);
        ws.dZ[slot * cd + (size_t)(4 * g4 + w) * d + v0 + i16] = pick(z);
        // dS <- Diag(e^{G_C}) dS' + Qbar^T dO - R^T dZ on this wave's rows
        const float4v nz = -z;
#pragma unroll
        for (int cl = 0; cl < 2; ++cl) {
            float4v a = St[cl] * as4v(op.gc[cl]);
#pragma unroll
            for (int s = 0; s < 4; ++s) a = mfma4(op.qb[cl][s], dO[s], a);
#pragma unroll
            for (int s = 0; s < 4; ++s) a = mfma4(op.rr[cl][s], nz[s], a);
            St[cl] = a;
        }
    };
    if (nck > 0) {
        RevOps<In> A, B, D;
        load_rev(nck - 1, A);
        load_rev(max(nck - 2, 0), B);
        int c = nck - 1;
        for (; c - 2 >= 0; c -= 3) {
            load_rev(max(c - 2, 0), D);
            rev_step(c, A);
            load_rev(max(c - 3, 0), A);
            rev_step(c - 1, B);
            load_rev(max(c - 4, 0), B);
            rev_step(c - 2, D);
        }
        if (c >= 0) rev_step(c, A);
        if (c - 1 >= 0) rev_step(c - 1, B);
    }
    if (ds0) {
#pragma unroll
        for (int cl = 0; cl < 2; ++cl)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ds0[pair * dd + (size_t)srow(cl, e) * d + v0 + i16] = St[cl][e];
    }
}

// ---- fp32 prefill at d = 128 on the prep kernel's factors -------------------------
// The forward pass of the same chunk algebra for fp32 storage at d = 128, with
// 16-token chunks: the prep kernel above writes K~, T, H, R, Kbar, Qbar and
// e^{G_C} per (chunk, head); this chain kernel then walks the chunks with the
// state tile in MFMA accumulators, as the backward's forward sweep does, and
// also forms the output:
//   Z = U - R S,  O = Qbar S + H Z,  S <- Diag(e^{G_C}) S + Kbar^T Z.
// Each wave adds its 32 channels' parts of R S and of Qbar S; the four parts
// of both meet in one double-buffered LDS exchange per chunk.  Every wave
// then adds H Z over the whole chunk (4 MFMAs) and stores one token row of
// each lane group of O.  A fifth wave prefetches, as in the backward chain.
struct FwdOutOps {
    float4 r[2];     // R[i16][32w + 16cl + 4g4 .. +3]        (A of R S)
    float4 qb[2];    // Qbar[i16][32w + 16cl + 4g4 .. +3]     (A of Qbar S)
    float kb[2][4];  // Kbar[4g4 + s][32w + 16cl + i16]      (A of Kbar^T Z)
    float4 gc[2];    // e^{G_C}[32w + 16cl + 4g4 .. +3]
    float hm[4];     // H[i16][4g4 + s]                        (A of H Z)
    float t;         // T[i16][4g4 + w]                        (A of T (beta V), step w)
    float b;         // beta[4g4 + w]
    float vr;        // V[4g4 + w][v0 + i16]
    int len;
};

__global__ __launch_bounds__(MTP) void kda_fwd_f32_chain_kernel(
    const float *__restrict__ v, const float *__restrict__ beta, int H, int row_len,
    const int32_t *__restrict__ cu, int n_pairs, const float *__restrict__ s0,
    float *__restrict__ o, float *__restrict__ s_final, Ws ws, int form) {
    constexpr int C = MC, d = MD, dd = MD * MD, cd = MC * MD;
    __shared__ float4v sPart[2][2][4][64];   // [buffer][R S or Qbar S][wave][lane]

    // Block id -> (pair, value tile) with the 8 tiles of a pair on one XCD.
    const int bid = blockIdx.x, lane8 = bid & 7, rest = bid >> 3;
    const int tile = rest & 7, pid = (rest >> 3) * 8 + lane8;
    if (pid >= n_pairs) return;
    const int n = pid / H, h = pid - n * H;
    const int tid = threadIdx.x, l = tid & 63, g4 = l >> 4, i16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int v0 = tile * TV;
    int ts, te;
    seq_range(cu, row_len, n, ts, te);
    const size_t pair = (size_t)pid;
    const int nck = (te - ts + C - 1) / C;
    const int base = chunk_base(ts, n, C);
    if (w == 4) {
        // Prefetch wave: one line in eight of chunk c + BWD_PD's operands at
        // step c (R, Kbar, Qbar, e^{G_C}, T, H, the value rows), each tile of
        // the pair taking a different eighth; a touch is waited for BWD_PR
        // steps after it was issued.
        constexpr int RL = MD * 4 / 128;   // lines per value row
        constexpr int NL = 3 * 64 + 4 + 8 + 8 + C * RL;
        auto line = [&](int c, int li) -> const uint32_t * {
            const size_t slot = (size_t)(base + c) * H + h;
            const int t0 = ts + c * C, len = min(C, te - t0);
            li = min(li, NL - 1);
            if (li < 192) {
                const float *blk = li < 64 ? ws.R : li < 128 ? ws.Kb : ws.Qb;
                return reinterpret_cast<const uint32_t *>(blk + slot * cd) + 32 * (li & 63);
            }
            li -= 192;
            if (li < 4) return reinterpret_cast<const uint32_t *>(ws.gC + slot * d) + 32 * li;
            li -= 4;
            if (li < 16)
                return reinterpret_cast<const uint32_t *>((li < 8 ? ws.T : ws.Hm) + slot * C * C) +
                       32 * (li & 7);
            li -= 16;
            const int row = min(li / RL, len - 1);
            return reinterpret_cast<const uint32_t *>(v + ((size_t)(t0 + row) * H + h) * d) +
                   32 * (li % RL);
        };
        uint32_t ring[BWD_PR];
#pragma unroll
        for (int j = 0; j < BWD_PR; ++j) ring[j] = 0u;
        auto touch = [&](int j, int c) {
            asm volatile("" ::"v"(ring[j]));
            ring[j] = *line(min(c + BWD_PD, nck - 1), 8 * l + tile);
            lds_barrier();
        };
        int c = 0;
        for (; c + BWD_PR <= nck; c += BWD_PR)
#pragma unroll
            for (int j = 0; j < BWD_PR; ++j) touch(j, c + j);
#pragma unroll
        for (int j = 0; j < BWD_PR - 1; ++j)
            if (c + j < nck) touch(j, c + j);
#pragma unroll
        for (int j = 0; j < BWD_PR; ++j) asm volatile("" ::"v"(ring[j]));
        return;
    }
    auto srow = [&](int cl, int e) { return 32 * w + 16 * cl + 4 * g4 + e; };
    // Rows past the chunk's end are read at its last token (in bounds) and
    // zeroed where they are used.
    auto load = [&](int c, FwdOutOps &op) {
        const size_t slot = (size_t)(base + c) * H + h;
        const int t0 = ts + c * C, len = min(C, te - t0);
        const float *R = ws.R + slot * cd, *Kb = ws.Kb + slot * cd, *Qb = ws.Qb + slot * cd;
        const float *gC = ws.gC + slot * d, *Hm = ws.Hm + slot * C * C;
#pragma unroll
        for (int cl = 0; cl < 2; ++cl) {
            op.r[cl] = *reinterpret_cast<const float4 *>(R + i16 * d + srow(cl, 0));
            op.qb[cl] = *reinterpret_cast<const float4 *>(Qb + i16 * d + srow(cl, 0));
            op.gc[cl] = *reinterpret_cast<const float4 *>(gC + srow(cl, 0));
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) op.kb[cl][s2] = Kb[(4 * g4 + s2) * d + 32 * w + 16 * cl + i16];
        }
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) op.hm[s2] = Hm[i16 * C + 4 * g4 + s2];
        op.t = ws.T[slot * C * C + i16 * C + 4 * g4 + w];
        const size_t row = (size_t)(t0 + min(4 * g4 + w, len - 1)) * H + h;
        op.b = beta[row];
        op.vr = v[row * d + v0 + i16];
        op.len = len;
    };
    auto pick = [&](const float4v &x) { return w == 0 ? x[0] : w == 1 ? x[1] : w == 2 ? x[2] : x[3]; };
    const bool beta_logit = form & kFormBetaLogit;

    float4v St[2];
#pragma unroll
    for (int cl = 0; cl < 2; ++cl)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            St[cl][e] = s0 ? s0[pair * dd + (size_t)srow(cl, e) * d + v0 + i16] : 0.f;

    auto step = [&](int c, const FwdOutOps &op) {
        // this wave's parts of -R S (plus step w of U) and of Qbar S
        float4v p = {0.f, 0.f, 0.f, 0.f}, po = p;
#pragma unroll
        for (int cl = 0; cl < 2; ++cl) {
            p = mfma4(op.r[cl].x, St[cl][0], p);
            p = mfma4(op.r[cl].y, St[cl][1], p);
            p = mfma4(op.r[cl].z, St[cl][2], p);
            p = mfma4(op.r[cl].w, St[cl][3], p);
            po = mfma4(op.qb[cl].x, St[cl][0], po);
            po = mfma4(op.qb[cl].y, St[cl][1], po);
            po = mfma4(op.qb[cl].z, St[cl][2], po);
            po = mfma4(op.qb[cl].w, St[cl][3], po);
        }
        p = -p;
        const float bw = beta_logit ? sigmoid(op.b) : op.b;
        p = mfma4(op.t, 4 * g4 + w < op.len ? bw * op.vr : 0.f, p);
        const int b = c & 1;
        sPart[b][0][w][l] = p;
        sPart[b][1][w][l] = po;
        lds_barrier();
        float4v z = sPart[b][0][0][l], oz = sPart[b][1][0][l];
#pragma unroll
        for (int u = 1; u < 4; ++u) {
            z += sPart[b][0][u][l];
            oz += sPart[b][1][u][l];
        }
        // O = Qbar S + H Z, token rows 4g4 + e of this lane group
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) oz = mfma4(op.hm[s2], z[s2], oz);
        if (4 * g4 + w < op.len)
            o[((size_t)(ts + c * C + 4 * g4 + w) * H + h) * d + v0 + i16] = pick(oz);
        // S <- Diag(e^{G_C}) S + Kbar^T Z on this wave's rows
#pragma unroll
        for (int cl = 0; cl < 2; ++cl) {
            float4v a = St[cl] * as4v(op.gc[cl]);
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) a = mfma4(op.kb[cl][s2], z[s2], a);
            St[cl] = a;
        }
    };
    // A ring of three chunks' operands, refilled two chunks ahead; loads past
    // the last chunk re-read it (in bounds, unused).
    if (nck > 0) {
        const int cl = nck - 1;
        FwdOutOps A, B, D;
        load(0, A);
        load(min(1, cl), B);
        int c = 0;
        for (; c + 3 <= nck; c += 3) {
            load(min(c + 2, cl), D);
            step(c, A);
            load(min(c + 3, cl), A);
            step(c + 1, B);
            load(min(c + 4, cl), B);
            step(c + 2, D);
        }
        if (c < nck) step(c, A);
        if (c + 1 < nck) step(c + 1, B);
    }
    if (s_final) {
#pragma unroll
        for (int cl = 0; cl < 2; ++cl)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                s_final[pair * dd + (size_t)srow(cl, e) * d + v0 + i16] = St[cl][e];
    }
}

// ---- gradient kernel ------------------------------------------------------------
__host__ __device__ inline int slice_rows(int d) { return d < 16 ? d : 16; }

struct GradLds {
    int q, k, G, v, dO, Z, dZ, dR, dL, dQb, dKb, Ssl, dSsl, beta, dbeta, Kt, Hm, T, dT, M1, gc,
        total;
};
__host__ __device__ inline GradLds grad_layout(int d, int C) {
    GradLds L;
    int o = 0;
    const int cd = C * row_stride(d), cc = C * C, sd = slice_rows(d) * row_stride(d);
    L.q = o; o += cd;
    L.k = o; o += cd;
    L.G = o; o += cd;
    L.v = o; o += cd;
    L.dO = o; o += cd;    // later dBV
    L.Z = o; o += cd;
    L.dZ = o; o += cd;
    L.dR = o; o += cd;    // later dG
    L.dL = o; o += cd;
    if (d == 128 && C == 16) {
        // Products on MFMA: no slices of S and dS' in LDS, and dQbar, dKbar
        // wait in accumulators until v and Z are dead, then take their place.
        L.dQb = L.v;
        L.dKb = L.Z;
        L.Ssl = L.dSsl = 0;
    } else {
        L.dQb = o; o += cd;   // dL/dQbar = dO S^T
        L.dKb = o; o += cd;   // dL/dKbar = Z dS'^T
        L.Ssl = o; o += sd;   // rows of S
        L.dSsl = o; o += sd;  // rows of dS'
    }
    L.beta = o; o += C;
    L.dbeta = o; o += C;
    L.Kt = o; o += cc;    // K~, later its gradient
    L.Hm = o; o += cc;    // dH
    L.T = o; o += cc;
    L.dT = o; o += cc;    // later dA . K~
    L.M1 = o; o += cc;    // T^T dT
    L.gc = o; o += d;     // e^{G_C} rowsum(dS' . S)
    L.total = o;
    return L;
}

template <int C, int D, typename In>
__global__ __launch_bounds__(GT) void kda_bwd_grad_kernel(
    const In *__restrict__ q, const In *__restrict__ k, const In *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float scale, int H,
    int row_len, const int32_t *__restrict__ cu, int n_seqs, const In *__restrict__ dout,
    float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dv,
    float *__restrict__ dg, float *__restrict__ dbeta, Ws ws) {
    constexpr int d = D;
    constexpr int XS = (C * (D < 16 ? D : 16) < GT) ? GT / (C * (D < 16 ? D : 16)) : 1;
    constexpr int PS = (C * C < GT) ? GT / (C * C) : 1;   // lanes sharing one dT / dH entry
    static_assert((XS == 1 || XS == 2) && (PS == 1 || PS == 2), "at most lane pairs");
    extern __shared__ float sm[];
    const GradLds L = grad_layout(d, C);
    float *sq = sm + L.q, *sk = sm + L.k, *sG = sm + L.G, *sv = sm + L.v, *sdO = sm + L.dO;
    float *sZ = sm + L.Z, *sdZ = sm + L.dZ, *sdR = sm + L.dR, *sdL = sm + L.dL;
    float *sdQb = sm + L.dQb, *sdKb = sm + L.dKb, *sS = sm + L.Ssl, *sdS = sm + L.dSsl;
    float *sb = sm + L.beta, *sdb = sm + L.dbeta, *sKt = sm + L.Kt, *sHm = sm + L.Hm;
    float *sT = sm + L.T, *sdT = sm + L.dT, *sM1 = sm + L.M1, *sgc = sm + L.gc;
    float *sdBV = sdO, *sdG = sdR, *sAK = sdT;

    const int slot = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
    const int tid = threadIdx.x;
    int t0, len, cix, te;
    if (!slot_chunk<C>(cu, row_len, n_seqs, slot, t0, len, cix, te)) return;
    const int cd = C * d, dd = d * d, SR = slice_rows(d), dp = row_stride(d);
    const size_t wslot = (size_t)slot * H + h;
    // At d = 128, C = 16 the chain kernel stores S only at the start of even
    // chunks and dS' only at the end of odd chunks and of the last one.  An
    // odd chunk rebuilds its S from chunk c - 1: S = Diag(e^{G_C}) S_prev +
    // Kbar^T Z of that chunk.  An even chunk that is not the last rebuilds its
    // dS' from chunk c + 1: dS' = Diag(e^{G_C}) dS'_next + Qbar^T dO - R^T dZ
    // of that chunk.  Both are the chain's own steps (the chunk recurrence and
    // its reverse), with operands from the workspace.  The staged operands sit
    // in the storage of dL (Z or dZ of the neighbour) and dR (dO of the next
    // chunk), both written only after the products with S and dS'.
    constexpr bool HALF = C == MC && D == MD;
    const bool s_rebuild = HALF && (cix & 1);
    const bool ds_rebuild = HALF && !(cix & 1) && t0 + C < te;

    float4 rS[8], rdS[8];   // rows of S and dS' (d = 128, C = 16)
    {
        const size_t off = ((size_t)t0 * H + h) * d, pitch = (size_t)H * d;
        Rows<GT> r[7];
        fetch_rows(r[0], q + off, pitch, C, len, d, tid);
        fetch_rows(r[1], k + off, pitch, C, len, d, tid);
        fetch_rows(r[2], g + off, pitch, C, len, d, tid);
        fetch_rows(r[3], v + off, pitch, C, len, d, tid);
        fetch_rows(r[4], dout + off, pitch, C, len, d, tid);
        fetch_rows(r[5], ws.Z + wslot * cd, d, C, C, d, tid);
        fetch_rows(r[6], ws.dZ + wslot * cd, d, C, C, d, tid);
        const float rb = tid < len ? beta[(size_t)(t0 + tid) * H + h] : 0.f;
        constexpr int NCC = (C * C + GT - 1) / GT;
        float rT[NCC], rK[NCC];
#pragma unroll
        for (int u = 0; u < NCC; ++u) {
            const int e = min(tid + u * GT, C * C - 1);
            rT[u] = ws.T[wslot * C * C + e];
            rK[u] = ws.Kt[wslot * C * C + e];
        }
        // Rows of S and dS' for the products below, issued after the inputs so
        // that committing those waits for them alone.
        if constexpr (C == 16 && D == 128) {
            const int l = tid & 63, g4 = l >> 4, ch = 16 * (tid >> 6) + (l & 15);
            const float *Sg = ws.S + (s_rebuild ? wslot - H : wslot) * dd;
            const float *dSg = ws.dS + (ds_rebuild ? wslot + H : wslot) * dd;
#pragma unroll
            for (int T = 0; T < 8; ++T) {
                const int u = 16 * T + 4 * g4;
                rS[T] = *reinterpret_cast<const float4 *>(Sg + (size_t)ch * d + u);
                rdS[T] = *reinterpret_cast<const float4 *>(dSg + (size_t)ch * d + u);
            }
        }
        Rows<GT> rx, ry;
        if (s_rebuild) {
            fetch_rows(rx, ws.Z + (wslot - H) * cd, d, C, C, d, tid);
        } else if (ds_rebuild) {
            fetch_rows(rx, ws.dZ + (wslot + H) * cd, d, C, C, d, tid);
            fetch_rows(ry, dout + off + C * pitch, pitch, C, min(C, te - t0 - C), d, tid);
        }
        float *dst[7] = {sq, sk, sG, sv, sdO, sZ, sdZ};
#pragma unroll
        for (int a = 0; a < 7; ++a) commit_rows(dst[a], r[a], C, d, tid);
        if (s_rebuild || ds_rebuild) commit_rows(sdL, rx, C, d, tid);
        if (ds_rebuild) commit_rows(sdR, ry, C, d, tid);
        if (tid < C) sb[tid] = rb;
#pragma unroll
        for (int u = 0; u < NCC; ++u)
            if (tid + u * GT < C * C) {
                sT[tid + u * GT] = rT[u];
                sKt[tid + u * GT] = rK[u];
            }
    }
    __syncthreads();
    cumsum_rows<C, GT>(sG, d, tid);
    __syncthreads();

    // The products with S and dS':
    //   dR = -dZ S^T,  dQbar = dO S^T,  dKbar = Z dS'^T,  gc = e^{G_C} rowsum(dS' . S).
    const float *Sg = ws.S + wslot * dd, *dSg = ws.dS + wslot * dd;
    // At d = 128, C = 16 (fp32 MFMA): wave w takes channels 16w .. 16w+15 (the
    // output columns), token rows are the output rows, and the value index u is
    // the reduction.  Instruction (T, s) takes u = 16T + 4 (l/16) + s from lane
    // l: its rows 16w + l % 16 of S and dS' are the float4 reads issued with
    // the inputs (32 values each), rows l % 16 of dZ, dO and Z come from LDS.
    // dQbar and dKbar stay in accumulators until v and Z are dead.
    float4v aQ = {0.f, 0.f, 0.f, 0.f}, aK = aQ;
    if constexpr (C == 16 && D == 128) {
        const int l = tid & 63, g4 = l >> 4, i16 = l & 15, w = tid >> 6;
        const int ch = 16 * w + i16;
        // The rebuilt tile in the layout of rS: computed transposed, value
        // rows 16T + l % 16 (A, from LDS) by channels (B), token 4 (l/16) + s in
        // step s, so accumulator element e is value 16T + 4 (l/16) + e of
        // channel ch.
        auto rebuild = [&](float4 (&X)[8], size_t nb, const float *A1, const float *B1,
                           const float *A2, const float *B2) {
            const float gc = ws.gC[nb * d + ch];
            float b1[4], b2[4];
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                b1[s2] = B1[nb * cd + (4 * g4 + s2) * d + ch];
                b2[s2] = B2 ? -B2[nb * cd + (4 * g4 + s2) * d + ch] : 0.f;
            }
#pragma unroll
            for (int T = 0; T < 8; ++T) {
                float4v a = as4v(X[T]) * gc;
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) {
                    const int x = (4 * g4 + s2) * dp + 16 * T + i16;
                    a = mfma4(A1[x], b1[s2], a);
                    if (A2) a = mfma4(A2[x], b2[s2], a);
                }
                X[T] = make_float4(a[0], a[1], a[2], a[3]);
            }
        };
        if (s_rebuild) {
            rebuild(rS, wslot - H, sdL, ws.Kb, nullptr, nullptr);
        } else if (ds_rebuild) {
            rebuild(rdS, wslot + H, sdR, ws.Qb, sdL, ws.R);
            __syncthreads();   // dR's storage is written below
        }
        float4v aR = {0.f, 0.f, 0.f, 0.f};
        float gsum = 0.f;
        const float *zr = sZ + i16 * dp + 4 * g4, *dzr = sdZ + i16 * dp + 4 * g4;
        const float *dor = sdO + i16 * dp + 4 * g4;
#pragma unroll
        for (int T = 0; T < 8; ++T) {
            const float s4[4] = {rS[T].x, rS[T].y, rS[T].z, rS[T].w};
            const float ds4[4] = {rdS[T].x, rdS[T].y, rdS[T].z, rdS[T].w};
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const int u = 16 * T + s2;
                aR = mfma4(dzr[u], s4[s2], aR);
                aQ = mfma4(dor[u], s4[s2], aQ);
                aK = mfma4(zr[u], ds4[s2], aK);
                gsum += ds4[s2] * s4[s2];
            }
        }
        // accumulator element e: token 4 (l/16) + e, channel ch
#pragma unroll
        for (int e = 0; e < 4; ++e) sdR[(4 * g4 + e) * dp + ch] = -aR[e];
        gsum += __shfl_xor(gsum, 16, 64);
        gsum += __shfl_xor(gsum, 32, 64);
        if (g4 == 0) sgc[ch] = fast_exp(sG[(C - 1) * dp + ch]) * gsum;
        __syncthreads();
    } else {
    Rows<GT> rS, rdS;
    fetch_rows(rS, Sg, d, SR, SR, d, tid);
    fetch_rows(rdS, dSg, d, SR, SR, d, tid);
    for (int r0 = 0; r0 < d; r0 += SR) {
        commit_rows(sS, rS, SR, d, tid);
        commit_rows(sdS, rdS, SR, d, tid);
        __syncthreads();
        if (r0 + SR < d) {
            fetch_rows(rS, Sg + (size_t)(r0 + SR) * d, d, SR, SR, d, tid);
            fetch_rows(rdS, dSg + (size_t)(r0 + SR) * d, d, SR, SR, d, tid);
        }
        for (int e = tid / XS; e < C * SR; e += GT / XS) {
            const int x = e / SR, rr = e - x * SR, part = tid % XS;
            float a = 0.f, b = 0.f, z = 0.f;
#pragma unroll 8
            for (int u = part * (d / XS); u < (part + 1) * (d / XS); ++u) {
                const float s = sS[rr * dp + u];
                a += sdZ[x * dp + u] * s;
                b += sdO[x * dp + u] * s;
                z += sZ[x * dp + u] * sdS[rr * dp + u];
            }
            if (XS == 2) {
                a += __shfl_xor(a, 1);
                b += __shfl_xor(b, 1);
                z += __shfl_xor(z, 1);
            }
            if (part == 0) {
                sdR[x * dp + r0 + rr] = -a;
                sdQb[x * dp + r0 + rr] = b;
                sdKb[x * dp + r0 + rr] = z;
            }
        }
        {
            // one slice row per LPR lanes of a wave, reduced by shuffles
            constexpr int LPR = GT / 16;
            static_assert(LPR <= 64 && 64 % LPR == 0, "a slice row within one wave");
            const int rr = tid / LPR, part = tid % LPR;
            float a = 0.f;
            if (rr < SR)
                for (int u = part; u < d; u += LPR) a += sdS[rr * dp + u] * sS[rr * dp + u];
#pragma unroll
            for (int m = LPR / 2; m >= 1; m >>= 1) a += __shfl_xor(a, m, 64);
            if (part == 0 && rr < SR) sgc[r0 + rr] = fast_exp(sG[(C - 1) * dp + r0 + rr]) * a;
        }
        __syncthreads();
    }
    }
    // dT = dZ (BV)^T + dR (BL)^T;  dH = dO Z^T (j <= i)
    if constexpr (C == 16 && D == 128) {
        // On fp32 MFMA, one 16 x 16 tile each: waves 0-3 take dT, waves 4-7 dH,
        // each wave 32 of the 128 channels (the reduction).  Lane l gives row
        // l % 16 of both operands at channel 32 (w % 4) + 4 (l/16) + s in step
        // s; L = k e^{G} is formed on the fly.  The four parts of each tile meet
        // in dL's storage, which is written only in the next phase.
        const int l = tid & 63, g4 = l >> 4, i16 = l & 15, w = tid >> 6;
        const int cb0 = 32 * (w & 3) + 4 * g4, r = i16 * dp;
        float4v acc = {0.f, 0.f, 0.f, 0.f};
        if (w < 4) {
#pragma unroll
            for (int t8 = 0; t8 < 8; ++t8) {
                const int c2 = cb0 + 16 * (t8 >> 2) + (t8 & 3);
                acc = mfma4(sdZ[r + c2], sv[r + c2], acc);
                acc = mfma4(sdR[r + c2], sk[r + c2] * fast_exp(sG[r + c2]), acc);
            }
        } else {
#pragma unroll
            for (int t8 = 0; t8 < 8; ++t8) {
                const int c2 = cb0 + 16 * (t8 >> 2) + (t8 & 3);
                acc = mfma4(sdO[r + c2], sZ[r + c2], acc);
            }
        }
        // accumulator element e: row i = 4 (l/16) + e, column j = l % 16
#pragma unroll
        for (int e = 0; e < 4; ++e) sdL[w * C * C + (4 * g4 + e) * C + i16] = acc[e];
        __syncthreads();
        {
            const int which = tid / (C * C), e = tid - which * (C * C);
            const int i = e / C, j = e - i * C;
            float a = 0.f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) a += sdL[(4 * which + ww) * C * C + e];
            if (which == 0) sdT[e] = sb[j] * a;
            else sHm[e] = j <= i ? a : 0.f;
        }
    } else {
        for (int e = tid / PS; e < C * C; e += GT / PS) {
            const int i = e / C, j = e - i * C, part = tid % PS;
            const int c0 = part * (d / PS), c1 = (part + 1) * (d / PS);
            float a = 0.f, hh = 0.f;
#pragma unroll 4
            for (int c2 = c0; c2 < c1; ++c2)
                a += sdZ[i * dp + c2] * sv[j * dp + c2] +
                     sdR[i * dp + c2] * sk[j * dp + c2] * fast_exp(sG[j * dp + c2]);
            if (j <= i)
#pragma unroll 4
                for (int c2 = c0; c2 < c1; ++c2) hh += sdO[i * dp + c2] * sZ[j * dp + c2];
            if (PS == 2) {
                a += __shfl_xor(a, 1);
                hh += __shfl_xor(hh, 1);
            }
            if (part == 0) {
                sdT[e] = sb[j] * a;
                sHm[e] = hh;
            }
        }
    }
    __syncthreads();
    // dBV = T^T dZ (into dO's storage), dBL = T^T dR;  M1 = T^T dT
    if constexpr (C == 16 && D == 128) {
        // On fp32 MFMA with the C tokens as the reduction: wave w takes channel
        // tile w of dBV and dBL, wave 0 also M1.  Lane l gives T[4 (l/16) + s][l % 16]
        // (A, transposed) and row 4 (l/16) + s of dZ, dR or dT (B) in step s.
        const int l = tid & 63, g4 = l >> 4, i16 = l & 15, w = tid >> 6;
        const int cc = 16 * w + i16;
        float4v bv = {0.f, 0.f, 0.f, 0.f}, bl = bv;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            const int i = 4 * g4 + s2;
            const float t = sT[i * C + i16];
            bv = mfma4(t, sdZ[i * dp + cc], bv);
            bl = mfma4(t, sdR[i * dp + cc], bl);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sdBV[(4 * g4 + e) * dp + cc] = bv[e];
            sdL[(4 * g4 + e) * dp + cc] = bl[e];
        }
        if (w == 0) {
            float4v m1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const int i = 4 * g4 + s2;
                m1 = mfma4(sT[i * C + i16], sdT[i * C + i16], m1);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) sM1[(4 * g4 + e) * C + i16] = m1[e];
        }
    } else {
        for (int e = tid; e < cd; e += GT) {
            const int j = e / d, c2 = e - j * d;
            float bv = 0.f, bl = 0.f;
            for (int i = j; i < C; ++i) {
                bv += sT[i * C + j] * sdZ[i * dp + c2];
                bl += sT[i * C + j] * sdR[i * dp + c2];
            }
            sdBV[j * dp + c2] = bv;
            sdL[j * dp + c2] = bl;
        }
        for (int e = tid; e < C * C; e += GT) {
            const int i = e / C, j = e - i * C;
            float a = 0.f;
            for (int m = i; m < C; ++m) a += sT[m * C + i] * sdT[m * C + j];
            sM1[e] = a;
        }
    }
    __syncthreads();
    // dbeta_j = dBV_j . v_j + dBL_j . L_j, row j over GT / C lanes of one wave
    {
        constexpr int LPR = GT / C;
        static_assert(LPR <= 64 && 64 % LPR == 0, "a row within one wave");
        const int j = tid / LPR, part = tid % LPR;
        float s = 0.f;
        for (int c2 = part; c2 < d; c2 += LPR)
            s += sdBV[j * dp + c2] * sv[j * dp + c2] +
                 sdL[j * dp + c2] * sk[j * dp + c2] * fast_exp(sG[j * dp + c2]);
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
        if (part == 0) sdb[j] = s;
    }
    // dA = M1 T^T (strictly lower); dA . K~ into dT's storage (dT is consumed);
    // dK~_ij = -beta_i dA_ij in place of K~
    for (int e = tid; e < C * C; e += GT) {
        const int i = e / C, j = e - i * C;
        float a = 0.f;
        if (j < i)
            for (int m = 0; m <= j; ++m) a += sM1[i * C + m] * sT[j * C + m];
        sAK[e] = a * sKt[e];
        sKt[e] = -sb[i] * a;
    }
    __syncthreads();
    // dv = beta dBV;  dL = beta dBL (in place);  dbeta_i -= sum_j dA_ij K~_ij
    if constexpr (C == 16 && D == 128) {
        // dQbar and dKbar into the storage of v and Z, which are dead now
        const int l = tid & 63, g4 = l >> 4, ch = 16 * (tid >> 6) + (l & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sdQb[(4 * g4 + e) * dp + ch] = aQ[e];
            sdKb[(4 * g4 + e) * dp + ch] = aK[e];
        }
    }
    for (int e = tid; e < cd; e += GT) {
        const int j = e / d, a = j * dp + (e - j * d);
        if (j < len) dv[((size_t)(t0 + j) * H + h) * d + (e - j * d)] = sb[j] * sdBV[a];
        sdL[a] *= sb[j];
    }
    for (int i = tid; i < C; i += GT) {
        float s = 0.f;
        for (int j = 0; j < i; ++j) s += sAK[i * C + j];
        sdb[i] -= s;
    }
    __syncthreads();
    // Per (row x, channel c), with E_ij = e^{G_ic - G_jc}:
    //   P1 = sum_{j<x} dK~_xj k_jc E_xj,  P2 = sum_{i>x} dK~_ix k_ic E_ix,
    //   P3 = sum_{j<=x} dH_xj k_jc E_xj,  P4 = sum_{i>=x} dH_ix (s q_ic) E_ix;
    // then the direct uses of e^{G} in Qbar, L and Kbar.  dK~ is zero on and
    // above its diagonal and dH above it, so the bounds on j and i hold by
    // themselves wherever the sums run over all rows.
    auto pairwise = [&](int x, int c2, float &P1, float &P2, float &P3, float &P4) {
        const float Gx = sG[x * dp + c2];
        P1 = P2 = P3 = P4 = 0.f;
        for (int j = 0; j <= x; ++j) {
            const float E = fast_exp(Gx - sG[j * dp + c2]) * sk[j * dp + c2];
            if (j < x) P1 += sKt[x * C + j] * E;
            P3 += sHm[x * C + j] * E;
        }
        for (int i = x; i < C; ++i) {
            const float E = fast_exp(sG[i * dp + c2] - Gx);
            if (i > x) P2 += sKt[i * C + x] * sk[i * dp + c2] * E;
            P4 += sHm[i * C + x] * scale * sq[i * dp + c2] * E;
        }
    };
    // dq and dk of row x, channel c2 to global memory; dG and the Kbar-term
    // of dG_C (summed over the rows below) into dR's and dL's storage, where
    // only this element's own thread reads them before the barrier.
    auto finish = [&](int x, int c2, float P1, float P2, float P3, float P4) {
        const int ax = x * dp + c2;
        const float Gx = sG[ax], kx = sk[ax], qx = scale * sq[ax];
        const float dQb = sdQb[ax], dKb = sdKb[ax], dLx = sdL[ax];
        const float eG = fast_exp(Gx), eK = fast_exp(sG[(C - 1) * dp + c2] - Gx);
        const float dqs = P3 + dQb * eG;
        const float dkx = P1 + P2 + P4 + dLx * eG + dKb * eK;
        const float dGx = kx * (P1 - P2 - P4) + qx * P3 + dQb * qx * eG + dLx * kx * eG -
                          dKb * kx * eK;
        if (x < len) {
            const size_t a = ((size_t)(t0 + x) * H + h) * d + c2;
            dq[a] = scale * dqs;
            dk[a] = dkx;
        }
        sdG[ax] = dGx;
        sdL[ax] = dKb * kx * eK;
    };
    if constexpr (C == 16 && D == 128) {
        // On fp32 MFMA.  With row r = 7 of the cumulative decays as reference,
        // e^{G_x - G_j} = e^{G_x - G_r} e^{G_r - G_j} in each channel, so every
        // sum is a C x C by C x d product between two row scalings:
        //   P1, P3 = e^{G_x - G_r} (dK~, dH) (k e^{G_r - G}),
        //   P2 = e^{G_r - G_x} dK~^T (k e^{G - G_r}),  P4 = e^{G_r - G_x} dH^T (s q e^{G - G_r}).
        // A channel that decays by at most 40 over the chunk keeps both factors
        // within e^{+-40}; a wave with a channel beyond that takes the pairwise
        // factors instead.  Wave w takes channels 16w .. 16w+15; lane l gives
        // token 4s + l/16 in step s, and accumulator element e is row 4 (l/16) + e.
        const int l = tid & 63, g4 = l >> 4, i16 = l & 15, ch = 16 * (tid >> 6) + i16;
        float P1[4], P2[4], P3[4], P4[4];
        if (__all(sG[ch] - sG[(C - 1) * dp + ch] <= 40.f)) {
            const float Gr = sG[7 * dp + ch];
            float4v a1 = {0.f, 0.f, 0.f, 0.f}, a2 = a1, a3 = a1, a4 = a1;
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const int j = 4 * s2 + g4, aj = j * dp + ch;
                const float Gj = sG[aj], kj = sk[aj], qj = scale * sq[aj];
                const float up = fast_exp(Gj - Gr), dn = fast_exp(Gr - Gj);
                a1 = mfma4(sKt[i16 * C + j], kj * dn, a1);
                a3 = mfma4(sHm[i16 * C + j], kj * dn, a3);
                a2 = mfma4(sKt[j * C + i16], kj * up, a2);
                a4 = mfma4(sHm[j * C + i16], qj * up, a4);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float Gx = sG[(4 * g4 + e) * dp + ch];
                const float up = fast_exp(Gx - Gr), dn = fast_exp(Gr - Gx);
                P1[e] = a1[e] * up;
                P3[e] = a3[e] * up;
                P2[e] = a2[e] * dn;
                P4[e] = a4[e] * dn;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) pairwise(4 * g4 + e, ch, P1[e], P2[e], P3[e], P4[e]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) finish(4 * g4 + e, ch, P1[e], P2[e], P3[e], P4[e]);
    } else {
        for (int e = tid; e < cd; e += GT) {
            const int x = e / d, c2 = e - x * d;
            float P1, P2, P3, P4;
            pairwise(x, c2, P1, P2, P3, P4);
            finish(x, c2, P1, P2, P3, P4);
        }
    }
    __syncthreads();
    // dG_C = gc + sum_x dKbar_x Kbar_x joins the last row; dg is the reverse
    // cumulative sum of dG over the valid rows (padding rows carry nothing).
    if constexpr (C == 16 && D == 128) {
        // Four threads per channel, each over four rows: the sums of its rows
        // (dG over the valid ones) meet in q's storage (q is dead after the
        // barrier above), then each thread adds the rows below its own.
        static_assert(GT == 4 * D, "four row quarters per channel");
        const int c2 = tid & (D - 1), qd = tid >> 7, x0 = 4 * qd;
        float sl = 0.f, sg = 0.f;
#pragma unroll
        for (int x = x0; x < x0 + 4; ++x) {
            sl += sdL[x * dp + c2];
            if (x < len) sg += sdG[x * dp + c2];
        }
        float *part = sq;   // [2][4][D] floats
        static_assert(2 * 4 * D <= C * (D + 1), "room for the row-quarter sums");
        part[qd * D + c2] = sl;
        part[4 * D + qd * D + c2] = sg;
        __syncthreads();
        float run = sgc[c2];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            run += part[u * D + c2];
            if (u > qd) run += part[4 * D + u * D + c2];
        }
#pragma unroll
        for (int x = x0 + 3; x >= x0; --x) {
            if (x < len) {
                run += sdG[x * dp + c2];
                dg[((size_t)(t0 + x) * H + h) * d + c2] = run;
            }
        }
    } else {
        for (int c2 = tid; c2 < d; c2 += GT) {
            float run = sgc[c2];
            for (int x = 0; x < C; ++x) run += sdL[x * dp + c2];
            for (int x = len - 1; x >= 0; --x) {
                run += sdG[x * dp + c2];
                dg[((size_t)(t0 + x) * H + h) * d + c2] = run;
            }
        }
    }
    for (int j = tid; j < len; j += GT) dbeta[(size_t)(t0 + j) * H + h] = sdb[j];
}

}  // namespace bwd

namespace {
// The chunk the backward runs for a requested one.  At d = 128 it is always
// 16 tokens (the fp32 MFMA kernels): the chunkwise form is exact for any
// chunk, so the requested size changes only the rounding order.
int bwd_run_chunk(int d, int chunk) {
    return d == bwd::MD && (chunk == 16 || chunk == 32 || chunk == 64) ? bwd::MC : chunk;
}
}  // namespace

bool bwd_supported(int dk, int dv, int chunk_requested) {
    if (dk != dv || !(dk == 16 || dk == 32 || dk == 64 || dk == 128)) return false;
    if (!(chunk_requested == 16 || chunk_requested == 32 || chunk_requested == 64)) return false;
    const int chunk = bwd_run_chunk(dk, chunk_requested);
    if (chunk * dk > bwd::MAX_BLOCK) return false;   // one fetched block per [C][d] operand
    const size_t cap = 163840 / sizeof(float);
    return (size_t)bwd::prep_layout(dk, chunk).total <= cap &&
           (size_t)bwd::chain_layout(dk, chunk).total <= cap &&
           (size_t)bwd::grad_layout(dk, chunk).total <= cap;
}

bool f32_mfma_applies(int dk, int dv, bool bf16, Gate, InputForm) {
    return !bf16 && dk == bwd::MD && dv == bwd::MD;
}

namespace bwd {
// The fp32 prefill's workspace per (chunk slot, head): R, Kbar, Qbar [C][d];
// T, K~, H [C][C]; e^{G_C} [d], as the prep kernel writes them.
__host__ __device__ inline size_t fwd_floats_per_slot() {
    return 3 * (size_t)MC * MD + 3 * (size_t)MC * MC + MD;
}
inline Ws fwd_ws_layout(float *base, size_t slots, int heads) {
    const size_t n = slots * heads, cd = n * MC * MD, cc = n * MC * MC;
    Ws w;
    w.S = w.dS = w.Z = w.dZ = nullptr;   // the prep kernel writes none of these
    w.R = base;
    w.Kb = w.R + cd;
    w.Qb = w.Kb + cd;
    w.T = w.Qb + cd;
    w.Kt = w.T + cc;
    w.Hm = w.Kt + cc;
    w.gC = w.Hm + cc;
    return w;
}
}  // namespace bwd

size_t f32_mfma_workspace_bytes(int64_t total_tokens, int64_t n_seqs, int heads) {
    return bwd::n_slots(total_tokens, (int)n_seqs, bwd::MC) * heads * bwd::fwd_floats_per_slot() *
           sizeof(float);
}

hipError_t launch_chunk_fwd_f32_mfma(const ChunkProblem &p) {
    using namespace bwd;
    const int64_t total = p.cu ? (int64_t)p.seqlen : (int64_t)p.n_seqs * p.seqlen;
    const size_t slots = n_slots(total, p.n_seqs, MC);
    const Ws ws = fwd_ws_layout(static_cast<float *>(p.workspace), slots, p.heads);
    const size_t lp = (size_t)prep_layout(MD, MC).total * sizeof(float);
    const void *prep = p.gate == Gate::PerChannel
                           ? reinterpret_cast<const void *>(&kda_bwd_prep_kernel<MC, MD, float, 0>)
                       : p.gate == Gate::Scalar
                           ? reinterpret_cast<const void *>(&kda_bwd_prep_kernel<MC, MD, float, 1>)
                           : reinterpret_cast<const void *>(&kda_bwd_prep_kernel<MC, MD, float, 2>);
    hipError_t e = hipFuncSetAttribute(prep, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lp);
    if (e != hipSuccess) return e;
    const int64_t n_pairs = (int64_t)p.n_seqs * p.heads;
    const int64_t chain_blocks = (n_pairs + 7) / 8 * 8 * (MD / TV);
    if (!launch_fits((int64_t)(slots * p.heads), THREADS) || !launch_fits(chain_blocks, MTP))
        return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)(slots * p.heads));
    const float *q = static_cast<const float *>(p.q), *k = static_cast<const float *>(p.k);
    const int form = p.form.flags();
    const float eps = p.form.eps;
    if (p.gate == Gate::PerChannel)
        hipLaunchKernelGGL((kda_bwd_prep_kernel<MC, MD, float, 0>), grid, dim3(THREADS), lp,
                           p.stream, q, k, p.g, p.beta, p.scale, p.heads, p.seqlen, p.cu,
                           p.n_seqs, ws, form, eps);
    else if (p.gate == Gate::Scalar)
        hipLaunchKernelGGL((kda_bwd_prep_kernel<MC, MD, float, 1>), grid, dim3(THREADS), lp,
                           p.stream, q, k, p.g, p.beta, p.scale, p.heads, p.seqlen, p.cu,
                           p.n_seqs, ws, form, eps);
    else
        hipLaunchKernelGGL((kda_bwd_prep_kernel<MC, MD, float, 2>), grid, dim3(THREADS), lp,
                           p.stream, q, k, nullptr, p.beta, p.scale, p.heads, p.seqlen, p.cu,
                           p.n_seqs, ws, form, eps);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kda_fwd_f32_chain_kernel, dim3((unsigned)chain_blocks), dim3(MTP), 0,
                       p.stream, static_cast<const float *>(p.v), p.beta, p.heads, p.seqlen, p.cu,
                       (int)n_pairs, p.s0, static_cast<float *>(p.o), p.s_final, ws, form);
    return hipGetLastError();
}

size_t bwd_workspace_bytes(int64_t total_tokens, int n_seqs, int heads, int d,
                           int chunk_requested) {
    const int chunk = bwd_run_chunk(d, chunk_requested);
    const size_t slots = bwd::n_slots(total_tokens, n_seqs, chunk);
    return slots * heads * bwd::ws_floats_per_slot(d, chunk) * sizeof(float);
}

namespace {
template <int C, int D, typename In>
hipError_t launch_bwd_cdt(const ChunkBwdProblem &p, const bwd::Ws &ws, size_t slots) {
    using namespace bwd;
    const In *q = static_cast<const In *>(p.q), *k = static_cast<const In *>(p.k);
    const In *v = static_cast<const In *>(p.v), *dout = static_cast<const In *>(p.dout);
    const size_t lp = (size_t)prep_layout(D, C).total * sizeof(float);
    const size_t lc = (size_t)chain_layout(D, C).total * sizeof(float);
    const size_t lg = (size_t)grad_layout(D, C).total * sizeof(float);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&kda_bwd_prep_kernel<C, D, In>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lp);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&kda_bwd_chain_kernel<C, D, In>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lc);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&kda_bwd_grad_kernel<C, D, In>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lg);
    if (e != hipSuccess) return e;
    const int64_t n_pairs = (int64_t)p.n_seqs * p.heads;
    const int64_t chain_blocks = (n_pairs + 7) / 8 * 8 * (D / TV);
    if (!launch_fits((int64_t)slots * p.heads, GT) ||
        !launch_fits(chain_blocks, (C == MC && D == MD) ? MTP : CT))
        return hipErrorInvalidConfiguration;
    const dim3 per_chunk((unsigned)(slots * p.heads));
    hipLaunchKernelGGL((kda_bwd_prep_kernel<C, D, In>), per_chunk, dim3(THREADS), lp, p.stream, q,
                       k, p.g, p.beta, p.scale, p.heads, p.seqlen, p.cu, p.n_seqs, ws, 0, 0.f);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (C == MC && D == MD) {
        hipLaunchKernelGGL((kda_bwd_chain_mfma_kernel<In>), dim3((unsigned)chain_blocks),
                           dim3(MTP), 0, p.stream, v, p.beta, p.heads, p.seqlen, p.cu, (int)n_pairs,
                           p.s0, p.dfinal, dout, p.ds0, ws);
    } else {
        hipLaunchKernelGGL((kda_bwd_chain_kernel<C, D, In>), dim3((unsigned)chain_blocks),
                           dim3(CT), lc, p.stream, v, p.beta, p.heads, p.seqlen, p.cu, (int)n_pairs,
                           p.s0, p.dfinal, dout, p.ds0, ws);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((kda_bwd_grad_kernel<C, D, In>), per_chunk, dim3(GT), lg, p.stream, q,
                       k, v, p.g, p.beta, p.scale, p.heads, p.seqlen, p.cu, p.n_seqs, dout,
                       p.dq, p.dk, p.dv, p.dg, p.dbeta, ws);
    return hipGetLastError();
}
template <int C, int D>
hipError_t launch_bwd_cd(const ChunkBwdProblem &p, const bwd::Ws &ws, size_t slots) {
    return p.bf16 ? launch_bwd_cdt<C, D, bf16_t>(p, ws, slots)
                  : launch_bwd_cdt<C, D, float>(p, ws, slots);
}
}  // namespace

hipError_t launch_chunk_bwd(const ChunkBwdProblem &p) {
    const int64_t total = p.cu ? (int64_t)p.seqlen : (int64_t)p.n_seqs * p.seqlen;
    const int chunk = bwd_run_chunk(p.d, p.chunk);
    const size_t slots = bwd::n_slots(total, p.n_seqs, chunk);
    const bwd::Ws ws = bwd::ws_layout(p.work, slots, p.heads, p.d, chunk);
    // The (d, chunk) pairs bwd_supported accepts, as they run.
    switch (p.d * 1000 + chunk) {
    case 16016: return launch_bwd_cd<16, 16>(p, ws, slots);
    case 16032: return launch_bwd_cd<32, 16>(p, ws, slots);
    case 16064: return launch_bwd_cd<64, 16>(p, ws, slots);
    case 32016: return launch_bwd_cd<16, 32>(p, ws, slots);
    case 32032: return launch_bwd_cd<32, 32>(p, ws, slots);
    case 64016: return launch_bwd_cd<16, 64>(p, ws, slots);
    case 64032: return launch_bwd_cd<32, 64>(p, ws, slots);
    case 128016: return launch_bwd_cd<16, 128>(p, ws, slots);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
