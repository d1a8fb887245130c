// kda_chunk_f32.hip -- chunkwise KDA prefill in fp32 for fp32 storage:
// d_k = d_v = d in {16, 32, 64} with C in {16, 32, 64}, and d = 128 with
// C in {16, 32, 64} (up to about 150 KB of LDS, within gfx950's 160 KB per
// workgroup).
//
// Same chunk algebra as the MFMA path ("Understanding Kimi Delta Attention",
// sections "The triangular system" and "Putting the chunks together", with
// A = -A_page so that (I + A) T = I), evaluated entirely in fp32 on the vector
// ALUs with every chunk operand resident in LDS.  This is the path whose
// accuracy budget is 1e-4; its speed is not a target.  At d = 128 it serves
// only the no-allocation entry point on problems whose fp32 MFMA factors
// would not fit its buffer (it needs no workspace); every other fp32 call at
// d = 128 takes the MFMA path in kda_chunk_bwd.hip.  One workgroup handles
// one (sequence, head, value tile) and walks its chunks in order with its
// columns of the state in LDS.  Value columns evolve independently, so the
// tiles need no communication; each recomputes the value-independent chunk
// factors (A, T, H) for itself.
//
// Per chunk, with L_j = k_j e^{G_j}:  Z = U - W S = T Diag(beta) (V - L S),
// so neither W nor U is ever formed: Y = V - L S overwrites the value tile,
// then Z = T Diag(beta) Y, O = (s Q e^{G}) S + H Z, and
// S <- Diag(e^{G_C}) S + (K e^{G_C - G})^T Z.  Every decay factor is the
// exponential of a difference of cumulative logs (or of G itself), as the
// derivation recommends, so any finite log-decay stays in range.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace f32_path {

constexpr int THREADS = 256;

// Value columns per workgroup: the whole width up to 64, else 16 (so the
// q, k, G rows of a 64-token chunk at d = 128 still fit in LDS).
__host__ __device__ inline int value_tile(int dv) { return dv <= 64 ? dv : 16; }

struct Lds {
    int P, VP, CP;                                      // row pitches (floats)
    int q, k, G, v, z, beta, nrm, A, T, S, total;       // offsets in floats (H reuses A)
};

// Rows are padded by one float so that threads walking different rows of the
// same column hit different LDS banks.
__host__ __device__ inline Lds lds_layout(int dk, int dv, int C) {
    Lds L;
    const int VT = value_tile(dv);
    L.P = dk + 1;
    L.VP = VT + 1;
    L.CP = C + 1;
    int o = 0;
    L.q = o; o += C * L.P;
    L.k = o; o += C * L.P;
    L.G = o; o += C * L.P;
    L.v = o; o += C * L.VP;   // v, then Y = V - L S
    L.z = o; o += C * L.VP;   // Z = T Diag(beta) Y
    L.beta = o; o += C;
    L.nrm = o; o += 2 * C;    // inverse L2 norms of the rows of k and q
    L.A = o; o += C * L.CP;
    L.T = o; o += C * L.CP;
    L.S = o; o += dk * L.VP;
    L.total = o;
    return L;
}

__global__ __launch_bounds__(THREADS) void kda_chunk_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ g, int gate, const float *__restrict__ beta, float scale, int form,
    float eps, int H, int dk, int dv, int C, int row_len, const int32_t *__restrict__ cu,
    const float *__restrict__ s0, float *__restrict__ s_final, float *__restrict__ o) {
    extern __shared__ float sm[];
    const Lds L = lds_layout(dk, dv, C);
    const int P = L.P, VP = L.VP, CP = L.CP;
    const int VT = value_tile(dv), n_vt = dv / VT;
    float *sq = sm + L.q, *sk = sm + L.k, *sG = sm + L.G, *sv = sm + L.v, *sz = sm + L.z;
    float *sb = sm + L.beta, *snrm = sm + L.nrm;
    float *sA = sm + L.A, *sT = sm + L.T, *sS = sm + L.S;
    float *sH = sA;   // H is built once T no longer needs A

    const int vt = blockIdx.x % n_vt, pair_id = blockIdx.x / n_vt;
    const int n = pair_id / H, h = pair_id - n * H;
    const int c0 = vt * VT;   // first value column of this tile
    const int tid = threadIdx.x;
    int ts, te;
    if (cu) {
        // Clamped so that a malformed cu_seqlens still stays inside [0, T).
        const int T = row_len;
        ts = min(T, max(0, cu[n]));
        te = min(T, max(ts, cu[n + 1]));
    } else {
        ts = n * row_len;
        te = ts + row_len;
    }
    const size_t pair = (size_t)n * H + h;
    for (int e = tid; e < dk * VT; e += THREADS) {
        const int r = e / VT, c = e - r * VT;
        sS[r * VP + c] = s0 ? s0[pair * dk * dv + (size_t)r * dv + c0 + c] : 0.f;
    }
    __syncthreads();

    for (int t0 = ts; t0 < te; t0 += C) {
        const int len = min(C, te - t0);
        // Load the chunk (rows >= len are zero: they contribute nothing).
        for (int e = tid; e < C * dk; e += THREADS) {
            const int i = e / dk, c = e - i * dk;
            const bool ok = i < len;
            const size_t a = ((size_t)(t0 + i) * H + h) * dk + c;
            sq[i * P + c] = ok ? q[a] : 0.f;
            sk[i * P + c] = ok ? k[a] : 0.f;
            // gate 0: log-decay per channel; 1: one per (token, head); 2: none
            float gv = 0.f;
            if (ok && gate != 2) {
                gv = gate == 0 ? g[a] : g[(size_t)(t0 + i) * H + h];
                if (form & kFormGateLogit) gv = log_sigmoid(gv);
            }
            sG[i * P + c] = gv;
        }
        for (int e = tid; e < C * VT; e += THREADS) {
            const int i = e / VT, c = e - i * VT;
            sv[i * VP + c] = i < len ? v[((size_t)(t0 + i) * H + h) * dv + c0 + c] : 0.f;
        }
        for (int i = tid; i < C; i += THREADS) {
            float b = i < len ? beta[(size_t)(t0 + i) * H + h] : 0.f;
            if ((form & kFormBetaLogit) && i < len) b = sigmoid(b);
            sb[i] = b;
        }
        __syncthreads();
        if (form & kFormL2Norm) {   // q, k rows divided by sqrt(sum of squares + eps)
            for (int x = tid; x < 2 * C; x += THREADS) {
                const float *row = (x < C ? sk : sq) + (x % C) * P;
                float ss = 0.f;
                for (int c = 0; c < dk; ++c) ss += row[c] * row[c];
                snrm[x] = 1.f / sqrtf(ss + eps);
            }
            __syncthreads();
            for (int e = tid; e < C * dk; e += THREADS) {
                const int i = e / dk, c = e - i * dk;
                sk[i * P + c] *= snrm[i];
                sq[i * P + c] *= snrm[C + i];
            }
            __syncthreads();
        }
        // G: inclusive cumulative log-decay per channel.
        for (int c = tid; c < dk; c += THREADS) {
            float run = 0.f;
            for (int i = 0; i < C; ++i) {
                run += sG[i * P + c];
                sG[i * P + c] = run;
            }
        }
        __syncthreads();
        // A_ij = beta_i sum_c k_ic k_jc e^{G_ic - G_jc}  (j < i).
        for (int e = tid; e < C * C; e += THREADS) {
            const int i = e / C, j = e - i * C;
            float a = 0.f;
            if (j < i)
                for (int c = 0; c < dk; ++c)
                    a += sk[i * P + c] * expf(sG[i * P + c] - sG[j * P + c]) * sk[j * P + c];
            sA[i * CP + j] = (j < i) ? sb[i] * a : 0.f;
        }
        __syncthreads();
        // T = (I + A)^{-1}: column j by forward substitution (one thread per column).
        for (int j = tid; j < C; j += THREADS) {
            for (int i = 0; i < C; ++i) {
                float s = (i == j) ? 1.f : 0.f;
                for (int kk = j; kk < i; ++kk) s -= sA[i * CP + kk] * sT[kk * CP + j];
                sT[i * CP + j] = (i < j) ? 0.f : s;
            }
        }
        // Y = V - L S (in place of V), L_j = k_j e^{G_j}: independent of A and T.
        for (int e = tid; e < C * VT; e += THREADS) {
            const int j = e / VT, c = e - j * VT;
            float acc = sv[j * VP + c];
            for (int r = 0; r < dk; ++r)
                acc -= sk[j * P + r] * expf(sG[j * P + r]) * sS[r * VP + c];
            sv[j * VP + c] = acc;
        }
        __syncthreads();
        // H_ij = s sum_c q_ic k_jc e^{G_ic - G_jc}  (j <= i), into A's storage;
        // Z = T Diag(beta) Y alongside (it reads T and Y only).
        for (int e = tid; e < C * C; e += THREADS) {
            const int i = e / C, j = e - i * C;
            float hh = 0.f;
            if (j <= i)
                for (int c = 0; c < dk; ++c)
                    hh += sq[i * P + c] * expf(sG[i * P + c] - sG[j * P + c]) * sk[j * P + c];
            sH[i * CP + j] = (j <= i) ? scale * hh : 0.f;
        }
        for (int e = tid; e < C * VT; e += THREADS) {
            const int i = e / VT, c = e - i * VT;
            float acc = 0.f;
            for (int j = 0; j <= i; ++j) acc += sT[i * CP + j] * sb[j] * sv[j * VP + c];
            sz[i * VP + c] = acc;
        }
        __syncthreads();
        // O = (s Q e^{G}) S + H Z.
        for (int e = tid; e < C * VT; e += THREADS) {
            const int i = e / VT, c = e - i * VT;
            if (i >= len) continue;
            float acc = 0.f;
            for (int r = 0; r < dk; ++r)
                acc += scale * sq[i * P + r] * expf(sG[i * P + r]) * sS[r * VP + c];
            for (int j = 0; j <= i; ++j) acc += sH[i * CP + j] * sz[j * VP + c];
            o[((size_t)(t0 + i) * H + h) * dv + c0 + c] = acc;
        }
        __syncthreads();
        // S <- Diag(e^{G_C}) S + (K e^{G_C - G})^T Z.
        for (int e = tid; e < dk * VT; e += THREADS) {
            const int r = e / VT, c = e - r * VT;
            const float gl = sG[(C - 1) * P + r];
            float acc = expf(gl) * sS[r * VP + c];
            for (int j = 0; j < C; ++j)
                acc += sk[j * P + r] * expf(gl - sG[j * P + r]) * sz[j * VP + c];
            sS[r * VP + c] = acc;
        }
        __syncthreads();
    }
    if (s_final)
        for (int e = tid; e < dk * VT; e += THREADS) {
            const int r = e / VT, c = e - r * VT;
            s_final[pair * dk * dv + (size_t)r * dv + c0 + c] = sS[r * VP + c];
        }
}

}  // namespace f32_path

bool f32_path_supported(int dk, int dv, int chunk, bool bf16) {
    if (bf16 || dk != dv) return false;
    if (!(dk == 16 || dk == 32 || dk == 64 || dk == 128)) return false;
    if (!(chunk == 16 || chunk == 32 || chunk == 64)) return false;
    return (size_t)f32_path::lds_layout(dk, dv, chunk).total * sizeof(float) <= 163840;
}

size_t f32_workspace_bytes(int64_t, int64_t, int, int) { return 0; }

hipError_t launch_chunk_fwd_f32(const ChunkProblem &p) {
    using namespace f32_path;
    const size_t lds = (size_t)lds_layout(p.dk, p.dv, p.chunk).total * sizeof(float);
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&kda_chunk_f32_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const int64_t blocks = (int64_t)p.n_seqs * p.heads * (p.dv / value_tile(p.dv));
    if (!launch_fits(blocks, THREADS)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kda_chunk_f32_kernel, dim3((unsigned)blocks), dim3(THREADS), lds,
                       p.stream, static_cast<const float *>(p.q), static_cast<const float *>(p.k),
                       static_cast<const float *>(p.v), p.g, (int)p.gate, p.beta, p.scale,
                       p.form.flags(), p.form.eps, p.heads, p.dk, p.dv, p.chunk, p.seqlen, p.cu,
                       p.s0, p.s_final, static_cast<float *>(p.o));
    return hipGetLastError();
}

}  // namespace kda
