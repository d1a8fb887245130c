// kda_chunk_f32.hip -- chunkwise KDA prefill in fp32 for fp32 storage and
// small widths (d_k = d_v = d in {16, 32, 64}, C in {16, 32, 64}; up to 148 KB
// of LDS, within gfx950's 160 KB per workgroup).
//
// Same chunk algebra as the MFMA path ("Understanding Kimi Delta Attention",
// sections "The triangular system" and "Putting the chunks together", with
// A = -A_page so that (I + A) T = I), evaluated entirely in fp32 on the vector
// ALUs with every chunk operand resident in LDS.  This is the path whose
// accuracy budget is 1e-4; its speed is not a target.  One workgroup handles
// one (sequence, head) and walks its chunks in order with the state in LDS.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace f32_path {

constexpr int THREADS = 256;

struct Lds {
    int q, k, G, v, beta, nrm, A, T, W, U, S, total;   // offsets in floats (H reuses A)
};

__host__ __device__ inline Lds lds_layout(int dk, int dv, int C) {
    Lds L;
    int o = 0;
    L.q = o; o += C * dk;
    L.k = o; o += C * dk;
    L.G = o; o += C * dk;
    L.v = o; o += C * dv;
    L.beta = o; o += C;
    L.nrm = o; o += 2 * C;   // inverse L2 norms of the rows of k and q
    L.A = o; o += C * C;
    L.T = o; o += C * C;
    L.W = o; o += C * dk;
    L.U = o; o += C * dv;
    L.S = o; o += dk * dv;
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
    float *sq = sm + L.q, *sk = sm + L.k, *sG = sm + L.G, *sv = sm + L.v, *sb = sm + L.beta;
    float *snrm = sm + L.nrm;
    float *sA = sm + L.A, *sT = sm + L.T, *sW = sm + L.W, *sU = sm + L.U;
    float *sH = sA;   // H is built once T no longer needs A
    float *sS = sm + L.S;

    const int n = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
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
    for (int e = tid; e < dk * dv; e += THREADS) sS[e] = s0 ? s0[pair * dk * dv + e] : 0.f;
    __syncthreads();

    for (int t0 = ts; t0 < te; t0 += C) {
        const int len = min(C, te - t0);
        // Load the chunk (rows >= len are zero: they contribute nothing).
        for (int e = tid; e < C * dk; e += THREADS) {
            const int i = e / dk, c = e - i * dk;
            const bool ok = i < len;
            const size_t a = ((size_t)(t0 + i) * H + h) * dk + c;
            sq[e] = ok ? q[a] : 0.f;
            sk[e] = ok ? k[a] : 0.f;
            // gate 0: log-decay per channel; 1: one per (token, head); 2: none
            float gv = 0.f;
            if (ok && gate != 2) {
                gv = gate == 0 ? g[a] : g[(size_t)(t0 + i) * H + h];
                if (form & kFormGateLogit) gv = log_sigmoid(gv);
            }
            sG[e] = gv;
        }
        for (int e = tid; e < C * dv; e += THREADS) {
            const int i = e / dv, c = e - i * dv;
            sv[e] = i < len ? v[((size_t)(t0 + i) * H + h) * dv + c] : 0.f;
        }
        for (int i = tid; i < C; i += THREADS) {
            float b = i < len ? beta[(size_t)(t0 + i) * H + h] : 0.f;
            if ((form & kFormBetaLogit) && i < len) b = sigmoid(b);
            sb[i] = b;
        }
        __syncthreads();
        if (form & kFormL2Norm) {   // q, k rows divided by sqrt(sum of squares + eps)
            for (int x = tid; x < 2 * C; x += THREADS) {
                const float *row = (x < C ? sk : sq) + (x % C) * dk;
                float ss = 0.f;
                for (int c = 0; c < dk; ++c) ss += row[c] * row[c];
                snrm[x] = 1.f / sqrtf(ss + eps);
            }
            __syncthreads();
            for (int e = tid; e < C * dk; e += THREADS) {
                const int i = e / dk;
                sk[e] *= snrm[i];
                sq[e] *= snrm[C + i];
            }
            __syncthreads();
        }
        // G: inclusive cumulative log-decay per channel.
        for (int c = tid; c < dk; c += THREADS) {
            float run = 0.f;
            for (int i = 0; i < C; ++i) {
                run += sG[i * dk + c];
                sG[i * dk + c] = run;
            }
        }
        __syncthreads();
        // A_ij = beta_i sum_c k_ic k_jc e^{G_ic - G_jc}  (j < i).
        for (int e = tid; e < C * C; e += THREADS) {
            const int i = e / C, j = e - i * C;
            float a = 0.f;
            if (j < i)
                for (int c = 0; c < dk; ++c)
                    a += sk[i * dk + c] * expf(sG[i * dk + c] - sG[j * dk + c]) * sk[j * dk + c];
            sA[e] = (j < i) ? sb[i] * a : 0.f;
        }
        __syncthreads();
        // T = (I + A)^{-1}: column j by forward substitution (one thread per column).
        for (int j = tid; j < C; j += THREADS) {
            for (int i = 0; i < C; ++i) {
                float s = (i == j) ? 1.f : 0.f;
                for (int kk = j; kk < i; ++kk) s -= sA[i * C + kk] * sT[kk * C + j];
                sT[i * C + j] = (i < j) ? 0.f : s;
            }
        }
        __syncthreads();
        // H_ij = s sum_c q_ic k_jc e^{G_ic - G_jc}  (j <= i), into A's storage.
        for (int e = tid; e < C * C; e += THREADS) {
            const int i = e / C, j = e - i * C;
            float hh = 0.f;
            if (j <= i)
                for (int c = 0; c < dk; ++c)
                    hh += sq[i * dk + c] * expf(sG[i * dk + c] - sG[j * dk + c]) * sk[j * dk + c];
            sH[e] = (j <= i) ? scale * hh : 0.f;
        }
        __syncthreads();
        // W = T Diag(beta) (K e^{G}),  U = T Diag(beta) V.
        for (int e = tid; e < C * dk; e += THREADS) {
            const int i = e / dk, c = e - i * dk;
            float acc = 0.f;
            for (int j = 0; j <= i; ++j)
                acc += sT[i * C + j] * sb[j] * sk[j * dk + c] * expf(sG[j * dk + c]);
            sW[e] = acc;
        }
        for (int e = tid; e < C * dv; e += THREADS) {
            const int i = e / dv, c = e - i * dv;
            float acc = 0.f;
            for (int j = 0; j <= i; ++j) acc += sT[i * C + j] * sb[j] * sv[j * dv + c];
            sU[e] = acc;
        }
        __syncthreads();
        // Z = U - W S (into sU).
        for (int e = tid; e < C * dv; e += THREADS) {
            const int i = e / dv, c = e - i * dv;
            float acc = sU[e];
            for (int r = 0; r < dk; ++r) acc -= sW[i * dk + r] * sS[r * dv + c];
            sU[e] = acc;
        }
        __syncthreads();
        // O = (s Q e^{G}) S + H Z.
        for (int e = tid; e < C * dv; e += THREADS) {
            const int i = e / dv, c = e - i * dv;
            if (i >= len) continue;
            float acc = 0.f;
            for (int r = 0; r < dk; ++r)
                acc += scale * sq[i * dk + r] * expf(sG[i * dk + r]) * sS[r * dv + c];
            for (int j = 0; j <= i; ++j) acc += sH[i * C + j] * sU[j * dv + c];
            o[((size_t)(t0 + i) * H + h) * dv + c] = acc;
        }
        __syncthreads();
        // S <- Diag(e^{G_C}) S + (K e^{G_C - G})^T Z.
        for (int e = tid; e < dk * dv; e += THREADS) {
            const int r = e / dv, c = e - r * dv;
            const float gl = sG[(C - 1) * dk + r];
            float acc = expf(gl) * sS[e];
            for (int j = 0; j < C; ++j)
                acc += sk[j * dk + r] * expf(gl - sG[j * dk + r]) * sU[j * dv + c];
            sS[e] = acc;
        }
        __syncthreads();
    }
    if (s_final)
        for (int e = tid; e < dk * dv; e += THREADS) s_final[pair * dk * dv + e] = sS[e];
}

}  // namespace f32_path

bool f32_path_supported(int dk, int dv, int chunk, bool bf16) {
    if (bf16 || dk != dv) return false;
    if (!(dk == 16 || dk == 32 || dk == 64)) return false;
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
    if (!launch_fits((int64_t)p.n_seqs * p.heads, THREADS)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kda_chunk_f32_kernel, dim3(p.n_seqs * p.heads), dim3(THREADS), lds,
                       p.stream, static_cast<const float *>(p.q), static_cast<const float *>(p.k),
                       static_cast<const float *>(p.v), p.g, (int)p.gate, p.beta, p.scale,
                       p.form.flags(), p.form.eps, p.heads, p.dk, p.dv, p.chunk, p.seqlen, p.cu,
                       p.s0, p.s_final, static_cast<float *>(p.o));
    return hipGetLastError();
}

}  // namespace kda
