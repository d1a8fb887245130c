// kda_chunk_bwd_f32.hip -- gradients of the chunkwise KDA prefill in fp32, for
// fp32 storage and small widths (d_k = d_v = d in {16, 32, 64}, chunk C with
// the whole working set in LDS: up to 160 KB).
//
// The pages derive no gradients.  This kernel reverses the chunk algebra of
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
// and the cumulative log-decay G, whose reverse cumulative sum is dg.  The
// chunks are walked in reverse with dS carried across chunk boundaries, just
// as the forward carries S; the chunk-start states come from a forward pass
// over the same sequence that stores them in the workspace.
//
// One workgroup per (sequence, head), every operand in LDS, fp32 on the
// vector ALUs.  This is the small-width path; its speed is not a target.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace bwd_f32 {

constexpr int THREADS = 256;

struct Lds {
    int q, k, G, v, dO, beta, dbeta, S, dS, dSn, Kt, Hm, T, dT, M1, R, Z, dZ, dR, dL, total;
};

__host__ __device__ inline Lds lds_layout(int d, int C) {
    Lds L;
    int o = 0;
    const int cd = C * d, cc = C * C, dd = d * d;
    L.q = o; o += cd;
    L.k = o; o += cd;
    L.G = o; o += cd;
    L.v = o; o += cd;
    L.dO = o; o += cd;
    L.beta = o; o += C;
    L.dbeta = o; o += C;
    L.S = o; o += dd;
    L.dS = o; o += dd;
    L.dSn = o; o += dd;
    L.Kt = o; o += cc;   // K~ (decay-weighted k_i . k_j, j < i), later its gradient
    L.Hm = o; o += cc;   // H, later its gradient
    L.T = o; o += cc;
    L.dT = o; o += cc;
    L.M1 = o; o += cc;   // T^T dT
    L.R = o; o += cd;
    L.Z = o; o += cd;
    L.dZ = o; o += cd;
    L.dR = o; o += cd;   // later the gradient of G
    L.dL = o; o += cd;
    L.total = o;
    return L;
}

// First chunk slot of sequence n in the checkpoint area: floor(start / C) + n.
// Consecutive sequences get disjoint ranges, within T / C + N + 1 slots.
__device__ __forceinline__ int chunk_base(int ts, int n, int C) { return ts / C + n; }

__global__ __launch_bounds__(THREADS) void kda_chunk_bwd_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float scale, int H, int d, int C,
    int row_len, const int32_t *__restrict__ cu, const float *__restrict__ s0,
    const float *__restrict__ dfinal, const float *__restrict__ dout, float *__restrict__ dq,
    float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ dg,
    float *__restrict__ dbeta, float *__restrict__ ds0, float *__restrict__ ckpt) {
    extern __shared__ float sm[];
    const Lds L = lds_layout(d, C);
    float *sq = sm + L.q, *sk = sm + L.k, *sG = sm + L.G, *sv = sm + L.v, *sdO = sm + L.dO;
    float *sb = sm + L.beta, *sdb = sm + L.dbeta;
    float *sS = sm + L.S, *sdS = sm + L.dS, *sdSn = sm + L.dSn;
    float *sKt = sm + L.Kt, *sHm = sm + L.Hm, *sT = sm + L.T, *sdT = sm + L.dT, *sM1 = sm + L.M1;
    float *sR = sm + L.R, *sZ = sm + L.Z, *sdZ = sm + L.dZ, *sdR = sm + L.dR, *sdL = sm + L.dL;
    float *sdG = sdR;

    const int n = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
    const int tid = threadIdx.x;
    const int cd = C * d, dd = d * d;
    int ts, te;
    if (cu) {
        const int T = row_len;   // clamped: a malformed cu_seqlens stays inside [0, T)
        ts = min(T, max(0, cu[n]));
        te = min(T, max(ts, cu[n + 1]));
    } else {
        ts = n * row_len;
        te = ts + row_len;
    }
    const size_t pair = (size_t)n * H + h;
    const int nck = (te - ts + C - 1) / C;
    const int base = chunk_base(ts, n, C);

    // Loads chunk c (rows >= len are zero), G as the inclusive cumulative sum.
    auto load_chunk = [&](int c, bool with_do) {
        const int t0 = ts + c * C, len = min(C, te - t0);
        for (int e = tid; e < cd; e += THREADS) {
            const int i = e / d;
            const bool ok = i < len;
            const size_t a = ((size_t)(t0 + (ok ? i : 0)) * H + h) * d + (e - i * d);
            sq[e] = ok ? q[a] : 0.f;
            sk[e] = ok ? k[a] : 0.f;
            sG[e] = ok ? g[a] : 0.f;
            sv[e] = ok ? v[a] : 0.f;
            if (with_do) sdO[e] = ok ? dout[a] : 0.f;
        }
        for (int i = tid; i < C; i += THREADS) sb[i] = i < len ? beta[(size_t)(t0 + i) * H + h] : 0.f;
        __syncthreads();
        for (int c2 = tid; c2 < d; c2 += THREADS) {
            float run = 0.f;
            for (int i = 0; i < C; ++i) {
                run += sG[i * d + c2];
                sG[i * d + c2] = run;
            }
        }
        __syncthreads();
        return len;
    };
    // K~_ij = sum_c k_ic k_jc e^{G_ic - G_jc} (j < i) and T = (I + Diag(beta) K~)^{-1}.
    auto build_T = [&]() {
        for (int e = tid; e < C * C; e += THREADS) {
            const int i = e / C, j = e - i * C;
            float a = 0.f;
            if (j < i)
                for (int c2 = 0; c2 < d; ++c2)
                    a += sk[i * d + c2] * expf(sG[i * d + c2] - sG[j * d + c2]) * sk[j * d + c2];
            sKt[e] = a;
        }
        __syncthreads();
        for (int j = tid; j < C; j += THREADS)
            for (int i = 0; i < C; ++i) {
                float s = (i == j) ? 1.f : 0.f;
                for (int kk = j; kk < i; ++kk) s -= sb[i] * sKt[i * C + kk] * sT[kk * C + j];
                sT[i * C + j] = (i < j) ? 0.f : s;
            }
        __syncthreads();
    };
    // R = T Diag(beta) (K e^{G}), Z = T Diag(beta) V - R S.
    auto build_RZ = [&]() {
        for (int e = tid; e < cd; e += THREADS) {
            const int i = e / d, c2 = e - i * d;
            float r = 0.f, u = 0.f;
            for (int j = 0; j <= i; ++j) {
                const float tb = sT[i * C + j] * sb[j];
                r += tb * sk[j * d + c2] * expf(sG[j * d + c2]);
                u += tb * sv[j * d + c2];
            }
            sR[e] = r;
            sZ[e] = u;
        }
        __syncthreads();
        for (int e = tid; e < cd; e += THREADS) {
            const int i = e / d, c2 = e - i * d;
            float z = sZ[e];
            for (int r = 0; r < d; ++r) z -= sR[i * d + r] * sS[r * d + c2];
            sdZ[e] = z;   // staged: Z is rewritten below once every thread has read sZ
        }
        __syncthreads();
        for (int e = tid; e < cd; e += THREADS) sZ[e] = sdZ[e];
        __syncthreads();
    };

    // ---- forward over the sequence: chunk-start states into the workspace ---------
    for (int e = tid; e < dd; e += THREADS) sS[e] = s0 ? s0[pair * dd + e] : 0.f;
    __syncthreads();
    for (int c = 0; c < nck; ++c) {
        float *slot = ckpt + ((size_t)(base + c) * H + h) * dd;
        for (int e = tid; e < dd; e += THREADS) slot[e] = sS[e];
        load_chunk(c, false);
        build_T();
        build_RZ();
        // S <- Diag(e^{G_C}) S + (K e^{G_C - G})^T Z  (padding rows add nothing)
        for (int e = tid; e < dd; e += THREADS) {
            const int r = e / d, c2 = e - r * d;
            const float gl = sG[(C - 1) * d + r];
            float acc = expf(gl) * sS[e];
            for (int j = 0; j < C; ++j) acc += sk[j * d + r] * expf(gl - sG[j * d + r]) * sZ[j * d + c2];
            sdSn[e] = acc;
        }
        __syncthreads();
        for (int e = tid; e < dd; e += THREADS) sS[e] = sdSn[e];
        __syncthreads();
    }

    // ---- backward over the chunks, last first ----------------------------------------
    for (int e = tid; e < dd; e += THREADS) sdS[e] = dfinal ? dfinal[pair * dd + e] : 0.f;
    __syncthreads();
    for (int c = nck - 1; c >= 0; --c) {
        const float *slot = ckpt + ((size_t)(base + c) * H + h) * dd;
        for (int e = tid; e < dd; e += THREADS) sS[e] = slot[e];
        const int len = load_chunk(c, true);
        const int t0 = ts + c * C;
        build_T();
        // H_ij = s sum_c q_ic k_jc e^{G_ic - G_jc} (j <= i)
        for (int e = tid; e < C * C; e += THREADS) {
            const int i = e / C, j = e - i * C;
            float hh = 0.f;
            if (j <= i)
                for (int c2 = 0; c2 < d; ++c2)
                    hh += sq[i * d + c2] * expf(sG[i * d + c2] - sG[j * d + c2]) * sk[j * d + c2];
            sHm[e] = scale * hh;
        }
        build_RZ();
        // dZ = Kbar dS' + H^T dO, Kbar_ir = k_ir e^{G_C,r - G_ir}
        for (int e = tid; e < cd; e += THREADS) {
            const int i = e / d, c2 = e - i * d;
            float z = 0.f;
            for (int r = 0; r < d; ++r)
                z += sk[i * d + r] * expf(sG[(C - 1) * d + r] - sG[i * d + r]) * sdS[r * d + c2];
            for (int i2 = i; i2 < C; ++i2) z += sHm[i2 * C + i] * sdO[i2 * d + c2];
            sdZ[e] = z;
        }
        __syncthreads();
        // dR = -dZ S^T;  dS = Diag(e^{G_C}) dS' + Qbar^T dO - R^T dZ (into dSn)
        for (int e = tid; e < cd; e += THREADS) {
            const int i = e / d, r = e - i * d;
            float a = 0.f;
            for (int c2 = 0; c2 < d; ++c2) a += sdZ[i * d + c2] * sS[r * d + c2];
            sdR[e] = -a;
        }
        for (int e = tid; e < dd; e += THREADS) {
            const int r = e / d, c2 = e - r * d;
            float a = expf(sG[(C - 1) * d + r]) * sdS[e];
            for (int i = 0; i < C; ++i)
                a += scale * sq[i * d + r] * expf(sG[i * d + r]) * sdO[i * d + c2] -
                     sR[i * d + r] * sdZ[i * d + c2];
            sdSn[e] = a;
        }
        __syncthreads();
        // dT = dZ (BV)^T + dR (BL)^T;  dH = dO Z^T (j <= i), into H's storage
        for (int e = tid; e < C * C; e += THREADS) {
            const int i = e / C, j = e - i * C;
            float a = 0.f;
            for (int c2 = 0; c2 < d; ++c2)
                a += sb[j] * (sdZ[i * d + c2] * sv[j * d + c2] +
                              sdR[i * d + c2] * sk[j * d + c2] * expf(sG[j * d + c2]));
            sdT[e] = a;
            float hh = 0.f;
            if (j <= i)
                for (int c2 = 0; c2 < d; ++c2) hh += sdO[i * d + c2] * sZ[j * d + c2];
            sHm[e] = hh;
        }
        // dBV = T^T dZ (into R's storage: R is no longer needed), dBL = T^T dR
        for (int e = tid; e < cd; e += THREADS) {
            const int j = e / d, c2 = e - j * d;
            float bv = 0.f, bl = 0.f;
            for (int i = j; i < C; ++i) {
                bv += sT[i * C + j] * sdZ[i * d + c2];
                bl += sT[i * C + j] * sdR[i * d + c2];
            }
            sR[e] = bv;
            sdL[e] = bl;
        }
        __syncthreads();
        // dbeta_j = dBV_j . v_j + dBL_j . L_j;  M1 = T^T dT
        for (int j = tid; j < C; j += THREADS) {
            float s = 0.f;
            for (int c2 = 0; c2 < d; ++c2)
                s += sR[j * d + c2] * sv[j * d + c2] +
                     sdL[j * d + c2] * sk[j * d + c2] * expf(sG[j * d + c2]);
            sdb[j] = s;
        }
        for (int e = tid; e < C * C; e += THREADS) {
            const int i = e / C, j = e - i * C;
            float a = 0.f;
            for (int a2 = i; a2 < C; ++a2) a += sT[a2 * C + i] * sdT[a2 * C + j];
            sM1[e] = a;
        }
        __syncthreads();
        // dv = beta dBV;  dL = beta dBL (in place);
        // dA = M1 T^T (strictly lower), dbeta_i -= sum_j dA_ij K~_ij,
        // dK~_ij = -beta_i dA_ij into K~'s storage (one thread per row)
        for (int e = tid; e < cd; e += THREADS) {
            const int j = e / d;
            if (j < len) dv[((size_t)(t0 + j) * H + h) * d + (e - j * d)] = sb[j] * sR[e];
            sdL[e] *= sb[j];
        }
        for (int i = tid; i < C; i += THREADS) {
            float s = 0.f;
            for (int j = 0; j < i; ++j) {
                float a = 0.f;
                for (int b = 0; b <= j; ++b) a += sM1[i * C + b] * sT[j * C + b];
                s += a * sKt[i * C + j];
                sKt[i * C + j] = -sb[i] * a;
            }
            for (int j = i; j < C; ++j) sKt[i * C + j] = 0.f;
            sdb[i] -= s;
        }
        __syncthreads();
        // Per (row x, channel c): the decay-weighted products of K~ and H give
        //   P1 = sum_{j<x} dK~_xj k_jc E_xj,  P2 = sum_{i>x} dK~_ix k_ic E_ix,
        //   P3 = sum_{j<=x} dH_xj k_jc E_xj,  P4 = sum_{i>=x} dH_ix (s q_ic) E_ix,
        // with E_ij = e^{G_ic - G_jc}; then the direct uses of e^{G} in Qbar, L, Kbar.
        for (int e = tid; e < cd; e += THREADS) {
            const int x = e / d, c2 = e - x * d;
            const float Gx = sG[e], kx = sk[e], qx = scale * sq[e];
            float P1 = 0.f, P2 = 0.f, P3 = 0.f, P4 = 0.f;
            for (int j = 0; j <= x; ++j) {
                const float E = expf(Gx - sG[j * d + c2]);
                if (j < x) P1 += sKt[x * C + j] * sk[j * d + c2] * E;
                P3 += sHm[x * C + j] * sk[j * d + c2] * E;
            }
            for (int i = x; i < C; ++i) {
                const float E = expf(sG[i * d + c2] - Gx);
                if (i > x) P2 += sKt[i * C + x] * sk[i * d + c2] * E;
                P4 += sHm[i * C + x] * scale * sq[i * d + c2] * E;
            }
            float dQb = 0.f, dKb = 0.f;   // (dO S^T)_xc, (Z dS'^T)_xc
            for (int c3 = 0; c3 < d; ++c3) {
                dQb += sdO[x * d + c3] * sS[c2 * d + c3];
                dKb += sZ[x * d + c3] * sdS[c2 * d + c3];
            }
            const float eG = expf(Gx), eK = expf(sG[(C - 1) * d + c2] - Gx);
            const float dqs = P3 + dQb * eG;
            const float dkx = P1 + P2 + P4 + sdL[e] * eG + dKb * eK;
            const float dGx = kx * (P1 - P2 - P4) + qx * P3 + dQb * qx * eG + sdL[e] * kx * eG -
                              dKb * kx * eK;
            if (x < len) {
                const size_t a = ((size_t)(t0 + x) * H + h) * d + c2;
                dq[a] = scale * dqs;
                dk[a] = dkx;
            }
            sdG[e] = dGx;
            sdL[e] = dKb * kx * eK;   // Kbar-term of dG_C, summed over rows below
        }
        __syncthreads();
        // dG_C = e^{G_C} rowsum(dS' . S) + sum_x dKbar_x Kbar_x joins the last
        // valid row; dg is the reverse cumulative sum of dG over the valid rows.
        for (int c2 = tid; c2 < d; c2 += THREADS) {
            float gc = 0.f;
            for (int c3 = 0; c3 < d; ++c3) gc += sdS[c2 * d + c3] * sS[c2 * d + c3];
            gc *= expf(sG[(C - 1) * d + c2]);
            for (int x = 0; x < C; ++x) gc += sdL[x * d + c2];
            float run = gc;
            for (int x = len - 1; x >= 0; --x) {
                run += sdG[x * d + c2];
                dg[((size_t)(t0 + x) * H + h) * d + c2] = run;
            }
        }
        for (int j = tid; j < len; j += THREADS) dbeta[(size_t)(t0 + j) * H + h] = sdb[j];
        __syncthreads();
        for (int e = tid; e < dd; e += THREADS) sdS[e] = sdSn[e];
        __syncthreads();
    }
    if (ds0)
        for (int e = tid; e < dd; e += THREADS) ds0[pair * dd + e] = sdS[e];
}

}  // namespace bwd_f32

bool bwd_f32_supported(int dk, int dv, int chunk) {
    if (dk != dv || !(dk == 16 || dk == 32 || dk == 64)) return false;
    if (!(chunk == 16 || chunk == 32 || chunk == 64)) return false;
    return (size_t)bwd_f32::lds_layout(dk, chunk).total * sizeof(float) <= 163840;
}

size_t bwd_f32_workspace_bytes(int64_t total_tokens, int n_seqs, int heads, int d, int chunk) {
    const int64_t slots = total_tokens / chunk + n_seqs + 1;
    return (size_t)slots * heads * d * d * sizeof(float);
}

hipError_t launch_chunk_bwd_f32(const ChunkBwdProblem &p) {
    using namespace bwd_f32;
    const size_t lds = (size_t)lds_layout(p.d, p.chunk).total * sizeof(float);
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&kda_chunk_bwd_f32_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kda_chunk_bwd_f32_kernel, dim3(p.n_seqs * p.heads), dim3(THREADS), lds,
                       p.stream, p.q, p.k, p.v, p.g, p.beta, p.scale, p.heads, p.d, p.chunk,
                       p.seqlen, p.cu, p.s0, p.dfinal, p.dout, p.dq, p.dk, p.dv, p.dg, p.dbeta,
                       p.ds0, p.ckpt);
    return hipGetLastError();
}

}  // namespace kda
