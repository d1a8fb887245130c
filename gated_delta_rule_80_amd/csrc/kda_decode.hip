// kda_decode.hip -- one recurrent KDA step per (session, head), gfx950.
//
// Per pair ("Understanding Kimi Delta Attention", box "KDA: retain, predict,
// correct"; read scale from "Demystifying Kimi Delta Attention"):
//   S_bar = Diag(a) S,  v_hat = S_bar^T k,  e = v - v_hat,
//   S_new = S_bar + beta k e^T,  o = S_new^T (s q).
// Because o = S_bar^T (s q) + beta (k . s q) e, both column reductions
// (S_bar^T k and S_bar^T (s q)) come from ONE read of the state, and the new
// state is written from registers: the fp32 state crosses HBM exactly once
// in each direction, which is the whole cost of a decode step.
//
// The decay is given per key channel (KDA), once per pair (a scalar gate:
// every channel decays by the same a), or not at all (a = 1).
//
// Layout: one workgroup per pair; thread (rg, cq) owns the float4 column
// quad cq of rows rg, rg + NRG, rg + 2 NRG, ...  Each wave's loads and
// stores cover whole 512-byte state rows (fully coalesced, nontemporal: the
// state is streamed, never re-read within a step).  Ordinary (temporal)
// accesses look faster only while the whole state fits the 256 MB Infinity
// Cache between steps (128 sessions x 32 heads at d = 128 nearly does); at
// twice that they are 15% slower than streaming ones.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

template <int DK, int DV>
struct DecodeCfg {
    static constexpr int NQ = DV / 4;                        // column quads
    // 512 threads (8 state rows each at d = 128) measured faster than 256 or
    // 1024 at 128, 256 and 512 sessions.
    static constexpr int THREADS = (NQ * DK < 512) ? NQ * DK : 512;
    static constexpr int NRG = THREADS / NQ;                 // row groups
    static constexpr int RPT = DK / NRG;                     // rows per thread
    static constexpr int NWAVES = (THREADS + 63) / 64;
    static_assert(DV % 4 == 0 && THREADS % NQ == 0 && DK % NRG == 0, "decode tiling");
    static_assert(64 % NQ == 0 || NQ % 64 == 0, "column quads per wave");
};

template <int DK, int DV, typename T, Gate GATE>
__global__ __launch_bounds__((DecodeCfg<DK, DV>::THREADS)) void kda_decode_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float scale, int form,
    float eps, float *__restrict__ state, T *__restrict__ o) {
    using Cfg = DecodeCfg<DK, DV>;
    constexpr int NQ = Cfg::NQ, NRG = Cfg::NRG, RPT = Cfg::RPT, NWAVES = Cfg::NWAVES;
    constexpr int THREADS = Cfg::THREADS;

    __shared__ float s_a[DK], s_k[DK], s_sq[DK], s_v[DV];
    __shared__ float4v s_red[NWAVES][2][NQ];
    __shared__ float s_kq[NWAVES], s_kk[NWAVES], s_qq[NWAVES];

    const size_t pair = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int cq = tid % NQ, rg = tid / NQ;

    // Stream this thread's part of the state in first: it is the long pole.
    float4v S[RPT];
    const float4v *sp = reinterpret_cast<const float4v *>(state + pair * DK * DV);
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        S[i] = __builtin_nontemporal_load(sp + (size_t)(rg + NRG * i) * NQ + cq);

    // Token vectors: a = exp(g) (sigmoid(g) for a logit gate), k, s*q, v; plus
    // the scalar k . (s q) and, for L2-normalised q and k, |k|^2 and |q|^2.
    const bool glogit = (form & kFormGateLogit) != 0;
    float kq = 0.f, kk2 = 0.f, qq2 = 0.f;
    for (int i = tid; i < DK; i += THREADS) {
        const size_t gi = pair * DK + i;
        const float kk = io<T>::load(k, gi), qq = io<T>::load(q, gi);
        float a = 1.f;
        if (GATE == Gate::PerChannel) a = glogit ? sigmoid(g[gi]) : fast_exp(g[gi]);
        if (GATE == Gate::Scalar) a = glogit ? sigmoid(g[pair]) : fast_exp(g[pair]);
        s_a[i] = a;
        s_k[i] = kk;
        s_sq[i] = scale * qq;
        kq += kk * (scale * qq);
        kk2 += kk * kk;
        qq2 += qq * qq;
    }
    for (int i = tid; i < DV; i += THREADS) s_v[i] = io<T>::load(v, pair * DV + i);
    kq = wave_sum(kq);
    if (lane == 0) s_kq[wave] = kq;
    if (form & kFormL2Norm) {
        kk2 = wave_sum(kk2);
        qq2 = wave_sum(qq2);
        if (lane == 0) {
            s_kk[wave] = kk2;
            s_qq[wave] = qq2;
        }
    }
    __syncthreads();
    // 1 / |k| and 1 / |q| when q and k are normalised here (else 1); every use
    // of k and q below is linear in them, so the factors are applied to sums.
    float ik = 1.f, iq = 1.f;
    if (form & kFormL2Norm) {
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) {
            a += s_kk[w];
            b += s_qq[w];
        }
        ik = rsqrtf(a + eps);
        iq = rsqrtf(b + eps);
    }

    // Retain, then both reductions over this thread's rows.
    float4v vh = {0.f, 0.f, 0.f, 0.f}, qs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + NRG * i;
        S[i] *= s_a[r];
        vh += s_k[r] * S[i];
        qs += s_sq[r] * S[i];
    }
    // Sum over the row groups: first inside the wave (lanes sharing cq) ...
#pragma unroll
    for (int off = NQ; off < 64; off <<= 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            vh[j] += __shfl_xor(vh[j], off, 64);
            qs[j] += __shfl_xor(qs[j], off, 64);
        }
    }
    // ... then across waves through LDS.
    if (NQ >= 64 || lane < NQ) {
        s_red[wave][0][cq] = vh;
        s_red[wave][1][cq] = qs;
    }
    __syncthreads();
    vh = s_red[0][0][cq];
    qs = s_red[0][1][cq];
    kq = s_kq[0];
#pragma unroll
    for (int w = 1; w < NWAVES; ++w) {
        vh += s_red[w][0][cq];
        qs += s_red[w][1][cq];
        kq += s_kq[w];
    }
    vh *= ik;
    qs *= iq;
    kq *= ik * iq;

    const float b = (form & kFormBetaLogit) ? sigmoid(beta[pair]) : beta[pair];
    float4v e;
#pragma unroll
    for (int j = 0; j < 4; ++j) e[j] = s_v[4 * cq + j] - vh[j];

    if (rg == 0) {
        const float bkq = b * kq;
#pragma unroll
        for (int j = 0; j < 4; ++j) io<T>::store(o, pair * DV + 4 * cq + j, qs[j] + bkq * e[j]);
    }

    float4v *spw = reinterpret_cast<float4v *>(state + pair * DK * DV);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + NRG * i;
        const float bk = b * ik * s_k[r];
        __builtin_nontemporal_store(S[i] + bk * e, spw + (size_t)r * NQ + cq);
    }
}

template <int DK, int DV, typename T, Gate GATE>
static hipError_t launch_decode_g(int n_pairs, InputForm f, const void *q, const void *k,
                                  const void *v, const float *g, const float *beta, float scale,
                                  float *state, void *o, hipStream_t stream) {
    using Cfg = DecodeCfg<DK, DV>;
    if (!launch_fits(n_pairs, Cfg::THREADS)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((kda_decode_kernel<DK, DV, T, GATE>), dim3(n_pairs), dim3(Cfg::THREADS),
                       0, stream, static_cast<const T *>(q), static_cast<const T *>(k),
                       static_cast<const T *>(v), g, beta, scale, f.flags(), f.eps, state,
                       static_cast<T *>(o));
    return hipGetLastError();
}

template <int DK, int DV, typename T>
static hipError_t launch_decode_t(Gate gate, InputForm f, int n_pairs, const void *q,
                                  const void *k, const void *v, const float *g,
                                  const float *beta, float scale, float *state, void *o,
                                  hipStream_t stream) {
    switch (gate) {
    case Gate::PerChannel:
        return launch_decode_g<DK, DV, T, Gate::PerChannel>(n_pairs, f, q, k, v, g, beta, scale,
                                                            state, o, stream);
    case Gate::Scalar:
        return launch_decode_g<DK, DV, T, Gate::Scalar>(n_pairs, f, q, k, v, g, beta, scale,
                                                        state, o, stream);
    case Gate::None:
        return launch_decode_g<DK, DV, T, Gate::None>(n_pairs, f, q, k, v, g, beta, scale, state,
                                                      o, stream);
    }
    return hipErrorInvalidValue;
}

// Returns hipErrorInvalidValue for a (d_k, d_v) that is not instantiated.
hipError_t launch_decode(int n_pairs, int dk, int dv, bool bf16, Gate gate, InputForm form,
                         const void *q, const void *k, const void *v, const float *g,
                         const float *beta, float scale, float *state, void *o,
                         hipStream_t stream) {
#define KDA_DECODE_CASE(D)                                                                     \
    if (dk == D && dv == D)                                                                    \
        return bf16 ? launch_decode_t<D, D, bf16_t>(gate, form, n_pairs, q, k, v, g, beta,     \
                                                    scale, state, o, stream)                   \
                    : launch_decode_t<D, D, float>(gate, form, n_pairs, q, k, v, g, beta, scale, \
                                                   state, o, stream);
    KDA_DECODE_CASE(128)
    KDA_DECODE_CASE(64)
    KDA_DECODE_CASE(32)
    KDA_DECODE_CASE(16)
#undef KDA_DECODE_CASE
    return hipErrorInvalidValue;
}

bool decode_supported(int dk, int dv) {
    return dk == dv && (dk == 128 || dk == 64 || dk == 32 || dk == 16);
}

}  // namespace kda
