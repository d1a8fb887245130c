// kda_post.hip -- output stage of a KDA layer after the recurrence, gfx950:
//   out[r, c] = o[r, c] / sqrt(mean_c' o[r, c']^2 + eps) * weight[c] * sigmoid(gate[r, c])
// ("Understanding Kimi Delta Attention", section "From mathematics to the GPU",
// names output gating and RMS normalisation among the layer's steps around the
// core).  One pass: o and gate are read once and out written once, so the
// kernel is bound by HBM.  A row of d_v channels is held by d_v / 4 lanes of
// one wave (4 channels each, one 8- or 16-byte access per tensor), and its sum
// of squares is reduced with in-wave shuffles.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

template <typename T> struct Vec4;
template <> struct Vec4<float> {
    __device__ static float4v load(const float *p) { return *reinterpret_cast<const float4v *>(p); }
    __device__ static void store(float *p, float4v x) { *reinterpret_cast<float4v *>(p) = x; }
};
template <> struct Vec4<bf16_t> {
    __device__ static float4v load(const bf16_t *p) {
        const uint2 u = *reinterpret_cast<const uint2 *>(p);
        return float4v{bf16_to_f32(u.x & 0xffff), bf16_to_f32(u.x >> 16), bf16_to_f32(u.y & 0xffff),
                       bf16_to_f32(u.y >> 16)};
    }
    __device__ static void store(bf16_t *p, float4v x) {
        uint2 u;
        u.x = pack_bf16x2(x[0], x[1]);
        u.y = pack_bf16x2(x[2], x[3]);
        *reinterpret_cast<uint2 *>(p) = u;
    }
};

template <typename T, int DV>
__global__ __launch_bounds__(256) void kda_output_rmsnorm_gate_kernel(
    int64_t rows, const T *__restrict__ o, const T *__restrict__ gate,
    const float *__restrict__ weight, float eps, T *out) {
    constexpr int TPR = DV / 4;          // lanes per row
    constexpr int RPB = 256 / TPR;       // rows per workgroup
    static_assert(DV % 4 == 0 && TPR <= 64 && 64 % TPR == 0, "row must fit one wave");
    const int tid = threadIdx.x, c4 = tid % TPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + tid / TPR;
    const bool ok = row < rows;
    const size_t base = (size_t)(ok ? row : 0) * DV + 4 * c4;
    const float4v x = ok ? Vec4<T>::load(o + base) : float4v{0, 0, 0, 0};
    float ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) ss += __shfl_xor(ss, m, 64);
    if (!ok) return;
    const float inv = rsqrtf(ss * (1.f / DV) + eps);
    const float4v z = Vec4<T>::load(gate + base);
    const float4v wv = *reinterpret_cast<const float4v *>(weight + 4 * c4);
    float4v y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = x[e] * inv * wv[e] * sigmoid(z[e]);
    Vec4<T>::store(out + base, y);
}

bool output_stage_supported(int dv) {
    return dv == 16 || dv == 32 || dv == 64 || dv == 128 || dv == 256;
}

template <typename T, int DV>
static hipError_t launch_post(int64_t rows, const void *o, const void *gate, const float *w,
                              float eps, void *out, hipStream_t stream) {
    constexpr int RPB = 256 / (DV / 4);
    const int64_t blocks = (rows + RPB - 1) / RPB;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((kda_output_rmsnorm_gate_kernel<T, DV>), dim3((unsigned)blocks), dim3(256),
                       0, stream, rows, static_cast<const T *>(o), static_cast<const T *>(gate), w,
                       eps, static_cast<T *>(out));
    return hipGetLastError();
}

hipError_t launch_output_rmsnorm_gate(int64_t rows, int dv, bool bf16, const void *o,
                                      const void *gate, const float *weight, float eps,
                                      void *out, hipStream_t stream) {
#define KDA_POST_CASE(D)                                                                      \
    if (dv == D)                                                                              \
        return bf16 ? launch_post<bf16_t, D>(rows, o, gate, weight, eps, out, stream)         \
                    : launch_post<float, D>(rows, o, gate, weight, eps, out, stream);
    KDA_POST_CASE(16)
    KDA_POST_CASE(32)
    KDA_POST_CASE(64)
    KDA_POST_CASE(128)
    KDA_POST_CASE(256)
#undef KDA_POST_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
