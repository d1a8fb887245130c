// kda_post.hip -- output stage of a KDA layer after the recurrence, gfx950:
//   out[r, c] = o[r, c] / sqrt(mean_c' o[r, c']^2 + eps) * weight[c] * sigmoid(gate[r, c])
// ("Understanding Kimi Delta Attention", section "From mathematics to the GPU",
// names output gating and RMS normalisation among the layer's steps around the
// core).  One pass: o and gate are read once and out written once, so the
// kernel is bound by HBM.  A row of d_v channels is held by d_v / 4 lanes of
// one wave (4 channels each, one 8- or 16-byte access per tensor), and its sum
// of squares is reduced with in-wave shuffles.  out may equal o: every lane
// reads all of its elements before it writes any, and no other lane touches
// them.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

// Four consecutive elements of one row: the raw words as loaded (Raw), and
// their values as fp32.
template <typename T> struct Vec4;
template <> struct Vec4<float> {
    typedef float4v Raw;
    __device__ static Raw load(const float *p) { return *reinterpret_cast<const float4v *>(p); }
    __device__ static float4v value(Raw r) { return r; }
    __device__ static void store(float *p, float4v x) { *reinterpret_cast<float4v *>(p) = x; }
};
template <> struct Vec4<bf16_t> {
    typedef uint2 Raw;
    __device__ static Raw load(const bf16_t *p) { return *reinterpret_cast<const uint2 *>(p); }
    __device__ static float4v value(Raw u) {
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

// Each thread takes RPT rows, 256 / (d_v / 4) rows apart, and issues every load
// of them before the first reduction, so a lane keeps 2 RPT accesses in flight.
constexpr int POST_RPT = 8;

template <typename T, int DV>
__global__ __launch_bounds__(256) void kda_output_rmsnorm_gate_kernel(
    int64_t rows, const T *__restrict__ o, const T *__restrict__ gate,
    const float *__restrict__ weight, float eps, T *out) {
    typedef typename Vec4<T>::Raw Raw;
    constexpr int TPR = DV / 4;          // lanes per row
    constexpr int RPI = 256 / TPR;       // rows per workgroup and step
    static_assert(DV % 4 == 0 && TPR <= 64 && 64 % TPR == 0, "row must fit one wave");
    const int tid = threadIdx.x, c4 = tid % TPR;
    const int64_t row0 = (int64_t)blockIdx.x * RPI * POST_RPT + tid / TPR;
    // Rows past the end load row 0 (in bounds; rows >= 1 whenever this runs)
    // and are neither reduced into a stored row nor stored.
    Raw xr[POST_RPT], zr[POST_RPT];
#pragma unroll
    for (int r = 0; r < POST_RPT; ++r) {
        const int64_t row = row0 + (int64_t)r * RPI;
        const size_t base = (size_t)(row < rows ? row : 0) * DV + 4 * c4;
        xr[r] = Vec4<T>::load(o + base);
        zr[r] = Vec4<T>::load(gate + base);
    }
    const float4v wv = *reinterpret_cast<const float4v *>(weight + 4 * c4);
#pragma unroll
    for (int r = 0; r < POST_RPT; ++r) {
        const float4v x = Vec4<T>::value(xr[r]);
        float ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
#pragma unroll
        for (int m = 1; m < TPR; m <<= 1) ss += __shfl_xor(ss, m, 64);
        const int64_t row = row0 + (int64_t)r * RPI;
        if (row < rows) {
            const float4v z = Vec4<T>::value(zr[r]);
            const float inv = rsqrtf(ss * (1.f / DV) + eps);
            float4v y;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = x[e] * inv * wv[e] * sigmoid(z[e]);
            Vec4<T>::store(out + (size_t)row * DV + 4 * c4, y);
        }
    }
}

bool output_stage_supported(int dv) {
    return dv == 16 || dv == 32 || dv == 64 || dv == 128 || dv == 256;
}

template <typename T, int DV>
static hipError_t launch_post(int64_t rows, const void *o, const void *gate, const float *w,
                              float eps, void *out, hipStream_t stream) {
    constexpr int RPB = 256 / (DV / 4) * POST_RPT;   // rows per workgroup
    const int64_t blocks = (rows + RPB - 1) / RPB;
    if (blocks == 0) return hipSuccess;
    if (!launch_fits(blocks, 256)) return hipErrorInvalidConfiguration;
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
