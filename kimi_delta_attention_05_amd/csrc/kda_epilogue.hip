// Output epilogue of the attention block (kimi_k3 FusedKDAChunkwise page,
// "Output handling"): each output row of 128 features is RMS-normalised,
// scaled by a per-channel weight and multiplied by a sigmoid output gate,
//   y = o / sqrt(mean(o^2) + eps) * weight * sigmoid(z).
//
// One 16-lane DPP row per output row, 8 features per lane (16-byte loads and
// stores of bf16, 32 bytes of fp32), 16 rows per 256-thread workgroup: every
// instruction moves whole consecutive rows. HBM-bound: o, z read once, y
// written once. The rows, the gate logits and the result each have their own
// dtype (bf16 or fp32).
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

// o is not __restrict__: y may alias it (the epilogue applied in place).
template <typename To, typename Tz, typename Ty>
__global__ __launch_bounds__(256) void norm_gate_kernel(const To *o, const Tz *__restrict__ z,
                                                        const float *__restrict__ w, float eps,
                                                        int64_t rows, Ty *y)
{
    const int j = threadIdx.x & 15;                    // features 8j .. 8j + 7
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const bool valid = row < rows;
    const size_t base = (size_t)(valid ? row : rows - 1) * kHeadDim + 8 * j;   // rows >= 1
    float x[8], g[8], wv[8];
    load8(o + base, x);
    load8(z + base, g);
    load8(w + 8 * j, wv);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    ss = row16_sum(ss);
    const float r = rsqrtf(ss * (1.0f / kHeadDim) + eps);
    float out[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = x[e] * r * wv[e] * sigmoid_f(g[e]);
    if (valid) store8_nt<Ty>(y + base, out);
}

// Rows staged as fp16 by the chunkwise forward: each 16-feature block of a row
// holds its values divided by a power of two, kept in sc[row][block]; lane j
// takes the scale of block j / 2. The products with the scales are exact, so y
// is rounded once, from the staged fp16 values.
template <typename Tz, typename Ty>
__global__ __launch_bounds__(256) void norm_gate_scaled_kernel(const _Float16 *__restrict__ o,
                                                               const float *__restrict__ sc,
                                                               const Tz *__restrict__ z,
                                                               const float *__restrict__ w, float eps,
                                                               int64_t rows, Ty *__restrict__ y)
{
    const int j = threadIdx.x & 15;
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const bool valid = row < rows;
    const size_t r0 = (size_t)(valid ? row : rows - 1);
    const size_t base = r0 * kHeadDim + 8 * j;
    const half8 h = *(const half8 *)(o + base);
    const float s = sc[r0 * (kHeadDim / 16) + (j >> 1)];
    float x[8], g[8], wv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)h[e] * s;
    load8(z + base, g);
    load8(w + 8 * j, wv);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    ss = row16_sum(ss);
    const float r = rsqrtf(ss * (1.0f / kHeadDim) + eps);
    float out[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = x[e] * r * wv[e] * sigmoid_f(g[e]);
    if (valid) store8_nt<Ty>(y + base, out);
}

// Rows of any other width D <= 256 (head sizes other than 128): one wave per
// row, lane l holding features l, l + 64, l + 128, l + 192 below D, the sum of
// squares reduced over the wave.
template <typename To, typename Tz, typename Ty>
__global__ __launch_bounds__(256) void norm_gate_any_kernel(const To *o,
                                                            const Tz *__restrict__ z,
                                                            const float *__restrict__ w, float eps,
                                                            int64_t rows, int D, Ty *y)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;                        // the whole wave
    const size_t base = (size_t)row * D;
    float x[4], ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int c = lane + 64 * e;
        x[e] = c < D ? to_f32(o[base + c]) : 0.0f;
        ss = fmaf(x[e], x[e], ss);
    }
    const float r = rsqrtf(wave_sum(ss) / (float)D + eps);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int c = lane + 64 * e;
        if (c < D) y[base + c] = from_f32<Ty>(x[e] * r * w[c] * sigmoid_f(to_f32(z[base + c])));
    }
}

template <typename Tz, typename Ty>
static hipError_t launch_norm_gate_scaled_t(const NormGateArgs &a) {
    if (a.D != kHeadDim) return hipErrorInvalidValue;
    const int64_t blocks = (a.rows + 15) / 16;
    norm_gate_scaled_kernel<Tz, Ty><<<(unsigned)blocks, 256, 0, a.stream>>>(
        (const _Float16 *)a.o, a.o_scale, (const Tz *)a.z, a.w, a.eps, a.rows, (Ty *)a.y);
    return hipGetLastError();
}

template <typename To, typename Tz, typename Ty>
static hipError_t launch_norm_gate_t(const NormGateArgs &a) {
    if (a.D != kHeadDim) {
        const unsigned blocks = (unsigned)((a.rows + 3) / 4);
        norm_gate_any_kernel<To, Tz, Ty><<<blocks, 256, 0, a.stream>>>(
            (const To *)a.o, (const Tz *)a.z, a.w, a.eps, a.rows, a.D, (Ty *)a.y);
    } else {
        const int64_t blocks = (a.rows + 15) / 16;
        norm_gate_kernel<To, Tz, Ty><<<(unsigned)blocks, 256, 0, a.stream>>>(
            (const To *)a.o, (const Tz *)a.z, a.w, a.eps, a.rows, (Ty *)a.y);
    }
    return hipGetLastError();
}

template <typename To, typename Tz>
static hipError_t launch_norm_gate_y(const NormGateArgs &a) {
    return a.y_bf16 ? launch_norm_gate_t<To, Tz, __bf16>(a) : launch_norm_gate_t<To, Tz, float>(a);
}

template <typename To>
static hipError_t launch_norm_gate_z(const NormGateArgs &a) {
    return a.z_bf16 ? launch_norm_gate_y<To, __bf16>(a) : launch_norm_gate_y<To, float>(a);
}

hipError_t launch_norm_gate(const NormGateArgs &a) {
    if (a.rows <= 0) return hipSuccess;
    if (a.o_scale) {                    // fp16 rows with block scales
        if (a.z_bf16) return a.y_bf16 ? launch_norm_gate_scaled_t<__bf16, __bf16>(a)
                                      : launch_norm_gate_scaled_t<__bf16, float>(a);
        return a.y_bf16 ? launch_norm_gate_scaled_t<float, __bf16>(a)
                        : launch_norm_gate_scaled_t<float, float>(a);
    }
    return a.bf16 ? launch_norm_gate_z<__bf16>(a) : launch_norm_gate_z<float>(a);
}

}  // namespace kda
