// Output epilogue of the attention block (kimi_k3 FusedKDAChunkwise page,
// "Output handling"): each output row of 128 features is RMS-normalised,
// scaled by a per-channel weight and multiplied by a sigmoid output gate,
//   y = o / sqrt(mean(o^2) + eps) * weight * sigmoid(z).
//
// One 16-lane DPP row per output row, 8 features per lane (16-byte loads and
// stores of bf16, 32 bytes of fp32), 16 rows per 256-thread workgroup: every
// instruction moves whole consecutive rows. HBM-bound: o, z read once, y
// written once.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

// o is not __restrict__: y may alias it (the epilogue applied in place).
template <typename T>
__global__ __launch_bounds__(256) void norm_gate_kernel(const T *o, const T *__restrict__ z,
                                                        const float *__restrict__ w, float eps,
                                                        int64_t rows, T *y)
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
    if (valid) store8_nt<T>(y + base, out);
}

// Rows of any other width D <= 256 (head sizes other than 128): one wave per
// row, lane l holding features l, l + 64, l + 128, l + 192 below D, the sum of
// squares reduced over the wave.
template <typename T, typename Z>
__global__ __launch_bounds__(256) void norm_gate_any_kernel(const T *o,
                                                            const Z *__restrict__ z,
                                                            const float *__restrict__ w, float eps,
                                                            int64_t rows, int D, T *y)
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
        if (c < D) y[base + c] = from_f32<T>(x[e] * r * w[c] * sigmoid_f(to_f32(z[base + c])));
    }
}

hipError_t launch_norm_gate(const NormGateArgs &a) {
    if (a.rows <= 0) return hipSuccess;
    if (a.D != kHeadDim) {
        const unsigned blocks = (unsigned)((a.rows + 3) / 4);
        if (a.bf16 && a.z_bf16)
            norm_gate_any_kernel<__bf16, __bf16><<<blocks, 256, 0, a.stream>>>(
                (const __bf16 *)a.o, (const __bf16 *)a.z, a.w, a.eps, a.rows, a.D, (__bf16 *)a.y);
        else if (a.bf16)
            norm_gate_any_kernel<__bf16, float><<<blocks, 256, 0, a.stream>>>(
                (const __bf16 *)a.o, (const float *)a.z, a.w, a.eps, a.rows, a.D, (__bf16 *)a.y);
        else if (a.z_bf16)
            norm_gate_any_kernel<float, __bf16><<<blocks, 256, 0, a.stream>>>(
                (const float *)a.o, (const __bf16 *)a.z, a.w, a.eps, a.rows, a.D, (float *)a.y);
        else
            norm_gate_any_kernel<float, float><<<blocks, 256, 0, a.stream>>>(
                (const float *)a.o, (const float *)a.z, a.w, a.eps, a.rows, a.D, (float *)a.y);
        return hipGetLastError();
    }
    const int64_t blocks = (a.rows + 15) / 16;
    if (a.bf16)
        norm_gate_kernel<__bf16><<<(unsigned)blocks, 256, 0, a.stream>>>(
            (const __bf16 *)a.o, (const __bf16 *)a.z, a.w, a.eps, a.rows, (__bf16 *)a.y);
    else
        norm_gate_kernel<float><<<(unsigned)blocks, 256, 0, a.stream>>>(
            (const float *)a.o, (const float *)a.z, a.w, a.eps, a.rows, (float *)a.y);
    return hipGetLastError();
}

}  // namespace kda
