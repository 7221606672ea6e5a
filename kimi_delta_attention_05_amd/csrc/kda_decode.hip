// Batched T=1 KDA decode step: one pass over the fp32 state, with the state
// rows of a (request, head) split over 8 waves (two workgroups of 4 waves), or
// over 16 waves of one workgroup with the fused output epilogue, whose norm
// needs all 128 outputs.
//
// Per (request b, head h) the value-first state S[128][128] is read once and
// written once. Every state row v is independent given the per-token vectors:
//   s   = S[v,:] * alpha                 (decay per key channel)
//   a_v = s . qh,   p_v = s . kh         (both dot products in the same pass)
//   u_v = beta (v_v - p_v)
//   S[v,:] = s + u_v kh                  (delta-rule write, in place)
//   o_v = a_v + u_v (kh . qh)            (= (S_new qh)_v, read after the write)
// Folding the read-out into the update pass through the scalar kh.qh is the
// one-pass "key-fold" reading of the kda-neuron-kernels commit log's recurrent
// forward; batching every (request, head) pair into one launch follows its
// batched decode. Transforms per the FlashInfer kda_backward contract.
//
// Thread layout: NW waves; a DPP row of 16 lanes covers one state row, lane j
// holding channels 4j .. 4j+3 and 64+4j .. 64+4j+3, so that each of the two
// 16-byte loads (and stores) of a row covers 256 contiguous bytes: whole cache
// lines per instruction. A wave covers 4 rows per iteration, the workgroup
// 4 NW, over NIT iterations. All loads of a lane are issued before any
// arithmetic.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

template <typename Tin, typename Tout, bool GATED, int NIT, int NW>
__global__ __launch_bounds__(64 * NW) void decode_step_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta_raw,
    const float *__restrict__ A_log, const float *__restrict__ dt_bias,
    float scale, float lower_bound, float *__restrict__ state, Tout *__restrict__ o,
    int H, const Tin *__restrict__ zg, const float *__restrict__ norm_w, float norm_eps,
    const int32_t *__restrict__ slots, int num_slots, int Hk)
{
    constexpr int RPI = 4 * NW;                // rows per iteration
    constexpr int NSPLIT = kHeadDim / (RPI * NIT);
    const int bh = blockIdx.x / NSPLIT;        // request * H + head
    const int part = blockIdx.x % NSPLIT;      // block of RPI NIT state rows
    const int rbase = RPI * NIT * part;
    const int h = bh % H;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane & 15;                   // channels 4j .. 4j+3 and 64+4j .. 64+4j+3
    const int r = lane >> 4;                   // row within the wave's 4 rows

    // state of this (request, head): row bh of the state array, or, with slot
    // indices, row slots[request] * H + h of a state pool; a request whose slot
    // lies outside [0, num_slots) is padding: its outputs are zero and no state
    // is touched (the decision is uniform over the workgroup)
    size_t sbh = (size_t)bh;
    if (slots) {
        const int sl = slots[bh / H];
        if (sl < 0 || sl >= num_slots) {
            if (threadIdx.x < RPI * NIT) o[(size_t)bh * kHeadDim + rbase + threadIdx.x] = from_f32<Tout>(0.0f);
            return;
        }
        sbh = (size_t)sl * H + h;
    }
    f32x4 *S4 = reinterpret_cast<f32x4 *>(state + sbh * (kHeadDim * kHeadDim));

    // Issue the state loads first: rows 16*it + 4*wave + r, 16-byte pieces j and 16+j.
    f32x4 st[NIT][2];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int row = rbase + RPI * it + 4 * wave + r;
        st[it][0] = __builtin_nontemporal_load(S4 + row * 32 + j);
        st[it][1] = __builtin_nontemporal_load(S4 + row * 32 + 16 + j);
    }

    // Per-token vectors for this lane's 8 channels (each 16-lane row holds all 128):
    // entry e is channel ch(e) = 4j + e for e < 4 and 64 + 4j + (e - 4) otherwise.
    const size_t tb = (size_t)bh * kHeadDim;
    // q and k of the request's q/k head h / (H / Hk) (grouped value heads; Hk = H without)
    const size_t tbk = ((size_t)(bh / H) * Hk + h / (H / Hk)) * kHeadDim;
    float qv[8], kv[8], al[8];
    const float a_gate = fast_exp2(A_log[h] * kLog2e);
    float sqq = 0.f, skk = 0.f, sqk = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int ch = (e < 4) ? 4 * j + e : 64 + 4 * j + (e - 4);
        qv[e] = to_f32(q[tbk + ch]);
        kv[e] = to_f32(k[tbk + ch]);
        sqq += qv[e] * qv[e];
        skk += kv[e] * kv[e];
        sqk += qv[e] * kv[e];
        const float x = a_gate * (g[tb + ch] + dt_bias[h * kHeadDim + ch]);
        al[e] = fast_exp2(lower_bound * sigmoid_f(x) * kLog2e);   // alpha = e^lambda
    }
    sqq = row16_sum(sqq);
    skk = row16_sum(skk);
    sqk = row16_sum(sqk);
    const float rq = rsqrtf(sqq + kL2Eps) * scale;
    const float rk = rsqrtf(skk + kL2Eps);
    const float kq = sqk * rq * rk;                                // kh . qh
    float qh[8], kh[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { qh[e] = qv[e] * rq; kh[e] = kv[e] * rk; }
    const float beta = sigmoid_f(beta_raw[bh]);

    __shared__ float so[RPI * NIT];            // outputs, stored coalesced at the end
    float vrow[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) vrow[it] = to_f32(v[tb + rbase + RPI * it + 4 * wave + r]);

#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int row = rbase + RPI * it + 4 * wave + r;
        float s[8] = {st[it][0][0], st[it][0][1], st[it][0][2], st[it][0][3],
                      st[it][1][0], st[it][1][1], st[it][1][2], st[it][1][3]};
        float a = 0.f, p = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            s[e] *= al[e];
            a += s[e] * qh[e];
            p += s[e] * kh[e];
        }
        a = row16_sum(a);
        p = row16_sum(p);
        const float u = beta * (vrow[it] - p);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += u * kh[e];
        const f32x4 s0 = {s[0], s[1], s[2], s[3]}, s1 = {s[4], s[5], s[6], s[7]};
        __builtin_nontemporal_store(s0, S4 + row * 32 + j);
        __builtin_nontemporal_store(s1, S4 + row * 32 + 16 + j);
        if (j == 0) so[row - rbase] = a + u * kq;
    }
    lds_barrier();
    if (threadIdx.x < RPI * NIT / 2) {           // wave 0, two outputs per lane
        const int i = 2 * threadIdx.x;
        float y0 = so[i], y1 = so[i + 1];
        if constexpr (GATED) {
            static_assert(RPI * NIT == kHeadDim, "the epilogue needs the head's 128 outputs in one workgroup");
            // output epilogue (kimi_k3 FusedKDAChunkwise page, "Output handling"):
            // RMS norm over the head's 128 outputs, channel weight, sigmoid gate
            const float ms = wave_sum(y0 * y0 + y1 * y1) * (1.0f / kHeadDim);
            const float r = rsqrtf(ms + norm_eps);
            y0 = y0 * r * norm_w[i] * sigmoid_f(to_f32(zg[tb + i]));
            y1 = y1 * r * norm_w[i + 1] * sigmoid_f(to_f32(zg[tb + i + 1]));
        }
        o[tb + rbase + i] = from_f32<Tout>(y0);
        o[tb + rbase + i + 1] = from_f32<Tout>(y1);
    }
}

// The plain step runs two 4-wave workgroups per (request, head), 64 state rows
// each (8 rows per wave, 68 VGPRs, 7 waves per SIMD); the step with the
// epilogue one 16-wave workgroup per (request, head), 8 rows per wave (60
// VGPRs), so that the norm sees the head's 128 outputs. Measured at B = 256,
// H = 32: plain 181 us (one 4-wave workgroup per head holding 128 rows: 198 us;
// the 8-wave form: 192 us; four workgroups of 32 rows: 184 us), with the
// epilogue 182 us (8 waves of 16 rows: 194 us; 4 waves of 32 rows: 201 us).
template <typename Tin, typename Tout>
static hipError_t launch_decode_t(const DecodeArgs &a) {
    const unsigned bh = (unsigned)(a.B * a.H);
    const int Hk = a.Hk > 0 ? a.Hk : a.H;
    if (a.z)
        decode_step_kernel<Tin, Tout, true, 2, 16><<<bh, 1024, 0, a.stream>>>(
            (const Tin *)a.q, (const Tin *)a.k, (const Tin *)a.v, a.g, a.beta_raw,
            a.A_log, a.dt_bias, a.scale, a.lower_bound, a.state, (Tout *)a.o, a.H,
            (const Tin *)a.z, a.norm_w, a.norm_eps, a.slots, a.num_slots, Hk);
    else
        decode_step_kernel<Tin, Tout, false, 4, 4><<<2 * bh, 256, 0, a.stream>>>(
            (const Tin *)a.q, (const Tin *)a.k, (const Tin *)a.v, a.g, a.beta_raw,
            a.A_log, a.dt_bias, a.scale, a.lower_bound, a.state, (Tout *)a.o, a.H,
            nullptr, nullptr, 0.f, a.slots, a.num_slots, Hk);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a) {
    if (a.in_bf16)
        return a.out_bf16 ? launch_decode_t<__bf16, __bf16>(a) : launch_decode_t<__bf16, float>(a);
    return a.out_bf16 ? launch_decode_t<float, __bf16>(a) : launch_decode_t<float, float>(a);
}

}  // namespace kda
