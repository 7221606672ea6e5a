// Training backward of the KDA recurrence (FlashInfer kda_backward page,
// "Supported contract": gradients for q, k, v, the raw gate, raw beta, A_log,
// dt_bias and the initial state, given the output adjoint; the persistent
// forward-checkpoint and reverse kernels of its "Workspace and CUDA Graphs"
// section; the kda-neuron-kernels commit log asks that the gradient be that of
// the exact forward).
//
// Forward per token (S value-first [V][K], fp32):
//   S' = S diag(alpha),  u = b (v - S' kh),  S <- S' + u kh^T,  o = S qh
// Reverse per token, dS the adjoint of the state after the token:
//   dS += do qh^T;  dqh = S^T do;  du = dS kh;  dkh = dS^T u - b S'^T du;
//   dv = b du;  db = du . (v - S' kh);  dS' = dS - b du kh^T;
//   dalpha = colsum(dS' * S_prev);  dS <- dS' diag(alpha)
// then dq, dk through the L2 normalisations, dg, ddt_bias, dA_log through the
// gate, dbeta through the sigmoid; dh0 is the adjoint left at the start.
//
// Every state row v evolves on its own in both directions; only dqh, dkh,
// dalpha and db sum over rows. Four launches:
//   bwd_ckpt_kernel     one workgroup per (sequence, head, block of 16 rows)
//                       runs the forward and stores the state every 16 tokens
//                       (the chunk-boundary checkpoints);
//   bwd_reverse_kernel  same grid: walks the chunks backwards, recomputes the
//                       states of each half chunk (8 tokens) from the chunk's
//                       checkpoint into registers, runs the reverse steps,
//                       writes dv, dh0 and each block's row sums of the
//                       per-token partials;
//   bwd_finalize_kernel one workgroup per (16 tokens, head): adds the 8 blocks'
//                       partials and applies the elementwise chains (dq, dk,
//                       dg, dbeta), plus per-block sums for the parameters;
//   bwd_param_kernel    one workgroup per head: ddt_bias and dA_log.
// No atomics: every sum has a fixed order, so results repeat bit for bit.
//
// Thread layout of the first two (the decode step's): 256 threads = 4 waves,
// a 16-lane DPP row owns one state row, lane j holds channels 4j..4j+3 and
// 64+4j..64+4j+3, so 128-wide dot products are row16 DPP sums.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kCk = 16;                          // checkpoint spacing (tokens)
constexpr int kBRows = 16;                       // state rows per workgroup
constexpr int kNVB = kHeadDim / kBRows;          // workgroups per (sequence, head)
constexpr int kPartCols = 3 * kHeadDim + 1;      // dqh, dkh, dalpha partials, db

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int chan(int j, int e) { return e < 4 ? 4 * j + e : 64 + 4 * j + (e - 4); }

// the 8 channels of lane j from a row of 128 elements
__device__ __forceinline__ void load_lane8(const float *row, int j, float (&x)[8]) {
    const f32x4 a = *(const f32x4 *)(row + 4 * j), b = *(const f32x4 *)(row + 64 + 4 * j);
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[e + 4] = b[e]; }
}
__device__ __forceinline__ void load_lane8(const __bf16 *row, int j, float (&x)[8]) {
    const bf16x4_t a = *(const bf16x4_t *)(row + 4 * j), b = *(const bf16x4_t *)(row + 64 + 4 * j);
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[e] = (float)a[e]; x[e + 4] = (float)b[e]; }
}
__device__ __forceinline__ void store_lane8(float *row, int j, const float (&x)[8]) {
    *(f32x4 *)(row + 4 * j) = f32x4{x[0], x[1], x[2], x[3]};
    *(f32x4 *)(row + 64 + 4 * j) = f32x4{x[4], x[5], x[6], x[7]};
}

// Sum over the four 16-lane rows of a wave (every lane gets the sum): the
// gfx950 permlane swaps exchange lanes l and l ^ 32, then l and l ^ 16, in
// VALU (no LDS round trip).
__device__ __forceinline__ float rows4_sum(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Four values reduced over the wave's four 16-lane rows at once: a 32-lane
// swap and add leaves a's half sums in lanes 0-31 and b's in 32-63 (c and d
// likewise in a second register), a 16-lane swap and add of those two then
// leaves in row 0 the full sum of a, in row 1 that of c, in row 2 b, in row 3
// d (each at the lane's own position in its row): 3 swaps + 3 adds for four
// sums instead of 8 + 8.
__device__ __forceinline__ float quad_rows_sum(float a, float b, float c, float d) {
    const auto ab = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    const auto cd = __builtin_amdgcn_permlane32_swap(__float_as_uint(c), __float_as_uint(d), false, false);
    const float x = __uint_as_float(ab[0]) + __uint_as_float(ab[1]);
    const float y = __uint_as_float(cd[0]) + __uint_as_float(cd[1]);
    const auto xy = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(xy[0]) + __uint_as_float(xy[1]);
}

// Workgroup b -> (sequence*H + head, row block). The 8 row blocks of one
// (sequence, head) share its token data, so they go to one XCD (blocks are
// dealt to the 8 XCDs round-robin by index).
__device__ __forceinline__ bool bwd_block(int64_t b, int64_t NH, int64_t &nh, int &vb) {
    const int x = (int)(b & 7);
    const int64_t rest = b >> 3;
    vb = (int)(rest & 7);
    nh = (rest >> 3) * 8 + x;
    return nh < NH;
}

// Per-token transforms of token t for lane j's channels (one DPP row per token).
template <typename Tin>
__device__ __forceinline__ void key_and_decay(const Tin *k, const float *g, const float (&dtb)[8],
                                              float a_gate, float lb, size_t tb, size_t tbk, int j,
                                              float (&kh)[8], float (&al)[8]) {
    float kv[8], gv[8];
    load_lane8(k + tbk, j, kv);
    load_lane8(g + tb, j, gv);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(kv[e], kv[e], ss);
    const float rk = rsqrtf(row16_sum(ss) + kL2Eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        kh[e] = kv[e] * rk;
        al[e] = fast_exp2(lb * sigmoid_f(a_gate * (gv[e] + dtb[e])) * kLog2e);
    }
}

template <typename Tin>
__global__ __launch_bounds__(256) void bwd_ckpt_kernel(
    const Tin *__restrict__ k, const Tin *__restrict__ v, const float *__restrict__ g,
    const float *__restrict__ beta_raw, const float *__restrict__ A_log,
    const float *__restrict__ dt_bias, float lb, const int64_t *__restrict__ cu, int N, int H,
    int Hk, const float *__restrict__ h0, float *__restrict__ ckpt)
{
    int64_t nh;
    int vb;
    if (!bwd_block(blockIdx.x, (int64_t)N * H, nh, vb)) return;
    const int n = (int)(nh / H), h = (int)(nh % H);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15;
    const int row = 4 * wave + (lane >> 4);          // state row within the block
    const int gid = threadIdx.x >> 4;                // token slot of the per-chunk transforms
    const int grow = vb * kBRows + row;
    const int64_t s0 = cu[n], s1 = cu[n + 1];
    const int64_t nck = (s1 - s0 + kCk - 1) / kCk;
    const int64_t slot0 = s0 / kCk + n;

    __shared__ float sKh[kCk][kHeadDim], sAl[kCk][kHeadDim];
    __shared__ float sB[kCk], sV[kCk][kBRows];

    float S[8];
    if (h0) load_lane8(h0 + ((size_t)nh * kHeadDim + grow) * kHeadDim, j, S);
    else {
#pragma unroll
        for (int e = 0; e < 8; ++e) S[e] = 0.f;
    }
    const float a_gate = fast_exp2(A_log[h] * kLog2e);
    float dtb[8];
    load_lane8(dt_bias + (size_t)h * kHeadDim, j, dtb);

    // raw token data of the chunk's token `gid`, loaded one chunk ahead so that
    // the loads of chunk c + 1 are in flight while chunk c runs
    float kv[8], gv[8], braw = 0.f, vv = 0.f;
    auto fetch = [&](int64_t c) {
        const int64_t t = s0 + c * kCk + gid;
        if (c < nck && t < s1) {
            const size_t tb = ((size_t)t * H + h) * kHeadDim;
            load_lane8(k + ((size_t)t * Hk + h / (H / Hk)) * kHeadDim, j, kv);
            load_lane8(g + tb, j, gv);
            braw = beta_raw[(size_t)t * H + h];
            vv = to_f32(v[tb + vb * kBRows + j]);
        }
    };
    fetch(0);
    for (int64_t c = 0; c < nck; ++c) {
        const int64_t c0 = s0 + c * kCk;
        const int L = (int)(s1 - c0 < kCk ? s1 - c0 : kCk);
        store_lane8(ckpt + (((size_t)(slot0 + c) * H + h) * kHeadDim + grow) * kHeadDim, j, S);
        if (gid < L) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(kv[e], kv[e], ss);
            const float rk = rsqrtf(row16_sum(ss) + kL2Eps);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sKh[gid][chan(j, e)] = kv[e] * rk;
                sAl[gid][chan(j, e)] = fast_exp2(lb * sigmoid_f(a_gate * (gv[e] + dtb[e])) * kLog2e);
            }
            if (j == 0) sB[gid] = sigmoid_f(braw);
            sV[gid][j] = vv;
        }
        lds_barrier();
        fetch(c + 1);
        // unrolled so that each token's LDS reads are issued ahead of the
        // previous token's dependency chain
#pragma unroll
        for (int i = 0; i < kCk; ++i) {
            if (i < L) {
                float kh[8], al[8];
                load_lane8(&sKh[i][0], j, kh);
                load_lane8(&sAl[i][0], j, al);
                float p = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) { S[e] *= al[e]; p = fmaf(S[e], kh[e], p); }
                const float u = sB[i] * (sV[i][row] - row16_sum(p));
#pragma unroll
                for (int e = 0; e < 8; ++e) S[e] = fmaf(u, kh[e], S[e]);
            }
        }
        lds_barrier();
    }
}

// Forward step of one token on a state row (lane j's 8 channels); returns
// w = v - S' kh for the row and updates S.
__device__ __forceinline__ float fwd_row_step(float (&S)[8], const float *kh_row, const float *al_row,
                                              int j, float b, float vv, float &u) {
    float kh[8], al[8];
    load_lane8(kh_row, j, kh);
    load_lane8(al_row, j, al);
    float p = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        S[e] *= al[e];
        p = fmaf(S[e], kh[e], p);
    }
    const float w = vv - row16_sum(p);
    u = b * w;
#pragma unroll
    for (int e = 0; e < 8; ++e) S[e] = fmaf(u, kh[e], S[e]);
    return w;
}

// Three workgroups per CU (at most 168 VGPRs and 53 KB of LDS each), so that
// the 8 row blocks x heads of the benchmark shape are resident in one round.
template <typename Tin, typename Tdo>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void bwd_reverse_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta_raw,
    const float *__restrict__ A_log, const float *__restrict__ dt_bias, float scale, float lb,
    const int64_t *__restrict__ cu, int N, int H, int Hk, const float *__restrict__ ckpt,
    const Tdo *__restrict__ dout, const float *__restrict__ dht, float *__restrict__ dv,
    float *__restrict__ part, float *__restrict__ dh0)
{
    constexpr int kSub = 8;            // states kept in registers at a time
    constexpr int kFlush = 4;          // tokens per flush of the per-wave sums
    int64_t nh;
    int vb;
    if (!bwd_block(blockIdx.x, (int64_t)N * H, nh, vb)) return;
    const int n = (int)(nh / H), h = (int)(nh % H);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15;
    const int row = 4 * wave + (lane >> 4);
    const int gid = threadIdx.x >> 4;
    const int grow = vb * kBRows + row;
    const int64_t s0 = cu[n], s1 = cu[n + 1];
    const int64_t nck = (s1 - s0 + kCk - 1) / kCk;
    const int64_t slot0 = s0 / kCk + n;

    __shared__ float sKh[kCk][kHeadDim], sQh[kCk][kHeadDim], sAl[kCk][kHeadDim];
    __shared__ float sB[kCk], sV[kCk][kBRows], sDo[kCk][kBRows], sU[kCk][kBRows], sW[kCk][kBRows];
    // per-wave sums (over the wave's 4 rows) of the partials of kFlush tokens
    __shared__ float sRed[kFlush][4][kPartCols];

    float dS[8];
    if (dht) load_lane8(dht + ((size_t)nh * kHeadDim + grow) * kHeadDim, j, dS);
    else {
#pragma unroll
        for (int e = 0; e < 8; ++e) dS[e] = 0.f;
    }
    const float a_gate = fast_exp2(A_log[h] * kLog2e);
    float dtb[8];
    load_lane8(dt_bias + (size_t)h * kHeadDim, j, dtb);

    for (int64_t c = nck - 1; c >= 0; --c) {
        const int64_t c0 = s0 + c * kCk;
        const int L = (int)(s1 - c0 < kCk ? s1 - c0 : kCk);
        const float *ck = ckpt + (((size_t)(slot0 + c) * H + h) * kHeadDim + grow) * kHeadDim;
        if (gid < L) {
            const int64_t t = c0 + gid;
            const size_t tb = ((size_t)t * H + h) * kHeadDim;
            const size_t tbk = ((size_t)t * Hk + h / (H / Hk)) * kHeadDim;
            float kh[8], al[8], qv[8];
            key_and_decay(k, g, dtb, a_gate, lb, tb, tbk, j, kh, al);
            load_lane8(q + tbk, j, qv);
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(qv[e], qv[e], ss);
            const float rq = rsqrtf(row16_sum(ss) + kL2Eps) * scale;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sKh[gid][chan(j, e)] = kh[e];
                sAl[gid][chan(j, e)] = al[e];
                sQh[gid][chan(j, e)] = qv[e] * rq;
            }
            if (j == 0) sB[gid] = sigmoid_f(beta_raw[(size_t)t * H + h]);
            sV[gid][j] = to_f32(v[tb + vb * kBRows + j]);
            sDo[gid][j] = to_f32(dout[tb + vb * kBRows + j]);
        }
        lds_barrier();

        // the chunk's two halves, last first: recompute the states before the
        // half's tokens from the checkpoint (registers), then the reverse steps
#pragma unroll 1
        for (int half = 1; half >= 0; --half) {
            const int i0 = half * kSub;
            if (i0 < L) {
                float S[8];
                load_lane8(ck, j, S);
#pragma unroll
                for (int i = 0; i < kSub; ++i) {     // tokens before the half: states not kept
                    if (i < i0) {
                        float u;
                        fwd_row_step(S, &sKh[i][0], &sAl[i][0], j, sB[i], sV[i][row], u);
                    }
                }
                float snap[kSub][8];
#pragma unroll
                for (int ii = 0; ii < kSub; ++ii) {
                    const int i = i0 + ii;
                    if (i < L) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) snap[ii][e] = S[e];
                        float u;
                        const float w = fwd_row_step(S, &sKh[i][0], &sAl[i][0], j, sB[i], sV[i][row], u);
                        if (j == 0) { sU[i][row] = u; sW[i][row] = w; }
                    }
                }
#pragma unroll
                for (int ii = kSub - 1; ii >= 0; --ii) {
                    const int i = i0 + ii;
                    if (i < L) {
                        const int64_t t = c0 + i;
                        float kh[8], al[8], qh[8];
                        load_lane8(&sKh[i][0], j, kh);
                        load_lane8(&sAl[i][0], j, al);
                        load_lane8(&sQh[i][0], j, qh);
                        const float b = sB[i], u = sU[i][row], w = sW[i][row], d_o = sDo[i][row];
                        float sp[8], pq[8], pk[8], pa[8];
                        float du = 0.f;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            sp[e] = snap[ii][e] * al[e];                 // S'
                            pq[e] = d_o * fmaf(u, kh[e], sp[e]);        // do_v * S_t[v, :]
                            dS[e] = fmaf(d_o, qh[e], dS[e]);
                            du = fmaf(dS[e], kh[e], du);
                        }
                        du = row16_sum(du);
                        const float bdu = b * du;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            pk[e] = u * dS[e] - bdu * sp[e];
                            const float dsp = fmaf(-bdu, kh[e], dS[e]);
                            pa[e] = dsp * snap[ii][e];
                            dS[e] = dsp * al[e];
                        }
                        const size_t tb = ((size_t)t * H + h) * kHeadDim;
                        if (j == 0) dv[tb + grow] = bdu;
                        // sums over the wave's 4 rows, kept per wave in LDS: each
                        // quad_rows_sum leaves in row r the sum of its value at
                        // offset qo = 0, 2, 1, 3 (rows 0..3), so every lane
                        // stores one sum per quad
                        float *red = &sRed[i % kFlush][wave][0];
                        const float pb = rows4_sum(du * w);
                        const int qo = (lane >> 4) == 1 ? 2 : ((lane >> 4) == 2 ? 1 : (lane >> 4));
#pragma unroll
                        for (int hq = 0; hq < 2; ++hq) {
                            const int e0 = 4 * hq;
                            const int cidx = 64 * hq + 4 * j + qo;          // chan(j, e0 + qo)
                            red[cidx] = quad_rows_sum(pq[e0], pq[e0 + 1], pq[e0 + 2], pq[e0 + 3]);
                            red[kHeadDim + cidx] = quad_rows_sum(pk[e0], pk[e0 + 1], pk[e0 + 2], pk[e0 + 3]);
                            red[2 * kHeadDim + cidx] = quad_rows_sum(pa[e0], pa[e0 + 1], pa[e0 + 2], pa[e0 + 3]);
                        }
                        if (lane == 0) red[3 * kHeadDim] = pb;
                        // after tokens i .. min(i + kFlush, L) - 1: add the 4
                        // waves' sums and store the block's row sums
                        if (i % kFlush == 0) {
                            const int ntok = (L - i < kFlush) ? L - i : kFlush;
                            lds_barrier();
                            for (int idx = threadIdx.x; idx < ntok * kPartCols; idx += 256) {
                                const int ti = idx / kPartCols, col = idx - ti * kPartCols;
                                const float sum = (sRed[ti][0][col] + sRed[ti][1][col]) +
                                                  (sRed[ti][2][col] + sRed[ti][3][col]);
                                const size_t tt = (size_t)(c0 + i + ti);
                                part[((tt * H + h) * kNVB + vb) * kPartCols + col] = sum;
                            }
                            lds_barrier();
                        }
                    }
                }
            }
        }
        lds_barrier();
    }
    if (dh0) store_lane8(dh0 + ((size_t)nh * kHeadDim + grow) * kHeadDim, j, dS);
}

// One DPP row per token, 16 tokens per workgroup, one q/k head per grid row:
// the value heads that share the q/k head (grouped value heads) add their dqh
// and dkh before the normalisations' chains; dg and dbeta are per value head.
template <typename Tin>
__global__ __launch_bounds__(256) void bwd_finalize_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta_raw, const float *__restrict__ A_log,
    const float *__restrict__ dt_bias, float scale, float lb, int64_t T, int H, int Hk,
    const float *__restrict__ part, float *__restrict__ dq, float *__restrict__ dk,
    float *__restrict__ dg, float *__restrict__ dbeta, float *__restrict__ pp)
{
    const int hk = blockIdx.y;
    const int G = H / Hk;
    const int64_t tblk = blockIdx.x;
    const int j = threadIdx.x & 15, gid = threadIdx.x >> 4;
    const int64_t t = tblk * 16 + gid;
    const bool valid = t < T;
    __shared__ float sP[16][kHeadDim + 1];

    float dqh[8], dkh[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { dqh[e] = 0.f; dkh[e] = 0.f; }
    for (int gg = 0; gg < G; ++gg) {
        const int h = hk * G + gg;
        float dgv[8];
        float cA = 0.f;
        if (valid) {
            const size_t tb = ((size_t)t * H + h) * kHeadDim;
            const float *src = part + (size_t)((size_t)t * H + h) * kNVB * kPartCols;
            float dal[8];
            float db = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) dal[e] = 0.f;
#pragma unroll
            for (int b = 0; b < kNVB; ++b) {
                float x[8];
                load_lane8(src + b * kPartCols, j, x);
#pragma unroll
                for (int e = 0; e < 8; ++e) dqh[e] += x[e];
                load_lane8(src + b * kPartCols + kHeadDim, j, x);
#pragma unroll
                for (int e = 0; e < 8; ++e) dkh[e] += x[e];
                load_lane8(src + b * kPartCols + 2 * kHeadDim, j, x);
#pragma unroll
                for (int e = 0; e < 8; ++e) dal[e] += x[e];
                db += src[b * kPartCols + 3 * kHeadDim];
            }
            float gv[8], dtb[8];
            load_lane8(g + tb, j, gv);
            load_lane8(dt_bias + (size_t)h * kHeadDim, j, dtb);
            const float a_gate = fast_exp2(A_log[h] * kLog2e);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float sg = sigmoid_f(a_gate * (gv[e] + dtb[e]));
                const float al = fast_exp2(lb * sg * kLog2e);
                dgv[e] = dal[e] * al * lb * sg * (1.0f - sg) * a_gate;
                cA = fmaf(dgv[e], gv[e] + dtb[e], cA);
            }
            store_lane8(dg + tb, j, dgv);
            cA = row16_sum(cA);
            if (j == 0) {
                const float bb = sigmoid_f(beta_raw[(size_t)t * H + h]);
                dbeta[(size_t)t * H + h] = db * bb * (1.0f - bb);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) dgv[e] = 0.f;
        }
        // this value head's sums over the 16 tokens, for the parameters
#pragma unroll
        for (int e = 0; e < 8; ++e) sP[gid][chan(j, e)] = dgv[e];
        if (j == 0) sP[gid][kHeadDim] = cA;
        lds_barrier();
        if (threadIdx.x <= kHeadDim) {
            float sum = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) sum += sP[r][threadIdx.x];
            pp[((size_t)tblk * H + h) * (kHeadDim + 1) + threadIdx.x] = sum;
        }
        lds_barrier();
    }
    if (valid) {
        const size_t tbk = ((size_t)t * Hk + hk) * kHeadDim;
        float qv[8], kv[8];
        load_lane8(q + tbk, j, qv);
        load_lane8(k + tbk, j, kv);
        float sq = 0.f, sk = 0.f, qd = 0.f, kd = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sq = fmaf(qv[e], qv[e], sq);
            sk = fmaf(kv[e], kv[e], sk);
            qd = fmaf(qv[e], dqh[e], qd);
            kd = fmaf(kv[e], dkh[e], kd);
        }
        sq = row16_sum(sq); sk = row16_sum(sk); qd = row16_sum(qd); kd = row16_sum(kd);
        const float rq = rsqrtf(sq + kL2Eps), rk = rsqrtf(sk + kL2Eps);
        const float cq = rq * rq * rq * qd, ck = rk * rk * rk * kd;
        float dqo[8], dko[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            dqo[e] = scale * (rq * dqh[e] - cq * qv[e]);
            dko[e] = rk * dkh[e] - ck * kv[e];
        }
        store_lane8(dq + tbk, j, dqo);
        store_lane8(dk + tbk, j, dko);
    }
}

// ddt_bias[h, c] = sum over tokens of dg; dA_log[h] = sum over tokens and
// channels of dg * (g + dt_bias): the per-16-token sums added in token order,
// split over two thread halves (even and odd blocks) and then combined.
__global__ __launch_bounds__(256) void bwd_param_kernel(const float *__restrict__ pp, int64_t ntb,
                                                        int H, float *__restrict__ dA_log,
                                                        float *__restrict__ ddt_bias)
{
    const int h = blockIdx.x;
    constexpr int NC = kHeadDim + 1;
    __shared__ float sAcc[2][NC];
    for (int col = threadIdx.x; col < 2 * NC; col += 256) {
        const int c = col % NC, half = col / NC;
        float s = 0.f;
        for (int64_t b = half; b < ntb; b += 2) s += pp[((size_t)b * H + h) * NC + c];
        sAcc[half][c] = s;
    }
    lds_barrier();
    if (threadIdx.x < NC) {
        const float s = sAcc[0][threadIdx.x] + sAcc[1][threadIdx.x];
        if (threadIdx.x < kHeadDim) ddt_bias[(size_t)h * kHeadDim + threadIdx.x] = s;
        else dA_log[h] = s;
    }
}

template <typename Tin, typename Tdo>
hipError_t launch_backward_t(const BackwardArgs &a) {
    const int Hk = a.Hk > 0 ? a.Hk : a.H;   // q/k heads (grouped value heads)
    const int64_t NH = (int64_t)a.N * a.H;
    const unsigned grid = (unsigned)(((NH + 7) / 8) * 64);
    bwd_ckpt_kernel<Tin><<<grid, 256, 0, a.stream>>>(
        (const Tin *)a.k, (const Tin *)a.v, a.g, a.beta_raw, a.A_log, a.dt_bias, a.lower_bound,
        a.cu, a.N, a.H, Hk, a.h0, a.ckpt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    bwd_reverse_kernel<Tin, Tdo><<<grid, 256, 0, a.stream>>>(
        (const Tin *)a.q, (const Tin *)a.k, (const Tin *)a.v, a.g, a.beta_raw, a.A_log,
        a.dt_bias, a.scale, a.lower_bound, a.cu, a.N, a.H, Hk, a.ckpt, (const Tdo *)a.dout, a.dht,
        a.dv, a.part, a.dh0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t ntb = (a.T + 15) / 16;
    if (ntb > 0) {
        bwd_finalize_kernel<Tin><<<dim3((unsigned)ntb, (unsigned)Hk), 256, 0, a.stream>>>(
            (const Tin *)a.q, (const Tin *)a.k, a.g, a.beta_raw, a.A_log, a.dt_bias, a.scale,
            a.lower_bound, a.T, a.H, Hk, a.part, a.dq, a.dk, a.dg, a.dbeta, a.pp);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    bwd_param_kernel<<<(unsigned)a.H, 256, 0, a.stream>>>(a.pp, ntb, a.H, a.dA_log, a.ddt_bias);
    return hipGetLastError();
}

}  // namespace

BackwardLayout backward_layout(int64_t T, int N, int H) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    BackwardLayout l;
    l.ckpt_bytes = up((size_t)(T / kCk + N) * H * kHeadDim * kHeadDim * 4);
    l.part_bytes = up((size_t)T * H * kNVB * kPartCols * 4);
    l.pp_bytes = up((size_t)((T + 15) / 16) * H * (kHeadDim + 1) * 4);
    l.total = l.ckpt_bytes + l.part_bytes + l.pp_bytes;
    return l;
}

hipError_t launch_backward(const BackwardArgs &a) {
    if (a.in_bf16)
        return a.do_bf16 ? launch_backward_t<__bf16, __bf16>(a) : launch_backward_t<__bf16, float>(a);
    return a.do_bf16 ? launch_backward_t<float, __bf16>(a) : launch_backward_t<float, float>(a);
}

}  // namespace kda
