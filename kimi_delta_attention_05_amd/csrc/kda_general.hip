// Recurrent KDA forward for any key and value head sizes (1..256 each).
//
// The chunkwise prefill and the decode kernels are built around K = V = 128
// (the FlashInfer "kda_backward" contract's head dimension): their register
// and LDS layouts follow from it. The FlashKDA issue page ("Proposed scope")
// asks for arbitrary key/value dimensions as well; this kernel serves those
// sizes with the token-by-token form of the recurrence, in fp32:
//
//   S <- S diag(alpha_t);  S <- S + b_t (v_t - S kh_t) kh_t^T;  o_t = S qh_t
//
// over packed variable-length sequences with optional initial and final
// states. A batched decode step is the same call with every sequence one token
// long (the state of request n is sequence n's state).
//
// One workgroup per (sequence, head, block of 16 state rows), 256 threads: a
// 16-lane DPP row owns one state row v, lane j holding the key channels
// j + 16 e (e < NE, NE = ceil(K / 16) rounded up to a power of two; channels
// at or past K hold zero state and zero keys, queries and decay 1). Tokens go
// in groups of 16: the workgroup turns a group's q, k, g, beta and v (loaded
// into registers while the previous group ran) into qh, kh, alpha, b in LDS (a
// DPP row per token), then each row runs the 16 steps, the two K-wide dot
// products being DPP row sums, and the group's outputs leave through LDS as 16
// contiguous values per token.
//
// The file also holds the row copy with zero fill through which head sizes up
// to 128 run on the chunkwise prefill and backward kernels instead (inputs
// widened to 128 channels and rows with zeros, results narrowed back).
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kGTok = 16;    // tokens per group
constexpr int kGRows = 16;   // state rows per workgroup

// Workgroup b -> (sequence * H + head, row block): the row blocks of one
// (sequence, head) share its token data, so they go to one XCD (workgroups are
// dealt to the 8 XCDs round-robin by index).
__device__ __forceinline__ bool general_block(int64_t b, int64_t NH, int nvb, int64_t &nh, int &vb) {
    const int x = (int)(b & 7);
    const int64_t rest = b >> 3;
    vb = (int)(rest % nvb);
    nh = (rest / nvb) * 8 + x;
    return nh < NH;
}

template <typename Tin, typename Tout, int NE>
__global__ __launch_bounds__(256) void recurrent_fwd_kernel(GeneralArgs p)
{
    constexpr int KP = 16 * NE;                      // padded key width
    const int H = p.H, K = p.K, V = p.V;
    const int nvb = (V + kGRows - 1) / kGRows;
    int64_t nh;
    int vb;
    if (!general_block(blockIdx.x, (int64_t)p.N * H, nvb, nh, vb)) return;
    const int n = (int)(nh / H), h = (int)(nh % H);
    const int hk = h / (H / p.Hk);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15;
    const int row = 4 * wave + (lane >> 4);         // state row within the block
    const int grow = vb * kGRows + row;             // state row v
    const bool row_ok = grow < V;
    const int gid = tid >> 4;                       // token of the group staged by this DPP row

    __shared__ float sQ[kGTok][KP], sK[kGTok][KP], sA[kGTok][KP];
    __shared__ float sB[kGTok], sV[kGTok][kGRows], sO[kGTok][kGRows];

    const Tin *q = (const Tin *)p.q, *k = (const Tin *)p.k, *v = (const Tin *)p.v;
    // with a state pool the state of request n is entry slots[n]; a request whose
    // slot lies outside the pool is padding: zero outputs, no state touched
    int64_t snh = nh;
    if (p.slots) {
        const int sl = p.slots[n];
        if (sl < 0 || sl >= p.num_slots) {
            const int vr = vb * kGRows + tid;
            if (tid < kGRows && vr < V) ((Tout *)p.o)[(size_t)nh * V + vr] = from_f32<Tout>(0.0f);
            return;
        }
        snh = (int64_t)sl * H + h;
    }
    const size_t sbase = ((size_t)snh * V + (row_ok ? grow : 0)) * K;
    float S[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const int c = j + 16 * e;
        S[e] = (p.h0 && row_ok && c < K) ? p.h0[sbase + c] : 0.0f;
    }
    const float a_gate = fast_exp2(p.A_log[h] * kLog2e);
    const float lb2 = p.lower_bound * kLog2e;
    float dtb[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const int c = j + 16 * e;
        dtb[e] = c < K ? p.dt_bias[(size_t)h * K + c] : 0.0f;
    }

    // no offsets (the decode step): sequence n is token n
    const int64_t s0 = p.cu_seqlens ? p.cu_seqlens[n] : n;
    const int64_t s1 = p.cu_seqlens ? p.cu_seqlens[n + 1] : n + 1;
    // raw token data of token `gid` of a group, loaded one group ahead so that the
    // next group's loads are in flight while the current group's steps run
    float qv[NE], kv[NE], gv[NE], braw = 0.f, vv = 0.f;
    auto fetch = [&](int64_t t0) {
        const int64_t t = t0 + gid;
        if (t < s1) {
            const size_t tq = ((size_t)t * p.Hk + hk) * K, tg = ((size_t)t * H + h) * K;
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                const int c = j + 16 * e;
                qv[e] = c < K ? to_f32(q[tq + c]) : 0.0f;
                kv[e] = c < K ? to_f32(k[tq + c]) : 0.0f;
                gv[e] = c < K ? p.g[tg + c] : 0.0f;
            }
            braw = p.beta_raw[(size_t)t * H + h];
            const int vr = vb * kGRows + j;
            vv = vr < V ? to_f32(v[((size_t)t * H + h) * V + vr]) : 0.0f;
        }
    };
    fetch(s0);
    for (int64_t t0 = s0; t0 < s1; t0 += kGTok) {
        const int L = (int)(s1 - t0 < kGTok ? s1 - t0 : kGTok);
        // ---- token transforms of the group -> LDS ----------------------------------
        if (gid < L) {
            float ss_q = 0.f, ss_k = 0.f;
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                ss_q = fmaf(qv[e], qv[e], ss_q);
                ss_k = fmaf(kv[e], kv[e], ss_k);
            }
            const float rq = rsqrtf(row16_sum(ss_q) + kL2Eps) * p.scale;
            const float rk = rsqrtf(row16_sum(ss_k) + kL2Eps);
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                const int c = j + 16 * e;
                sQ[gid][c] = qv[e] * rq;
                sK[gid][c] = kv[e] * rk;
                sA[gid][c] = c < K ? fast_exp2(lb2 * sigmoid_f(a_gate * (gv[e] + dtb[e]))) : 1.0f;
            }
            if (j == 0) sB[gid] = sigmoid_f(braw);
            sV[gid][j] = vv;
        }
        lds_barrier();
        fetch(t0 + kGTok);
        // ---- the group's steps, one state row per DPP row --------------------------
        auto step = [&](int i) {
            float sk = 0.f;
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                S[e] *= sA[i][j + 16 * e];
                sk = fmaf(S[e], sK[i][j + 16 * e], sk);
            }
            const float u = sB[i] * (sV[i][row] - row16_sum(sk));
            float sq = 0.f;
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                S[e] = fmaf(u, sK[i][j + 16 * e], S[e]);
                sq = fmaf(S[e], sQ[i][j + 16 * e], sq);
            }
            sq = row16_sum(sq);
            if (j == 0) sO[i][row] = sq;
        };
        if (L == kGTok) {
            // whole group: unrolled, so that the LDS reads of later steps are
            // issued while earlier steps' dot products are still in flight
#pragma unroll
            for (int i = 0; i < kGTok; ++i) step(i);
        } else {
            for (int i = 0; i < L; ++i) step(i);
        }
        lds_barrier();
        // ---- outputs: 16 contiguous values per token -------------------------------
        {
            const int i = tid >> 4, r = tid & 15, vr = vb * kGRows + r;
            if (i < L && vr < V)
                ((Tout *)p.o)[((size_t)(t0 + i) * H + h) * V + vr] = from_f32<Tout>(sO[i][r]);
        }
    }
    if (p.ht && row_ok) {
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int c = j + 16 * e;
            if (c < K) p.ht[sbase + c] = S[e];
        }
    }
}

template <typename Tin, typename Tout>
hipError_t launch_general_t(const GeneralArgs &a) {
    const int nvb = (a.V + kGRows - 1) / kGRows;
    const int64_t groups = ((int64_t)a.N * a.H + 7) / 8;
    const dim3 grid((unsigned)(groups * 8 * nvb));
    const int ne = (a.K + 15) / 16;
    if (ne <= 1)      recurrent_fwd_kernel<Tin, Tout, 1><<<grid, 256, 0, a.stream>>>(a);
    else if (ne <= 2) recurrent_fwd_kernel<Tin, Tout, 2><<<grid, 256, 0, a.stream>>>(a);
    else if (ne <= 4) recurrent_fwd_kernel<Tin, Tout, 4><<<grid, 256, 0, a.stream>>>(a);
    else if (ne <= 6) recurrent_fwd_kernel<Tin, Tout, 6><<<grid, 256, 0, a.stream>>>(a);
    else if (ne <= 8) recurrent_fwd_kernel<Tin, Tout, 8><<<grid, 256, 0, a.stream>>>(a);
    else if (ne <= 12) recurrent_fwd_kernel<Tin, Tout, 12><<<grid, 256, 0, a.stream>>>(a);
    else              recurrent_fwd_kernel<Tin, Tout, 16><<<grid, 256, 0, a.stream>>>(a);
    return hipGetLastError();
}

// Row copy with zero fill, for running head sizes below 128 on the chunkwise
// kernels: destination row d (of dst_cols elements) is source row
// (d / rd) * rs + d % rd when d % rd < rs, its first min(src_cols, dst_cols)
// elements copied and the rest zero; otherwise the row is zero. rd = rs = 1
// maps row to row (tokens, parameters); rd = 128, rs = V widens the value rows
// of a state to 128, rd = V, rs = 128 narrows them back.
template <typename E>
__global__ __launch_bounds__(256) void pad_rows_kernel(const E *__restrict__ src, int src_cols,
                                                       int64_t rs, E *__restrict__ dst,
                                                       int dst_cols, int64_t rd, int64_t rows,
                                                       bool src_vec, bool dst_vec)
{
    // a thread moves NV consecutive elements (16 bytes) of a destination row,
    // with 16-byte loads and stores where the rows are 16-byte aligned
    constexpr int NV = 16 / sizeof(E);
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    union Piece { u32x4 v; E e[NV]; };
    const int per_row = (dst_cols + NV - 1) / NV;
    const int64_t n = rows * per_row, stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const int64_t d = i / per_row;
        const int c0 = (int)(i - d * per_row) * NV;
        int64_t grp = d, r = 0;
        if (rd > 1) {
            grp = d / rd;
            r = d - grp * rd;
        }
        Piece x;
        x.v = u32x4{0u, 0u, 0u, 0u};
        if (r < rs) {
            const E *sp = src + (grp * rs + r) * src_cols;
            if (src_vec && c0 + NV <= src_cols) {
                x.v = *(const u32x4 *)(sp + c0);
            } else {
#pragma unroll
                for (int e = 0; e < NV; ++e)
                    if (c0 + e < src_cols) x.e[e] = sp[c0 + e];
            }
        }
        E *dp = dst + d * dst_cols;
        if (dst_vec && c0 + NV <= dst_cols) {
            *(u32x4 *)(dp + c0) = x.v;
        } else {
#pragma unroll
            for (int e = 0; e < NV; ++e)
                if (c0 + e < dst_cols) dp[c0 + e] = x.e[e];
        }
    }
}

}  // namespace

hipError_t launch_pad_rows(const void *src, int src_cols, int64_t rs, void *dst, int dst_cols,
                           int64_t rd, int64_t dst_rows, int elem_bytes, hipStream_t stream) {
    if (dst_rows <= 0 || dst_cols <= 0) return hipSuccess;
    const int nv = 16 / elem_bytes;
    const int64_t n = dst_rows * ((dst_cols + nv - 1) / nv);
    const int64_t blocks = (n + 255) / 256;
    const unsigned grid = (unsigned)(blocks < (1 << 16) ? blocks : (1 << 16));
    const bool sv = ((int64_t)src_cols * elem_bytes) % 16 == 0 && ((uintptr_t)src & 15) == 0;
    const bool dv = ((int64_t)dst_cols * elem_bytes) % 16 == 0 && ((uintptr_t)dst & 15) == 0;
    if (elem_bytes == 4)
        pad_rows_kernel<uint32_t><<<grid, 256, 0, stream>>>((const uint32_t *)src, src_cols, rs,
                                                            (uint32_t *)dst, dst_cols, rd, dst_rows,
                                                            sv, dv);
    else
        pad_rows_kernel<uint16_t><<<grid, 256, 0, stream>>>((const uint16_t *)src, src_cols, rs,
                                                            (uint16_t *)dst, dst_cols, rd, dst_rows,
                                                            sv, dv);
    return hipGetLastError();
}

int64_t general_blocks(int64_t N, int64_t H, int V) {
    return ((N * H + 7) / 8) * 8 * ((V + kGRows - 1) / kGRows);
}

hipError_t launch_recurrent_fwd(const GeneralArgs &a) {
    if (a.in_bf16)
        return a.out_bf16 ? launch_general_t<__bf16, __bf16>(a) : launch_general_t<__bf16, float>(a);
    return a.out_bf16 ? launch_general_t<float, __bf16>(a) : launch_general_t<float, float>(a);
}

}  // namespace kda
