// Training backward of the KDA recurrence (FlashInfer kda_backward page,
// "Supported contract": gradients for q, k, v, the raw gate, raw beta, A_log,
// dt_bias and the initial state, given the output adjoint; its "Workspace and
// CUDA Graphs" section: forward checkpoints in a caller workspace, then the
// reverse pass; the kda-neuron-kernels commit log asks that the gradient be
// that of the exact forward).
//
// Forward per token (S value-first [V][K], fp32):
//   S' = S diag(alpha),  u = b (v - S' kh),  S <- S' + u kh^T,  o = S qh.
// Over a chunk of L <= 16 tokens from the state S0 (G_t = the sum of the
// log-decays lambda of the chunk's tokens up to t, Gam = e^G, GC = Gam of the
// chunk's last token, SUF = GC / Gam = the product of the decays after t):
//   KE = kh Gam, QG = qh Gam, KG = kh SUF, KI = kh / Gam             [L][K]
//   P = KE KI^T, A = strict_lower(diag(b) P), M = lower(QG KI^T), X = (I + A)^-1,
//   T = X diag(b), R = V - KE S0^T, U = T R, O = QG S0^T + M U,
//   S1 = S0 diag(GC) + U^T KG.
// Its adjoint, given dO and the adjoint dS1 of the state after the chunk:
//   dU = M^T dO + KG dS1^T,  dR = T^T dU (= dv),
//   dS0 = dS1 diag(GC) + dO^T QG - dR^T KE,
// and, summed over the state rows v (the "partials"),
//   dQG = dO S0,  dKG = U dS1,  dKE = -dR S0,  dM = lower(dO U^T),  dT = dU R^T,
//   dGC = sum_v S0 * dS1;
// then, per chunk and without the state: dX = dT diag(b), db = colsum(X * dT)
// + rowsum(dA * P) with dA = strict_lower(-X^T dX X^T), dP = diag(b) dA,
// dKE += dP KI, dQG += dM KI, dKI = dP^T KE + dM^T QG,
// dkh = dKE Gam + dKG SUF + dKI / Gam, dqh = dQG Gam, and the log-decay adjoint
// dlambda_t = sum_{s >= t} (dKE KE + dQG QG - dKI KI)_s + sum_{s < t} (dKG KG)_s
// + GC dGC; then dq, dk through the L2 normalisations, dg, ddt_bias, dA_log
// through the gate, dbeta through the sigmoid.
//
// Five launches over 16-token chunks:
//   bwd_prep_kernel        one workgroup per (chunk slot, head), chunk-parallel:
//                          the chunk's operands KE, KG, QG, T, M^T, GC, X, P as
//                          a record in the workspace;
//   bwd_ckpt_kernel        one workgroup per (sequence, head, half of the state
//                          rows), chunk-serial: the forward over the chunks (fp32
//                          MFMA), storing the state at every chunk start;
//   bwd_chunk_kernel       same grid, chunks backwards: dS in registers, dv,
//                          dh0, and per chunk the partials summed over the
//                          half's 64 state rows;
//   bwd_chunk_final_kernel one workgroup per (chunk slot, q/k head): adds the two
//                          halves' partials and finishes the chunk's gradients;
//   bwd_param_kernel       one workgroup per head: ddt_bias and dA_log.
// The chunk-serial kernels copy each chunk's record into LDS (DMA, one chunk
// ahead, double-buffered) and load the next chunk's state rows while the
// current chunk runs, so that a chunk's step is the MFMA work and two barriers.
// No atomics: every sum has a fixed order, so results repeat bit for bit.
//
// Products are 16 x 16 x 16 tiles on the fp32 MFMA (exact fp32 products, fp32
// accumulation), so the arithmetic is that of an fp32 reference. A wave owns 16
// state rows; its operands stay in the MFMA register layouts, and a transposed
// operand is produced by computing the transposed product (the accumulator of
// X^T is the row operand of X) rather than by a pass through LDS.
#include <atomic>

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kCk = 16;                        // chunk length (tokens)
constexpr int kTP = 132;                       // LDS pitch (floats) of [16][128] tiles
constexpr int kSP = 20;                        // LDS pitch of [16][16] tiles
constexpr int kTile = 16 * kTP, kSmall = 16 * kSP;
constexpr int kPartChunk = 3 * 16 * kHeadDim + 2 * 16 * 16 + kHeadDim;   // partial floats per (chunk, head, half)
constexpr int kPartRec = kPartChunk + 2 * 256;  // their record (dM, dT in two parts each)
static_assert(kPartChunk <= kPartRec && kPartRec <= 64 * kHeadDim,
              "a half's partial record fits in its checkpoint rows");

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

// Raw (unconverted) loads, so that a load issued one chunk ahead is waited for
// only where its value is used.
template <typename T> struct Vec4T;
template <> struct Vec4T<float> { typedef f32x4 type; };
template <> struct Vec4T<__bf16> { typedef bf16x4_t type; };
template <typename T> using vec4 = typename Vec4T<T>::type;
template <typename T> struct Raw8 { vec4<T> a, b; };

template <typename T>
__device__ __forceinline__ void raw8_load(Raw8<T> &r, const T *row, int j) {
    r.a = *(const vec4<T> *)(row + 4 * j);
    r.b = *(const vec4<T> *)(row + 64 + 4 * j);
}
template <typename T>
__device__ __forceinline__ void raw8_get(const Raw8<T> &r, float (&x)[8]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[e] = (float)r.a[e]; x[e + 4] = (float)r.b[e]; }
}
template <typename T>
__device__ __forceinline__ f32x4 f4(const vec4<T> &x) {
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}

// 16x16x16 fp32 product on the fp32 MFMA (four 16x16x4 steps). `a` holds row lr
// of the left factor at columns 4 lg .. 4 lg + 3 ("row layout"), `b` holds rows
// 4 lg .. 4 lg + 3 of the right factor at column lr ("column layout", which is
// also the accumulator layout of the result). The accumulator of a product
// X^T therefore is X in row layout.
__device__ __forceinline__ f32x4 bmm16(const f32x4 &a, const f32x4 &b, f32x4 acc) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[kk], b[kk], acc, 0, 0, 0);
    return acc;
}
__device__ __forceinline__ f32x4 lds4(const float *p) { return *(const f32x4 *)p; }
__device__ __forceinline__ f32x4 lds4col(const float *p, int ld) {   // p[0], p[ld], p[2 ld], p[3 ld]
    return f32x4{p[0], p[ld], p[2 * ld], p[3 * ld]};
}

// Workgroup -> (sequence * H + head, half of the state rows); the two halves of
// one (sequence, head) share its token data and go to one XCD (workgroups are
// dealt to the 8 XCDs round-robin by index).
__device__ __forceinline__ bool half_block(int64_t b, int64_t NH, int64_t &nh, int &half) {
    const int xcd = (int)(b & 7);
    const int64_t local = b >> 3;
    half = (int)(local & 1);
    nh = (local >> 1) * 8 + xcd;
    return nh < NH;
}

// ---- the chunk's operands --------------------------------------------------

// Raw token data of one chunk for the thread (token gid, lane j of its DPP row).
template <typename Tin, bool WITH_Q>
struct TokIn {
    Raw8<Tin> q, k;
    Raw8<float> g;
    float braw;
};

// Unconditional loads (no branch around them, so that the wait for a load
// issued one chunk ahead stays exact): a token past the sequence end reads the
// sequence's last token instead, and its values are ignored where used.
template <typename Tin, bool WITH_Q>
__device__ __forceinline__ void tok_load(TokIn<Tin, WITH_Q> &r, const Tin *q, const Tin *k,
                                         const float *g, const float *beta_raw, int64_t c0,
                                         int64_t s1, int H, int Hk, int h, int gid, int j) {
    const int64_t t = c0 + gid < s1 ? c0 + gid : s1 - 1;
    const size_t tbk = ((size_t)t * Hk + h / (H / Hk)) * kHeadDim;
    if constexpr (WITH_Q) raw8_load(r.q, q + tbk, j);
    raw8_load(r.k, k + tbk, j);
    raw8_load(r.g, g + ((size_t)t * H + h) * kHeadDim, j);
    r.braw = beta_raw[(size_t)t * H + h];
}

// Phase 1 (all threads, a DPP row per token): qh (scaled), kh and alpha of the
// token into the QG, KE and KG tiles, beta into B. Tokens past the sequence end
// act as q = k = 0, alpha = 1, beta = 0.
template <typename LY, bool WITH_Q, typename Tin>
__device__ __forceinline__ void operands_phase1(float *sm, const TokIn<Tin, WITH_Q> &r,
                                                const float (&dtb)[8], float a_gate, float lb,
                                                float scale, int L, int gid, int j) {
    float qh[8], kh[8], al[8], bb = 0.f;
    if (gid < L) {
        float qv[8], kv[8], gv[8];
        raw8_get(r.k, kv);
        raw8_get(r.g, gv);
        float sk = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sk = fmaf(kv[e], kv[e], sk);
        const float rk = rsqrtf(row16_sum(sk) + kL2Eps);
        if constexpr (WITH_Q) {
            raw8_get(r.q, qv);
            float sq = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) sq = fmaf(qv[e], qv[e], sq);
            const float rq = rsqrtf(row16_sum(sq) + kL2Eps) * scale;
#pragma unroll
            for (int e = 0; e < 8; ++e) qh[e] = qv[e] * rq;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kh[e] = kv[e] * rk;
            al[e] = fast_exp2(lb * sigmoid_f(a_gate * (gv[e] + dtb[e])) * kLog2e);
        }
        bb = sigmoid_f(r.braw);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { qh[e] = 0.f; kh[e] = 0.f; al[e] = 1.f; }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if constexpr (WITH_Q) sm[LY::QG + gid * kTP + chan(j, e)] = qh[e];
        sm[LY::KE + gid * kTP + chan(j, e)] = kh[e];
        sm[LY::KG + gid * kTP + chan(j, e)] = al[e];
    }
    if (j == 0) sm[LY::B + gid] = bb;
}

// Phase 2 (a thread per key channel): the products of alpha along the chunk
// (Gam_t up to and including t, SUF_t after t; products of at most 16 factors
// >= e^-5, so Gam >= e^-80 and never subnormal), and KE, QG, KG, KI written in
// place over the phase-1 values of the same column; GC into GC. With KEEP, Gam
// also stays in the GAM tile.
template <typename LY, bool WITH_Q, bool KEEP>
__device__ __forceinline__ void operands_phase2(float *sm, int tid) {
    if (tid < kHeadDim) {
        const int c = tid;
        float al[16], kh[16], qh[16], gam[16], suf[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            al[t] = sm[LY::KG + t * kTP + c];
            kh[t] = sm[LY::KE + t * kTP + c];
            if constexpr (WITH_Q) qh[t] = sm[LY::QG + t * kTP + c];
        }
        float run = 1.f;
#pragma unroll
        for (int t = 0; t < 16; ++t) { run *= al[t]; gam[t] = run; }
        run = 1.f;
#pragma unroll
        for (int t = 15; t >= 0; --t) { suf[t] = run; run *= al[t]; }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            sm[LY::KE + t * kTP + c] = kh[t] * gam[t];
            if constexpr (WITH_Q) sm[LY::QG + t * kTP + c] = qh[t] * gam[t];
            sm[LY::KG + t * kTP + c] = kh[t] * suf[t];
            sm[LY::KI + t * kTP + c] = kh[t] / gam[t];
            if constexpr (KEEP) sm[LY::GAM + t * kTP + c] = gam[t];
        }
        sm[LY::GC + c] = gam[15];
    }
}

// A = strict_lower(diag(b) P) with P = KE KI^T, from one wave (lane holds
// P[4 lg + i][lr]); the product's strictly lower part also kept in P_out if set.
// Returns the lane's accumulator (P[4 lg + i][lr], unmasked).
template <typename LY>
__device__ __forceinline__ f32x4 chunk_A(float *sm, int lane, float *P_out) {
    const int lr = lane & 15, lg = lane >> 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
        acc = bmm16(lds4(sm + LY::KE + lr * kTP + 16 * kb + 4 * lg), lds4(sm + LY::KI + lr * kTP + 16 * kb + 4 * lg), acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * lg + i;
        sm[LY::A + r * kSP + lr] = (r > lr) ? sm[LY::B + r] * acc[i] : 0.f;
        if (P_out) P_out[r * kSP + lr] = (r > lr) ? acc[i] : 0.f;
    }
    return acc;
}

// Column jc of X = (I + A)^-1 by forward substitution (A strictly lower), in
// registers: x[i] = delta(i, jc) - sum_{m < i} A[i][m] x[m].
__device__ __forceinline__ void inverse_column(const float *A, int jc, float (&x)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float acc = (i == jc) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < i; ++m) acc = fmaf(-A[i * kSP + m], x[m], acc);
        x[i] = acc;
    }
}

// The sequence and chunk whose operands live in `slot` (chunk c of sequence n
// is in slot cu[n] / 16 + n + c): the last n with cu[n] / 16 + n <= slot. False
// for a slot no chunk uses.
__device__ __forceinline__ bool slot_chunk(const int64_t *cu, int N, int64_t slot, int &n,
                                           int64_t &c) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] / kCk + mid <= slot) lo = mid;
        else hi = mid - 1;
    }
    n = lo;
    c = slot - (cu[n] / kCk + n);
    return c >= 0 && c < (cu[n + 1] - cu[n] + kCk - 1) / kCk;
}

// ---- per-chunk operand records --------------------------------------------------

// One record per (chunk slot, value head), written by bwd_prep_kernel and copied
// whole into LDS by the chunk-serial kernels (the LDS layout is the record's;
// offsets in floats, [16][128] tiles at pitch 132, [16][16] at pitch 20):
//   KE, KG, T = X diag(b), GC        (the checkpoint pass copies these, 19 KiB)
//   QG, MT = lower(QG KI^T)^T, B     (the reverse pass copies all of it, 28 KiB)
// and after those, read only by the finalize kernel:
//   X = (I + A)^-1, P = strict_lower(KE KI^T)   ([16][16] each at pitch 20)
struct OpRec {
    static constexpr int KE = 0, KG = KE + kTile, T = KG + kTile, GC = T + kSmall;
    static constexpr int QG = GC + kHeadDim, MT = QG + kTile, B = MT + kSmall;
    static constexpr int END = 7168;                     // 28 blocks of 1 KiB
    static constexpr int CKPT_BLOCKS = 19;               // blocks holding KE, KG, T, GC
    static constexpr int X = END, P = X + kSmall;
    static constexpr int STRIDE = P + kSmall;            // floats per record
};
static_assert(OpRec::B + 16 <= OpRec::END && OpRec::GC + kHeadDim <= 256 * OpRec::CKPT_BLOCKS,
              "record layout");
static_assert(OpRec::QG % 4 == 0 && OpRec::T % 4 == 0 && OpRec::GC % 4 == 0, "16-byte aligned tiles");

// LDS of bwd_prep_kernel: the record, then KI and A.
struct PrepLds {
    static constexpr int KE = OpRec::KE, KG = OpRec::KG, T = OpRec::T, GC = OpRec::GC;
    static constexpr int QG = OpRec::QG, MT = OpRec::MT, B = OpRec::B;
    static constexpr int KI = OpRec::END, A = KI + kTile, END = A + kSmall;
    static constexpr int XS = KI, PS = XS + kSmall;       // X, P once KI is no longer read
    static constexpr size_t BYTES = (size_t)END * 4;
};

// One workgroup per (chunk slot, value head), chunk-parallel: the chunk's
// transforms and decays (operands_phase1/2), A and M (waves 0 and 1, MFMA),
// X = (I + A)^-1 (wave 0), T = X diag(b), then the record written out, with X
// and P (staged in the KI tile, which is no longer read by then) after it.
template <typename Tin>
__global__ __launch_bounds__(256) void bwd_prep_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta_raw, const float *__restrict__ A_log,
    const float *__restrict__ dt_bias, float scale, float lb, const int64_t *__restrict__ cu, int N,
    int H, int Hk, float *__restrict__ ops)
{
    using LY = PrepLds;
    extern __shared__ __align__(16) float sm[];
    const int64_t slot = blockIdx.x;
    const int h = blockIdx.y;
    int n;
    int64_t c;
    if (!slot_chunk(cu, N, slot, n, c)) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4, gid = tid >> 4, j = tid & 15;
    const int64_t s1 = cu[n + 1], c0 = cu[n] + c * kCk;
    const int L = (int)(s1 - c0 < kCk ? s1 - c0 : kCk);
    const float a_gate = fast_exp2(A_log[h] * kLog2e);
    float dtb[8];
    load_lane8(dt_bias + (size_t)h * kHeadDim, j, dtb);
    {
        TokIn<Tin, true> tk;
        tok_load(tk, q, k, g, beta_raw, c0, s1, H, Hk, h, gid, j);
        operands_phase1<LY, true>(sm, tk, dtb, a_gate, lb, scale, L, gid, j);
    }
    lds_barrier();
    operands_phase2<LY, true, false>(sm, tid);
    lds_barrier();
    f32x4 pacc = {0.f, 0.f, 0.f, 0.f};
    if (wave == 0) pacc = chunk_A<LY>(sm, lane, nullptr);
    if (wave == 1) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
            acc = bmm16(lds4(sm + LY::QG + lr * kTP + 16 * kb + 4 * lg), lds4(sm + LY::KI + lr * kTP + 16 * kb + 4 * lg), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * lg + i;
            sm[LY::MT + lr * kSP + r] = (r >= lr) ? acc[i] : 0.f;
        }
    }
    lds_barrier();
    if (wave == 0) {
        float x[16];
        inverse_column(sm + LY::A, lr, x);
        if (lg == 0) {
            const float bj = sm[LY::B + lr];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                sm[LY::T + i * kSP + lr] = x[i] * bj;
                sm[LY::XS + i * kSP + lr] = x[i];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * lg + i;
            sm[LY::PS + r * kSP + lr] = (r > lr) ? pacc[i] : 0.f;
        }
    }
    lds_barrier();
    f32x4 *dst = (f32x4 *)(ops + ((size_t)slot * H + h) * OpRec::STRIDE);
#pragma unroll
    for (int r = 0; r < OpRec::END / 1024; ++r) dst[tid + 256 * r] = lds4(sm + 4 * (tid + 256 * r));
    if (tid < 2 * kSmall / 4) dst[OpRec::X / 4 + tid] = lds4(sm + LY::XS + 4 * tid);
}

// DMA copy of blocks [0, nblk) of a record into LDS: wave w copies the 1 KiB
// blocks w, w + 4, ... (completion tracked by vmcnt; readers wait, then a barrier).
template <int NBLK>
__device__ __forceinline__ void copy_record(const float *rec, float *lds, int wave, int lane) {
    const i32x4 r = make_rsrc(rec, (uint32_t)(OpRec::END * 4));
#pragma unroll
    for (int b = 0; b < (NBLK + 3) / 4; ++b) {
        const int blk = 4 * b + wave;
        if (4 * b + 3 < NBLK || blk < NBLK) {
            // wave-uniform by construction; made scalar explicitly for the copy's operands
            const int sblk = __builtin_amdgcn_readfirstlane(blk);
            copy16_to_lds(r, 16u * (uint32_t)lane, 1024u * (uint32_t)sblk, lds + 256 * sblk);
        }
    }
}

// Wait until at most N of this wave's vector memory operations are in flight
// (they complete in issue order): N is split over the two vmcnt fields.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 0xF) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
}

// ---- forward checkpoints ------------------------------------------------------

// The state of 16 rows per wave in registers as the transposed accumulator
// tiles Sa[kb][i] = S[vbase + lr][16 kb + 4 lg + i]; per chunk: the checkpoint,
// R = V - KE S^T (also stored: the reverse pass reads it back), U = T R,
// S^T <- diag(GC) S^T + KG^T U, with the next chunk's operands copied into the
// other LDS buffer meanwhile.
template <typename Tin>
__global__ __launch_bounds__(256) void bwd_ckpt_kernel(
    const Tin *__restrict__ v, const float *__restrict__ ops, const int64_t *__restrict__ cu,
    int N, int H, const float *__restrict__ h0, float *__restrict__ ckpt, float *__restrict__ rr)
{
    constexpr int BUF = 256 * OpRec::CKPT_BLOCKS;
    extern __shared__ __align__(16) float sm[];
    int64_t nh;
    int half;
    if (!half_block(blockIdx.x, (int64_t)N * H, nh, half)) return;
    const int n = (int)(nh / H), h = (int)(nh % H);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int vbase = 64 * half + 16 * wave;
    const int64_t s0 = cu[n], s1 = cu[n + 1];
    const int64_t nch = (s1 - s0 + kCk - 1) / kCk;
    const int64_t slot0 = s0 / kCk + n;
    const float *rec0 = ops + ((size_t)slot0 * H + h) * OpRec::STRIDE;
    const size_t rec_step = (size_t)H * OpRec::STRIDE;

    f32x4 Sa[8];
    if (h0) {
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
            Sa[kb] = *(const f32x4 *)(h0 + ((size_t)nh * kHeadDim + vbase + lr) * kHeadDim + 16 * kb + 4 * lg);
    } else {
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) Sa[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) asm volatile("" ::"v"(Sa[kb]));   // settled before the chunk loop
    if (nch == 0) return;
    // v[t = 4 lg + i][vbase + lr] of one chunk, loaded one chunk ahead
    // (tokens past the sequence end read its last token, masked where used)
    Tin vb[4];
    auto fetch_v = [&](int64_t c) {
        const int64_t c0 = s0 + c * kCk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t t = c0 + 4 * lg + i < s1 ? c0 + 4 * lg + i : s1 - 1;
            vb[i] = v[((size_t)t * H + h) * kHeadDim + vbase + lr];
        }
    };
    copy_record<OpRec::CKPT_BLOCKS>(rec0, sm, wave, lane);
    fetch_v(0);
    wait_vmem_le<0>();
    lds_barrier();
    // v of the current chunk as floats (masked past the sequence end); each
    // chunk converts the next chunk's values after its end-of-chunk wait, so
    // that no load is waited for at the top of the loop
    auto v_of = [&](int64_t c) {
        const int64_t c0 = s0 + c * kCk;
        const int L = (int)(s1 - c0 < kCk ? s1 - c0 : kCk);
        f32x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = 4 * lg + i < L ? (float)vb[i] : 0.f;
        return x;
    };
    f32x4 Vb = v_of(0);
    for (int64_t c = 0; c < nch; ++c) {
        const float *OP = sm + (c & 1) * BUF;
        // the next chunk's operands (the last chunk's again at the end) and v
        const int64_t cn = c + 1 < nch ? c + 1 : c;
        copy_record<OpRec::CKPT_BLOCKS>(rec0 + cn * rec_step, sm + ((c + 1) & 1) * BUF, wave, lane);
        fetch_v(cn);
        asm volatile("" ::: "memory");   // keep the loads here, a whole chunk ahead of their use
        float *ck = ckpt + ((size_t)(slot0 + c) * H + h) * kHeadDim * kHeadDim;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
            *(f32x4 *)(ck + (size_t)(vbase + lr) * kHeadDim + 16 * kb + 4 * lg) = Sa[kb];
        f32x4 R = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
            R = bmm16(lds4(OP + OpRec::KE + lr * kTP + 16 * kb + 4 * lg), Sa[kb], R);
        R = Vb - R;
        const f32x4 U = bmm16(lds4(OP + OpRec::T + lr * kSP + 4 * lg), R, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
            Sa[kb] = bmm16(lds4col(OP + OpRec::KG + (4 * lg) * kTP + 16 * kb + lr, kTP), U,
                           Sa[kb] * lds4(OP + OpRec::GC + 16 * kb + 4 * lg));
        // R of this wave's rows kept for the reverse pass, in lane order (stored
        // here rather than where it is formed: a store in the middle of the MFMA
        // stream measurably stalls it)
        *(f32x4 *)(rr + ((((size_t)(slot0 + c) * H + h) * 2 + half) * 4 + wave) * 256 + 4 * lane) = R;
        // the copy and the v loads landed (the 9 stores may still be in flight)
        wait_vmem_le<9>();
        Vb = v_of(cn);
        asm volatile("" ::"v"(Vb));
        lds_barrier();
    }
}

// ---- reverse pass -------------------------------------------------------------

// LDS of bwd_chunk_kernel: two record buffers, and two buffers of the rows
// the chain waves share with the partial waves: dS1 of the workgroup's 64
// state rows [64][132], and U, -dR (row layouts), dU and R ([t][v]) at pitch 68.
struct ChunkLds {
    static constexpr int SP = 68;
    static constexpr int REC = 0, SH = 2 * OpRec::END;
    static constexpr int DS1 = 0, US = DS1 + 64 * kTP, DRS = US + 16 * SP, DUS = DRS + 16 * SP;
    static constexpr int RS = DUS + 16 * SP, SHB = RS + 16 * SP;     // one share buffer
    static constexpr int END = SH + 2 * SHB;
    static constexpr size_t BYTES = (size_t)END * 4;
};
static_assert(ChunkLds::BYTES <= 160 * 1024, "LDS budget");

// A chain wave's inputs for one chunk: R of its rows (from the checkpoint pass)
// and dO of its rows in the column layout.
template <typename Tdo>
struct ChainIn {
    f32x4 R;               // R[t = 4 lg + i][vbase + lr]
    Tdo dOb[4];            // dO[t = 4 lg + i][vbase + lr]
};
// A partial wave's inputs: the column operand of S0 over the workgroup's 64 rows
// and the wave's 32 key columns, and dO of the 64 rows in the row layout.
template <typename Tdo>
struct PartIn {
    f32x4 S0s[8];          // [2 vb + kt]: S0[64 half + 16 vb + 4 lg + i][kcol + 16 kt + lr]
    vec4<Tdo> dOr[4];      // [vb]: dO[t = lr][64 half + 16 vb + 4 lg + kk]
};

template <typename Tdo>
__device__ __forceinline__ void settle(const ChainIn<Tdo> &r) {
    asm volatile("" ::"v"(r.R));
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" ::"v"((float)r.dOb[i]));
}

// Unconditional loads: tokens past the sequence end read its last token (masked where used).
template <typename Tdo>
__device__ __forceinline__ void chain_load(ChainIn<Tdo> &r, const float *rr, const Tdo *dout,
                                           int64_t slot, int64_t c0, int64_t s1, int H, int h,
                                           int half, int wave, int lane) {
    const int lr = lane & 15, lg = lane >> 4;
    const int vbase = 64 * half + 16 * wave;
    r.R = *(const f32x4 *)(rr + ((((size_t)slot * H + h) * 2 + half) * 4 + wave) * 256 + 4 * lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t t = c0 + 4 * lg + i < s1 ? c0 + 4 * lg + i : s1 - 1;
        r.dOb[i] = dout[((size_t)t * H + h) * kHeadDim + vbase + lr];
    }
}
template <typename Tdo>
__device__ __forceinline__ void part_load(PartIn<Tdo> &r, const float *ckpt, const Tdo *dout,
                                          int64_t slot, int64_t c0, int64_t s1, int H, int h,
                                          int half, int kcol, int lane) {
    const int lr = lane & 15, lg = lane >> 4;
    const float *ck = ckpt + ((size_t)slot * H + h) * kHeadDim * kHeadDim;
#pragma unroll
    for (int vb = 0; vb < 4; ++vb)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                r.S0s[2 * vb + kt][i] = ck[(size_t)(64 * half + 16 * vb + 4 * lg + i) * kHeadDim + kcol + 16 * kt + lr];
    const int64_t t = c0 + lr < s1 ? c0 + lr : s1 - 1;
#pragma unroll
    for (int vb = 0; vb < 4; ++vb)
        r.dOr[vb] = *(const vec4<Tdo> *)(dout + ((size_t)t * H + h) * kHeadDim + 64 * half + 16 * vb + 4 * lg);
}

// Eight waves per workgroup (sequence, head, half of the state rows). Waves 0-3
// (the chain) carry dS for 16 rows each through chunk c: dU, dR (dv), dS0, and
// write their rows of dS1, U, -dR, dU and R to a share buffer. Waves 4-7 (the
// partials) meanwhile form the partial sums of chunk c + 1 from the other share
// buffer, each for 32 key columns over the 64 rows, and write them over the
// checkpoint rows of that chunk (which only they read, one step earlier). The
// two MFMA streams share each SIMD; one barrier per step hands the buffers over.
template <typename Tdo>
__global__ __launch_bounds__(512) void bwd_chunk_kernel(
    const float *__restrict__ ops, const int64_t *__restrict__ cu, int N, int H, float *ckpt,
    const float *__restrict__ rr, const Tdo *__restrict__ dout, const float *__restrict__ dht,
    float *__restrict__ dv, float *__restrict__ dh0)
{
    using LY = ChunkLds;
    extern __shared__ __align__(16) float sm[];
    int64_t nh;
    int half;
    if (!half_block(blockIdx.x, (int64_t)N * H, nh, half)) return;
    const int n = (int)(nh / H), h = (int)(nh % H);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const bool chainw = wave < 4;
    const int cw = __builtin_amdgcn_readfirstlane(wave & 3);  // index within the role
    const int lr = lane & 15, lg = lane >> 4;
    const int vloc = 16 * cw, vbase = 64 * half + vloc;      // a chain wave's state rows
    const int kcol = 32 * cw;                                // a partial wave's key columns
    const int64_t s0 = cu[n], s1 = cu[n + 1];
    const int64_t nch = (s1 - s0 + kCk - 1) / kCk;
    const int64_t slot0 = s0 / kCk + n;
    const float *rec0 = ops + ((size_t)slot0 * H + h) * OpRec::STRIDE;
    const size_t rec_step = (size_t)H * OpRec::STRIDE;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    // chain waves: dSa[kb] = dS[vbase + lr][16 kb + 4 lg + i], the adjoint of the
    // state after the current chunk
    f32x4 dSa[8];
    if (chainw && dht) {
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
            dSa[kb] = *(const f32x4 *)(dht + ((size_t)nh * kHeadDim + vbase + lr) * kHeadDim + 16 * kb + 4 * lg);
    } else {
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) dSa[kb] = zero;
    }
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) asm volatile("" ::"v"(dSa[kb]));   // settled before the loop

    ChainIn<Tdo> cA, cB;
    PartIn<Tdo> pA, pB;
    if (chainw && nch > 0) {
        const int64_t c = nch - 1;
        copy_record<OpRec::END / 256>(rec0 + c * rec_step, sm + LY::REC, cw, lane);
        chain_load(cA, rr, dout, slot0 + c, s0 + c * kCk, s1, H, h, half, cw, lane);
        wait_vmem_le<0>();
        settle(cA);
    }
    lds_barrier();

    // Step i: the chain on chunk nch - 1 - i, the partials on chunk nch - i; each
    // role runs its own loop (so that neither keeps the other's registers live),
    // with one barrier per step in both.
    auto cstep = [&](int64_t i, ChainIn<Tdo> &ccur, ChainIn<Tdo> &cnxt) __attribute__((always_inline)) {
        const int sb = (int)(i & 1);
        {
            const int64_t c = nch - 1 - i;
            if (c >= 0) {
                const float *OP = sm + LY::REC + sb * OpRec::END;
                float *SH = sm + LY::SH + sb * LY::SHB;
                const int64_t c0 = s0 + c * kCk;
                const int L = (int)(s1 - c0 < kCk ? s1 - c0 : kCk);
                {   // the chunk before (chunk 0 again in the last pass: the loads stay unconditional)
                    const int64_t cp = c > 0 ? c - 1 : 0;
                    copy_record<OpRec::END / 256>(rec0 + cp * rec_step, sm + LY::REC + (sb ^ 1) * OpRec::END, cw, lane);
                    chain_load(cnxt, rr, dout, slot0 + cp, s0 + cp * kCk, s1, H, h, half, cw, lane);
                }
                f32x4 dOb;
#pragma unroll
                for (int i2 = 0; i2 < 4; ++i2) dOb[i2] = 4 * lg + i2 < L ? (float)ccur.dOb[i2] : 0.f;
                const f32x4 R = ccur.R;   // V - KE S0^T ([t][v] accumulator; zero past the end)
                // KG dS1^T ([t][v] accumulator); dS1 shared
                f32x4 dUk = zero;
#pragma unroll
                for (int kb = 0; kb < 8; ++kb) {
                    dUk = bmm16(lds4(OP + OpRec::KG + lr * kTP + 16 * kb + 4 * lg), dSa[kb], dUk);
                    *(f32x4 *)(SH + LY::DS1 + (vloc + lr) * kTP + 16 * kb + 4 * lg) = dSa[kb];
                }
                // dS <- dS1 diag(GC) + QG^T dO
#pragma unroll
                for (int kb = 0; kb < 8; ++kb)
                    dSa[kb] = bmm16(lds4col(OP + OpRec::QG + (4 * lg) * kTP + 16 * kb + lr, kTP), dOb,
                                    dSa[kb] * lds4(OP + OpRec::GC + 16 * kb + 4 * lg));
                // U in row layout (the accumulator of U^T = R^T T^T); dU = M^T dO + KG dS1^T;
                // dR = T^T dU (= dv) and its row layout (the accumulator of dR^T = dU^T T)
                const f32x4 Trow = lds4(OP + OpRec::T + lr * kSP + 4 * lg);
                const f32x4 Tcol = lds4col(OP + OpRec::T + (4 * lg) * kSP + lr, kSP);
                const f32x4 Ua = bmm16(R, Trow, zero);
                const f32x4 dU = bmm16(lds4(OP + OpRec::MT + lr * kSP + 4 * lg), dOb, dUk);
                const f32x4 ndR = -bmm16(Tcol, dU, zero);
                const f32x4 ndRa = -bmm16(dU, Tcol, zero);
#pragma unroll
                for (int i2 = 0; i2 < 4; ++i2)
                    if (4 * lg + i2 < L) dv[((size_t)(c0 + 4 * lg + i2) * H + h) * kHeadDim + vbase + lr] = -ndR[i2];
                // dS0^T = ... - KE^T dR
#pragma unroll
                for (int kb = 0; kb < 8; ++kb)
                    dSa[kb] = bmm16(lds4col(OP + OpRec::KE + (4 * lg) * kTP + 16 * kb + lr, kTP), ndR, dSa[kb]);
                // this wave's rows of U, -dR (row layouts), dU, R ([t][v]) shared
                *(f32x4 *)(SH + LY::US + lr * LY::SP + vloc + 4 * lg) = Ua;
                *(f32x4 *)(SH + LY::DRS + lr * LY::SP + vloc + 4 * lg) = ndRa;
#pragma unroll
                for (int i2 = 0; i2 < 4; ++i2) {
                    const int o = (4 * lg + i2) * LY::SP + vloc + lr;
                    SH[LY::DUS + o] = dU[i2];
                    SH[LY::RS + o] = R[i2];
                }
                // the next record and inputs landed; settled here, where the
                // hardware has them (the compiler does not see the record copy, so
                // a wait it placed at the next step would wait for the next copy too)
                wait_vmem_le<0>();
                settle(cnxt);
            }
        }
        lds_barrier();
    };
    auto pstep = [&](int64_t i, PartIn<Tdo> &pcur, PartIn<Tdo> &pnxt) __attribute__((always_inline)) {
        const int sb = (int)(i & 1);
        // lane indices taken as new in each step, so that the per-lane offsets are
        // formed where they are used instead of being kept live (and spilled)
        int lane = (int)threadIdx.x & 63;
        asm volatile("" : "+v"(lane));
        const int lr = lane & 15, lg = lane >> 4;
        {
            const int64_t cp = nch - i;            // the partials' chunk
            if (nch - 1 - i >= 0)                  // inputs of the chunk after it, for the next step
                part_load(pnxt, ckpt, dout, slot0 + (nch - 1 - i), s0 + (nch - 1 - i) * kCk, s1, H, h,
                          half, kcol, lane);
            if (cp <= nch - 1) {
                const float *SH = sm + LY::SH + (sb ^ 1) * LY::SHB;
                const int64_t c0 = s0 + cp * kCk;
                const int L = (int)(s1 - c0 < kCk ? s1 - c0 : kCk);
                f32x4 dOr[4];
#pragma unroll
                for (int vb = 0; vb < 4; ++vb) dOr[vb] = lr < L ? f4<Tdo>(pcur.dOr[vb]) : zero;
                // dQG = dO S0, dKG = U dS1, dKE = -dR S0 ([t][k] accumulators), dGC = sum_v S0 dS1
                f32x4 pq[2] = {zero, zero}, pk[2] = {zero, zero}, pe[2] = {zero, zero};
                float gs[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
                // dM = lower(dO U^T) (waves 4, 5) and dT = dU R^T (waves 6, 7), each
                // over 32 of the 64 rows (the final kernel adds the two parts): its
                // two products interleaved with the others, so that their latency
                // does not trail the step
                const bool isM = cw < 2;
                const int vb0 = 2 * (cw & 1);
                f32x4 accM = zero;
#pragma unroll
                for (int vb = 0; vb < 4; ++vb) {
                    if (vb & 1) {
                        const int vm = vb0 + (vb >> 1);
                        const f32x4 a_ = isM ? dOr[vm] : lds4(SH + LY::DUS + lr * LY::SP + 16 * vm + 4 * lg);
                        accM = bmm16(a_, lds4(SH + (isM ? LY::US : LY::RS) + lr * LY::SP + 16 * vm + 4 * lg), accM);
                    }
                    const f32x4 a_u = lds4(SH + LY::US + lr * LY::SP + 16 * vb + 4 * lg);
                    const f32x4 a_dr = lds4(SH + LY::DRS + lr * LY::SP + 16 * vb + 4 * lg);
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt) {
                        const f32x4 s0c = pcur.S0s[2 * vb + kt];
                        const f32x4 ds1c = lds4col(SH + LY::DS1 + (16 * vb + 4 * lg) * kTP + kcol + 16 * kt + lr, kTP);
                        pq[kt] = bmm16(dOr[vb], s0c, pq[kt]);
                        pk[kt] = bmm16(a_u, ds1c, pk[kt]);
                        pe[kt] = bmm16(a_dr, s0c, pe[kt]);
#pragma unroll
                        for (int i2 = 0; i2 < 4; ++i2) gs[kt][i2] = fmaf(s0c[i2], ds1c[i2], gs[kt][i2]);
                    }
                }
                // over this half's checkpoint rows of the chunk, which these waves
                // alone read and have read (loaded one step earlier)
                float *dst = ckpt + ((size_t)(slot0 + cp) * H + h) * kHeadDim * kHeadDim + (size_t)half * 64 * kHeadDim;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i2 = 0; i2 < 4; ++i2) {
                        const int o = (4 * lg + i2) * kHeadDim + kcol + 16 * kt + lr;
                        dst[o] = pq[kt][i2];
                        dst[2048 + o] = pk[kt][i2];
                        dst[4096 + o] = pe[kt][i2];
                    }
                // dGC: the 16 rows 4 lg + i of each block summed over i, then over the four lane groups
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    float x = (gs[kt][0] + gs[kt][1]) + (gs[kt][2] + gs[kt][3]);
                    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
                    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
                    const auto b2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
                    x = __uint_as_float(b2[0]) + __uint_as_float(b2[1]);
                    if (lg == 0) dst[6656 + kcol + 16 * kt + lr] = x;
                }
                {
                    const int off = (isM ? 6144 : 6400) + (cw & 1) * 640;
#pragma unroll
                    for (int i2 = 0; i2 < 4; ++i2) {
                        const int r = 4 * lg + i2;
                        dst[off + r * 16 + lr] = (!isM || r >= lr) ? accM[i2] : 0.f;
                    }
                }
            }
        }
        lds_barrier();
    };
    if (chainw) {
        for (int64_t i = 0;; i += 2) {
            cstep(i, cA, cB);
            if (i + 1 > nch) break;
            cstep(i + 1, cB, cA);
            if (i + 2 > nch) break;
        }
        if (dh0) {
#pragma unroll
            for (int kb = 0; kb < 8; ++kb)
                *(f32x4 *)(dh0 + ((size_t)nh * kHeadDim + vbase + lr) * kHeadDim + 16 * kb + 4 * lg) = dSa[kb];
        }
    } else {
        for (int64_t i = 0;; i += 2) {
            pstep(i, pA, pB);
            if (i + 1 > nch) break;
            pstep(i + 1, pB, pA);
            if (i + 2 > nch) break;
        }
    }
}

// LDS of bwd_chunk_final_kernel. GAM holds the decay products up to each token;
// XE, XQ, XI the products dP KI, dM KI, dKI, the first two then overwritten in
// place by the per-token log-decay adjoint (DG) and dKG * KG (EK), which in turn
// becomes the per-token gate gradients (SP).
struct FinalLds {
    static constexpr int KE = 0, QG = KE + kTile, KG = QG + kTile, KI = KG + kTile;
    static constexpr int XI = KI + kTile, XE = XI + kTile, GAM = XE + kTile, XQ = GAM + kTile;
    static constexpr int DG = XE, EK = XQ, SP = EK;
    static constexpr int P = XQ + kTile, X = P + kSmall, DM = X + kSmall;
    static constexpr int DT = DM + kSmall, Y = DT + kSmall, DA = Y + kSmall;
    static constexpr int GC = DA + kSmall, DGC = GC + kHeadDim, B = DGC + kHeadDim;
    static constexpr int END = B + 16;
    static constexpr size_t BYTES = (size_t)END * 4;
};
static_assert(FinalLds::BYTES <= 80 * 1024, "two workgroups per CU");

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
#pragma unroll 8
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

// One workgroup per (chunk slot, q/k head): the value heads that share the
// q/k head (grouped value heads) run one after the other and add their dqh and
// dkh before the normalisations' chains. Per value head: the operands again
// (the same code as the operand kernel), X and P from the record that kernel
// wrote (the values it formed, so the same as the passes between used), the
// two halves' partials added, the small-matrix adjoints (dX, dA, dP, dbeta), then per
// token row dKE, dQG, dKI, dkh, dqh and the log-decay adjoint, its reverse sum
// over the chunk (a thread per channel), and the gate's chain.
template <typename Tin>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_chunk_final_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta_raw, const float *__restrict__ A_log,
    const float *__restrict__ dt_bias, float scale, float lb, const int64_t *__restrict__ cu, int N,
    int H, int Hk, const float *__restrict__ part, const float *__restrict__ ops,
    float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dg, float *__restrict__ dbeta,
    float *__restrict__ pp)
{
    using LY = FinalLds;
    extern __shared__ __align__(16) float sm[];
    const int64_t slot = blockIdx.x;
    const int hk = blockIdx.y, G = H / Hk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int gid = tid >> 4, j = tid & 15;
    constexpr int NC = kHeadDim + 1;

    int n;
    int64_t c;
    if (!slot_chunk(cu, N, slot, n, c)) {
        // a slot no chunk uses: its parameter sums are zero
        for (int gg = 0; gg < G; ++gg)
            for (int col = tid; col < NC; col += 256) pp[((size_t)slot * H + hk * G + gg) * NC + col] = 0.f;
        return;
    }
    const int64_t s0 = cu[n], s1 = cu[n + 1];
    const int64_t c0 = s0 + c * kCk;
    const int L = (int)(s1 - c0 < kCk ? s1 - c0 : kCk);

    float dqh[8], dkh[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { dqh[e] = 0.f; dkh[e] = 0.f; }
    TokIn<Tin, true> tk;
    for (int gg = 0; gg < G; ++gg) {
        const int h = hk * G + gg;
        // the thread index taken as new in each pass, so that the many per-thread
        // LDS offsets below are formed where they are used instead of being kept
        // live (and spilled) across the loop
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, gid = tid >> 4, j = tid & 15;
        const float a_gate = fast_exp2(A_log[h] * kLog2e);
        float dtb[8];
        load_lane8(dt_bias + (size_t)h * kHeadDim, j, dtb);
        // the two halves' partials (issued before the operands are formed)
        const float *p0 = part + ((size_t)slot * H + h) * kHeadDim * kHeadDim, *p1 = p0 + 64 * kHeadDim;
        float pq[8], pk[8], pe[8];
        {
            float x0[8], x1[8];
            load_lane8(p0 + gid * kHeadDim, j, x0);
            load_lane8(p1 + gid * kHeadDim, j, x1);
#pragma unroll
            for (int e = 0; e < 8; ++e) pq[e] = x0[e] + x1[e];
            load_lane8(p0 + 2048 + gid * kHeadDim, j, x0);
            load_lane8(p1 + 2048 + gid * kHeadDim, j, x1);
#pragma unroll
            for (int e = 0; e < 8; ++e) pk[e] = x0[e] + x1[e];
            load_lane8(p0 + 4096 + gid * kHeadDim, j, x0);
            load_lane8(p1 + 4096 + gid * kHeadDim, j, x1);
#pragma unroll
            for (int e = 0; e < 8; ++e) pe[e] = x0[e] + x1[e];
        }
        // dM and dT: two parts per half (rows 0-31 and 32-63 of the half)
        const float dMv = (p0[6144 + tid] + p0[6784 + tid]) + (p1[6144 + tid] + p1[6784 + tid]);
        const float dTv = (p0[6400 + tid] + p0[7040 + tid]) + (p1[6400 + tid] + p1[7040 + tid]);
        const float dGCv = tid < kHeadDim ? p0[6656 + tid] + p1[6656 + tid] : 0.f;
        // X and P of the chunk, as the operand kernel formed them (threads 0 .. 79: X,
        // 80 .. 159: P, four values each)
        f32x4 xp = {0.f, 0.f, 0.f, 0.f};
        if (tid < 2 * kSmall / 4)
            xp = ((const f32x4 *)(ops + ((size_t)slot * H + h) * OpRec::STRIDE + OpRec::X))[tid];

        // the token rows are kept (tk) for the gate chain below and for the dq, dk
        // chains after the loop, instead of being read again
        tok_load(tk, q, k, g, beta_raw, c0, s1, H, Hk, h, gid, j);
        operands_phase1<LY, true>(sm, tk, dtb, a_gate, lb, scale, L, gid, j);
        lds_barrier();
        operands_phase2<LY, true, true>(sm, tid);
        lds_barrier();
        sm[LY::DM + gid * kSP + j] = dMv;
        sm[LY::DT + gid * kSP + j] = dTv;
        if (tid < kHeadDim) sm[LY::DGC + tid] = dGCv;
        if (tid < 2 * kSmall / 4)
            *(f32x4 *)(sm + (tid < kSmall / 4 ? LY::X + 4 * tid : LY::P + 4 * (tid - kSmall / 4))) = xp;
        lds_barrier();
        // Y = dX X^T with dX = dT diag(b)
        {
            float y = 0.f;
#pragma unroll
            for (int jj = 0; jj < 16; ++jj)
                y = fmaf(sm[LY::DT + gid * kSP + jj] * sm[LY::B + jj], sm[LY::X + j * kSP + jj], y);
            sm[LY::Y + gid * kSP + j] = y;
        }
        lds_barrier();
        // dA = strict_lower(-X^T Y)
        {
            float d = 0.f;
            if (gid > j) {
#pragma unroll
                for (int i = 0; i < 16; ++i) d = fmaf(sm[LY::X + i * kSP + gid], sm[LY::Y + i * kSP + j], d);
                d = -d;
            }
            sm[LY::DA + gid * kSP + j] = d;
        }
        lds_barrier();
        if (tid < 16) {
            // db_t = sum_i X[i][t] dT[i][t] + sum_{m < t} dA[t][m] P[t][m]
            const int t = tid;
            float db = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) db = fmaf(sm[LY::X + i * kSP + t], sm[LY::DT + i * kSP + t], db);
#pragma unroll
            for (int m = 0; m < 16; ++m) db = fmaf(sm[LY::DA + t * kSP + m], sm[LY::P + t * kSP + m], db);
            if (t < L) {
                const float bb = sm[LY::B + t];
                dbeta[(size_t)(c0 + t) * H + h] = db * bb * (1.0f - bb);
            }
        }
        // dP KI, dM KI and dKI = dP^T KE + dM^T QG (dP = diag(b) dA) on the MFMA,
        // wave w for the key columns 32 w .. 32 w + 31, into the XE, XQ, XI tiles
        {
            const int lr = lane & 15, lg = lane >> 4;
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            const f32x4 dPr = lds4(sm + LY::DA + lr * kSP + 4 * lg) * sm[LY::B + lr];
            const f32x4 dMr = lds4(sm + LY::DM + lr * kSP + 4 * lg);
            const f32x4 dPc = lds4col(sm + LY::DA + (4 * lg) * kSP + lr, kSP) * lds4(sm + LY::B + 4 * lg);
            const f32x4 dMc = lds4col(sm + LY::DM + (4 * lg) * kSP + lr, kSP);
#pragma unroll
            for (int kbi = 0; kbi < 2; ++kbi) {
                const int col = 16 * (2 * wave + kbi) + lr;
                const f32x4 kic = lds4col(sm + LY::KI + (4 * lg) * kTP + col, kTP);
                const f32x4 kec = lds4col(sm + LY::KE + (4 * lg) * kTP + col, kTP);
                const f32x4 qgc = lds4col(sm + LY::QG + (4 * lg) * kTP + col, kTP);
                const f32x4 xe = bmm16(dPr, kic, z), xq = bmm16(dMr, kic, z);
                const f32x4 xi = bmm16(dMc, qgc, bmm16(dPc, kec, z));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int o = (4 * lg + i) * kTP + col;
                    sm[LY::XE + o] = xe[i];
                    sm[LY::XQ + o] = xq[i];
                    sm[LY::XI + o] = xi[i];
                }
            }
        }
        lds_barrier();
        // token row gid: dKE = dKE_p + dP KI, dQG = dQG_p + dM KI; dkh, dqh, the
        // per-token log-decay adjoint DG and dKG * KG (EK), over XE and XQ in place
        {
            float xe[8], xq[8], dki[8], gam[8], gcv[8], ke[8], qg[8], ki[8], kg[8], dgp[8], ek[8];
            load_lane8(sm + LY::XE + gid * kTP, j, xe);
            load_lane8(sm + LY::XQ + gid * kTP, j, xq);
            load_lane8(sm + LY::XI + gid * kTP, j, dki);
            load_lane8(sm + LY::GAM + gid * kTP, j, gam);
            load_lane8(sm + LY::GC, j, gcv);
            load_lane8(sm + LY::KE + gid * kTP, j, ke);
            load_lane8(sm + LY::QG + gid * kTP, j, qg);
            load_lane8(sm + LY::KI + gid * kTP, j, ki);
            load_lane8(sm + LY::KG + gid * kTP, j, kg);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float dke = pe[e] + xe[e], dqg = pq[e] + xq[e];
                const float suf = gcv[e] / gam[e];     // the decay after the token
                dkh[e] += dke * gam[e] + pk[e] * suf + dki[e] / gam[e];
                dqh[e] = fmaf(dqg, gam[e], dqh[e]);
                dgp[e] = dke * ke[e] + dqg * qg[e] - dki[e] * ki[e];
                ek[e] = pk[e] * kg[e];
            }
            store_lane8(sm + LY::DG + gid * kTP, j, dgp);
            store_lane8(sm + LY::EK + gid * kTP, j, ek);
        }
        lds_barrier();
        if (tid < kHeadDim) {
            // dlambda_t = sum_{s >= t} DG_s + sum_{s < t} dKG_s KG_s + GC dGC
            const int cc = tid;
            float dgs[16], suffix[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) dgs[t] = sm[LY::DG + t * kTP + cc];
            float run = 0.f;
#pragma unroll
            for (int t = 15; t >= 0; --t) { run += dgs[t]; suffix[t] = run; }
            const float base = sm[LY::GC + cc] * sm[LY::DGC + cc];
            float pre = 0.f;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                sm[LY::DG + t * kTP + cc] = (suffix[t] + pre) + base;
                pre += sm[LY::EK + t * kTP + cc];
            }
        }
        lds_barrier();
        float dgv[8];
        float cA = 0.f;
        if (gid < L) {
            const size_t tb = ((size_t)(c0 + gid) * H + h) * kHeadDim;
            float gv[8], dl[8];
            raw8_get(tk.g, gv);
            load_lane8(sm + LY::DG + gid * kTP, j, dl);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float sg = sigmoid_f(a_gate * (gv[e] + dtb[e]));
                dgv[e] = dl[e] * lb * sg * (1.0f - sg) * a_gate;
                cA = fmaf(dgv[e], gv[e] + dtb[e], cA);
            }
            store_lane8(dg + tb, j, dgv);
            cA = row16_sum(cA);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) dgv[e] = 0.f;
        }
        // this value head's sums over the chunk's tokens, for the parameters
        store_lane8(sm + LY::SP + gid * kTP, j, dgv);
        if (j == 0) sm[LY::SP + gid * kTP + kHeadDim] = cA;
        lds_barrier();
        if (tid < NC) {
            float sum = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) sum += sm[LY::SP + r * kTP + tid];
            pp[((size_t)slot * H + h) * NC + tid] = sum;
        }
        lds_barrier();
    }
    if (gid < L) {
        const size_t tbk = ((size_t)(c0 + gid) * Hk + hk) * kHeadDim;
        float qv[8], kv[8];
        raw8_get(tk.q, qv);
        raw8_get(tk.k, kv);
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

// One flag word per kernel: bit d set once its dynamic-LDS limit is set on device d.
hipError_t set_lds_limit(const void *fn, int lds, std::atomic<uint64_t> &done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_relaxed) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_relaxed);
    return e;
}

template <typename Tin, typename Tdo>
hipError_t launch_backward_t(const BackwardArgs &a) {
    const int Hk = a.Hk > 0 ? a.Hk : a.H;   // q/k heads (grouped value heads)
    const int64_t NH = (int64_t)a.N * a.H;
    const int64_t slots = num_slots(a.T, a.N, kCk);
    const unsigned grid = (unsigned)(((NH + 7) / 8) * 16);
    hipError_t e = hipSuccess;
    if (slots > 0) {
        bwd_prep_kernel<Tin><<<dim3((unsigned)slots, (unsigned)a.H), 256, PrepLds::BYTES, a.stream>>>(
            (const Tin *)a.q, (const Tin *)a.k, a.g, a.beta_raw, a.A_log, a.dt_bias, a.scale,
            a.lower_bound, a.cu, a.N, a.H, Hk, a.ops);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    bwd_ckpt_kernel<Tin><<<grid, 256, 2 * 256 * OpRec::CKPT_BLOCKS * 4, a.stream>>>(
        (const Tin *)a.v, a.ops, a.cu, a.N, a.H, a.h0, a.ckpt, a.rr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    static std::atomic<uint64_t> chunk_lds{0}, final_lds{0};
    e = set_lds_limit((const void *)&bwd_chunk_kernel<Tdo>, (int)ChunkLds::BYTES, chunk_lds);
    if (e != hipSuccess) return e;
    bwd_chunk_kernel<Tdo><<<grid, 512, ChunkLds::BYTES, a.stream>>>(
        a.ops, a.cu, a.N, a.H, a.ckpt, a.rr, (const Tdo *)a.dout, a.dht, a.dv, a.dh0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    e = set_lds_limit((const void *)&bwd_chunk_final_kernel<Tin>, (int)FinalLds::BYTES, final_lds);
    if (e != hipSuccess) return e;
    bwd_chunk_final_kernel<Tin><<<dim3((unsigned)slots, (unsigned)Hk), 256, FinalLds::BYTES, a.stream>>>(
        (const Tin *)a.q, (const Tin *)a.k, a.g, a.beta_raw, a.A_log, a.dt_bias, a.scale,
        a.lower_bound, a.cu, a.N, a.H, Hk, a.ckpt, a.ops, a.dq, a.dk, a.dg, a.dbeta, a.pp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    bwd_param_kernel<<<(unsigned)a.H, 256, 0, a.stream>>>(a.pp, slots, a.H, a.dA_log, a.ddt_bias);
    return hipGetLastError();
}

}  // namespace

BackwardLayout backward_layout(int64_t T, int N, int H) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    BackwardLayout l;
    const size_t slots = (size_t)num_slots(T, N, kCk);
    // (the reverse pass's partial records reuse the checkpoint rows)
    l.ckpt_bytes = up(slots * H * kHeadDim * kHeadDim * 4);
    l.pp_bytes = up(slots * H * (kHeadDim + 1) * 4);
    l.ops_bytes = up(slots * H * OpRec::STRIDE * 4);
    l.rr_bytes = up(slots * H * 2 * 4 * 256 * 4);
    l.total = l.ckpt_bytes + l.pp_bytes + l.ops_bytes + l.rr_bytes;
    return l;
}

hipError_t launch_backward(const BackwardArgs &a) {
    if (a.in_bf16)
        return a.do_bf16 ? launch_backward_t<__bf16, __bf16>(a) : launch_backward_t<__bf16, float>(a);
    return a.do_bf16 ? launch_backward_t<float, __bf16>(a) : launch_backward_t<float, float>(a);
}

}  // namespace kda
