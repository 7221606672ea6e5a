// Chunkwise KDA prefill: intra-chunk kernel (fully parallel over chunks and
// heads) and persistent inter-chunk kernel (serial over the chunks of each
// sequence, parallel over sequences, heads and 16-row blocks of the state).
//
// The chunk algebra (derived from the recurrence; the kda-neuron-kernels
// commit log only names the exact "16-sub-chunk + WY" prefill): inside a chunk
// of C rows starting from state S0 [V,K], with G the inclusive cumulative
// log-decay per key channel (restarting at the chunk start),
//   A[i,j] = beta_i sum_c kh_i[c] kh_j[c] e^{G_i[c]-G_j[c]}      (i > j)
//   T      = (I + A)^-1 diag(beta)
//   W      = T (kh * e^G)       Ub = T v
//   qg     = qh * e^G           M[i,j] = sum_c qh_i[c] kh_j[c] e^{G_i[c]-G_j[c]}  (i >= j)
//   kg     = kh * e^{G_C - G}   GamC = e^{G_C}
//   U      = Ub - W S0^T        O = qg S0^T + M U        S_C = S0 diag(GamC) + U^T kg
// Row v of S_C and column v of O depend on row v of S0 only, so the state is
// split into 16-row blocks, one wavefront each.
//
// Exponent range: G falls by up to 5 per token, so e^{-G} over a whole chunk
// overflows fp32. A and M are formed on 16-row sub-chunks with the reference
// G_r of the first row of the left block: left factors e^{G_i - G_r} <= 1, right
// factors e^{G_r - G_j} (<= 1 off the diagonal, <= e^{75} on it). This is why
// the pages insist on 16-row sub-chunks and a lower bound >= -5.
//
// Every decay factor is a product of per-token alpha = e^lambda over a row
// range, built from block-local prefix products P_t = prod_{s=16b+1..t} alpha_s
// (>= e^{-75}, never subnormal) and per-block totals. A cumulative sum of
// lambda in fp32 would reach ~-460 (log2 units) within a chunk and lose ~1e-4
// of absolute accuracy in every difference G_i - G_j; products keep each factor
// to a few fp32 ulps.
//
// Precision: bf16 inputs run the products on fp16 MFMA with fp32
// accumulation; operands that are not bounded by 1 (the state, U, v) are
// scaled by a power of two chosen from their wavefront / tile maximum, which is
// exact. Diagonal sub-chunk blocks (factors up to e^{75}) use a three-product
// bf16 split. fp32 inputs run every product on the fp32 MFMA.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

constexpr int KP = kHeadDim + 4;   // LDS row pitch (floats) of [C][128] tiles

size_t record_bytes(int chunk, bool precise) {
    switch (chunk) {
        case 16: return precise ? Record<16, true>::BYTES : Record<16, false>::BYTES;
        case 32: return precise ? Record<32, true>::BYTES : Record<32, false>::BYTES;
        case 64: return precise ? Record<64, true>::BYTES : Record<64, false>::BYTES;
        default: return 0;
    }
}

// ---- fragment policy: fp16 storage + fp16 MFMA, or fp32 storage + fp32 MFMA --

template <bool PRECISE> struct Frag;

template <> struct Frag<false> {
    using T = half8;
    static __device__ __forceinline__ T make(const float (&x)[8], float inv) {
        T r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = (_Float16)(x[e] * inv);
        return r;
    }
    static __device__ __forceinline__ T load(const void *p) { return *(const T *)p; }
    static __device__ __forceinline__ void store(void *p, const float (&x)[8]) {
        *(T *)p = make(x, 1.0f);
    }
    static __device__ __forceinline__ f32x4 mma(const T &a, const T &b, f32x4 c) {
        return mfma_h(a, b, c);
    }
    static constexpr int BYTES = 16;
};

template <> struct Frag<true> {
    struct T { float v[8]; };
    static __device__ __forceinline__ T make(const float (&x)[8], float) {
        T r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r.v[e] = x[e];
        return r;
    }
    static __device__ __forceinline__ T load(const void *p) {
        T r;
        const f32x4 a = ((const f32x4 *)p)[0], b = ((const f32x4 *)p)[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) { r.v[e] = a[e]; r.v[e + 4] = b[e]; }
        return r;
    }
    static __device__ __forceinline__ void store(void *p, const float (&x)[8]) {
        ((f32x4 *)p)[0] = f32x4{x[0], x[1], x[2], x[3]};
        ((f32x4 *)p)[1] = f32x4{x[4], x[5], x[6], x[7]};
    }
    static __device__ __forceinline__ f32x4 mma(const T &a, const T &b, f32x4 c) {
        return mfma_f32x8(a.v, b.v, c);
    }
    static constexpr int BYTES = 32;
};

__device__ __forceinline__ float inv_pow2(float s) {   // exact 1/s for s = 2^e
    return __uint_as_float((uint32_t)(254 - (int)((__float_as_uint(s) >> 23) & 0xFF)) << 23);
}

// Locate chunk `slot` of the packed batch: returns false for an unused slot.
template <int C>
__device__ __forceinline__ bool locate_slot(const int64_t *__restrict__ cu, int N, int64_t slot,
                                            int &n, int64_t &t0, int &L) {
    if (N <= 0) return false;
    int lo = 0, hi = N - 1;
    while (lo < hi) {                     // largest n with floor(cu[n]/C) + n <= slot
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] / C + mid <= slot) lo = mid; else hi = mid - 1;
    }
    n = lo;
    const int64_t s0 = cu[n], len = cu[n + 1] - s0;
    const int64_t j = slot - (s0 / C) - n;
    if (j < 0 || j * C >= len) return false;
    t0 = s0 + j * C;
    const int64_t rem = len - j * C;
    L = rem < C ? (int)rem : C;
    return true;
}

// =============================================================================
// Intra-chunk kernel: one workgroup (8 waves) per (chunk slot, head).
//
// LDS holds three [C][128] fp32 tiles that are rewritten in place as the phases
// go: sQ = qh -> qh*P -> v (scaled); sK = kh -> kh*P; sP = alpha -> P -> kh/P,
// with P_t the block-local prefix product of alpha. Every operand of A and M is
// then one of those rows times at most one per-(block, channel) factor.
// =============================================================================
constexpr int kIntraWaves = 8;

template <int C, typename Tin, bool PRECISE>
__global__ __launch_bounds__(64 * kIntraWaves) void intra_kernel(PrefillArgs p)
{
    using G = ChunkGeom<C>;
    using R = Record<C, PRECISE>;
    using F = Frag<PRECISE>;
    constexpr int NB = G::NB, CS = G::CS, NW = kIntraWaves, NT = 64 * NW;
    constexpr int AP = C + 4;
    constexpr int NPO = NB * (NB - 1) / 2 + 1;   // off-diagonal block pairs (+1: never empty)

    __shared__ __align__(16) float sQ[C][KP];
    __shared__ __align__(16) float sK[C][KP];
    __shared__ __align__(16) float sP[C][KP];
    __shared__ __align__(16) float sA[C][AP];   // A, strictly lower, beta-scaled
    __shared__ __align__(16) float sT[C][AP];   // M (staging), then T
    __shared__ __align__(16) float sA0[NB][kHeadDim];  // alpha of each block's first row
    __shared__ __align__(16) float sPe[NB][kHeadDim];  // P at each block's last row
    __shared__ __align__(16) float sQF[NB][kHeadDim];  // prod alpha over rows 0 .. 16b
    __shared__ __align__(16) float sKF[NB][kHeadDim];  // prod alpha over rows 16b+1 .. C-1
    __shared__ __align__(16) float sEF[NPO][kHeadDim]; // prod alpha over rows 16b+1 .. 16a
    __shared__ float sBeta[C];
    __shared__ float sInv[3][16][17];
    __shared__ float sVmax[NW];

    const int H = p.H;
    const int h = blockIdx.y;
    int n, L;
    int64_t t0;
    if (!locate_slot<C>(p.cu_seqlens, p.N, blockIdx.x, n, t0, L)) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    unsigned char *rec = p.ws + ((size_t)blockIdx.x * H + h) * R::BYTES;

    // ---- phase 1: rows; a DPP row of 16 lanes holds one token (8 channels per lane)
    constexpr int RG = C / 4;                   // groups of 4 rows
    constexpr int RIT = (RG + NW - 1) / NW;     // groups per wave
    const int c8 = 8 * lr;
    const float agate = fast_exp2(p.A_log[h] * kLog2e);
    const float lb2 = p.lower_bound * kLog2e;
    float db[8];
    load8(p.dt_bias + h * kHeadDim + c8, db);
    float vreg[RIT][8];
    float vmax = 0.f;
#pragma unroll
    for (int it = 0; it < RIT; ++it) {
        const int grp = wave + NW * it;
        if (grp >= RG) break;
        const int t = 4 * grp + lg;
        const bool valid = t < L;
        float qv[8], kv[8], gv[8];
        if (valid) {
            const size_t base = ((size_t)(t0 + t) * H + h) * kHeadDim + c8;
            load8((const Tin *)p.q + base, qv);
            load8((const Tin *)p.k + base, kv);
            load8((const Tin *)p.v + base, vreg[it]);
            load8(p.g + base, gv);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[e] = kv[e] = vreg[it][e] = gv[e] = 0.f;
        }
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) { sq += qv[e] * qv[e]; sk += kv[e] * kv[e]; }
        sq = row16_sum(sq);
        sk = row16_sum(sk);
        const float fq = rsqrtf(sq + kL2Eps) * p.scale, fk = rsqrtf(sk + kL2Eps);
        float al[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            qv[e] *= fq;
            kv[e] *= fk;
            // alpha = e^lambda; padding rows have lambda = 0
            al[e] = valid ? fast_exp2(lb2 * sigmoid_f(agate * (gv[e] + db[e]))) : 1.f;
            vmax = fmaxf(vmax, fabsf(vreg[it][e]));
        }
        *(f32x4 *)&sQ[t][c8] = f32x4{qv[0], qv[1], qv[2], qv[3]};
        *(f32x4 *)&sQ[t][c8 + 4] = f32x4{qv[4], qv[5], qv[6], qv[7]};
        *(f32x4 *)&sK[t][c8] = f32x4{kv[0], kv[1], kv[2], kv[3]};
        *(f32x4 *)&sK[t][c8 + 4] = f32x4{kv[4], kv[5], kv[6], kv[7]};
        *(f32x4 *)&sP[t][c8] = f32x4{al[0], al[1], al[2], al[3]};
        *(f32x4 *)&sP[t][c8 + 4] = f32x4{al[4], al[5], al[6], al[7]};
        if (lr == 0) sBeta[t] = valid ? sigmoid_f(p.beta_raw[(size_t)(t0 + t) * H + h]) : 0.f;
    }
    vmax = wave_max(vmax);
    if (lane == 0) sVmax[wave] = vmax;
    __syncthreads();

    // ---- phase 1b: block-local prefix products P_t = prod alpha_{16b+1 .. t} --
    if (tid < NB * kHeadDim) {
        const int b = tid / kHeadDim, c = tid % kHeadDim;
        float a[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) a[i] = sP[16 * b + i][c];
        sA0[b][c] = a[0];
        float run = 1.f;
        sP[16 * b][c] = 1.f;
#pragma unroll
        for (int i = 1; i < 16; ++i) { run *= a[i]; sP[16 * b + i][c] = run; }
        sPe[b][c] = run;
    }
    __syncthreads();

    // ---- phase 1c: per-channel block factors; qh*P, kh*P, kh/P in place --------
    if (tid < kHeadDim) {
        const int c = tid;
        float tot[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) tot[b] = sA0[b][c] * sPe[b][c];
        float pre = 1.f;
#pragma unroll
        for (int b = 0; b < NB; ++b) { sQF[b][c] = pre * sA0[b][c]; pre *= tot[b]; }
        float suf = 1.f;
#pragma unroll
        for (int b = NB - 1; b >= 0; --b) { sKF[b][c] = sPe[b][c] * suf; suf *= tot[b]; }
#pragma unroll
        for (int a = 1; a < NB; ++a) {
            float e = sA0[a][c];
#pragma unroll
            for (int b = a - 1; b >= 0; --b) {
                sEF[a * (a - 1) / 2 + b][c] = sPe[b][c] * e;
                e *= tot[b];
            }
        }
        ((float *)(rec + R::GC_OFF))[c] = pre;     // total decay of the chunk
    }
    for (int idx = tid; idx < C * (kHeadDim / 4); idx += NT) {
        const int t = idx / (kHeadDim / 4), c = 4 * (idx % (kHeadDim / 4));
        const f32x4 pp = *(const f32x4 *)&sP[t][c];
        const f32x4 kk = *(const f32x4 *)&sK[t][c];
        const f32x4 qq = *(const f32x4 *)&sQ[t][c];
        f32x4 kr;
#pragma unroll
        for (int e = 0; e < 4; ++e) kr[e] = kk[e] * fast_rcp(pp[e]);
        *(f32x4 *)&sQ[t][c] = qq * pp;
        *(f32x4 *)&sK[t][c] = kk * pp;
        *(f32x4 *)&sP[t][c] = kr;
    }
    __syncthreads();

    // ---- phase 2: A and M blocks; qg and kgT fragments ------------------------
    {
        constexpr int NP = NB * (NB + 1) / 2;
        for (int pi = wave; pi < NP; pi += NW) {
            int a = 0, b = pi;                       // pair index -> (a, b), b <= a
            while (b > a) { b -= a + 1; ++a; }
            const int il = 16 * a + lr, jr = 16 * b + lr;
            const float *ef = sEF[a * (a - 1) / 2 + b];   // only read when b < a
            f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int c = 32 * s + 8 * lg;
                float aK[8], aQ[8], bK[8];
                load8(&sK[il][c], aK);              // kh e^{G_i - G_16a}
                load8(&sQ[il][c], aQ);              // qh e^{G_i - G_16a}
                load8(&sP[jr][c], bK);              // kh / P_j
                if (a != b) {                        // e^{G_16a - G_j} = EF / P_j
                    float f[8];
                    load8(ef + c, f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) bK[e] *= f[e];
                }
                if constexpr (PRECISE) {
                    accA = mfma_f32x8(aK, bK, accA);
                    accM = mfma_f32x8(aQ, bK, accM);
                } else if (a == b) {                 // right factors up to e^75
                    accA = mfma_x3(aK, bK, accA);
                    accM = mfma_x3(aQ, bK, accM);
                } else {                             // all factors <= 1
                    accA = mfma_f16(aK, bK, accA);
                    accM = mfma_f16(aQ, bK, accM);
                }
            }
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int io = 16 * a + 4 * lg + ii, jo = 16 * b + lr;
                sA[io][jo] = (io > jo) ? sBeta[io] * accA[ii] : 0.f;
                sT[io][jo] = (io >= jo) ? accM[ii] : 0.f;
            }
        }
        constexpr int NQ = NB * 4, NKG = 8 * CS;
        for (int f = wave; f < NQ + NKG; f += NW) {
            float x[8];
            unsigned char *dst;
            if (f < NQ) {                            // qg = qh e^{G_t} = (qh P_t) QF
                const int tb = f >> 2, s = f & 3;
                const int t = 16 * tb + lr;
                const int c0 = 32 * s + 4 * lg;
                const f32x4 q0 = *(const f32x4 *)&sQ[t][c0], q1 = *(const f32x4 *)&sQ[t][c0 + 16];
                const f32x4 f0 = *(const f32x4 *)&sQF[tb][c0], f1 = *(const f32x4 *)&sQF[tb][c0 + 16];
#pragma unroll
                for (int e = 0; e < 4; ++e) { x[e] = q0[e] * f0[e]; x[e + 4] = q1[e] * f1[e]; }
                dst = rec + R::QG_OFF + ((size_t)(tb * 4 + s) * 64 + lane) * F::BYTES;
            } else {                                 // kg = kh e^{G_C - G_t} = (kh / P_t) KF
                const int kb = (f - NQ) / CS, s = (f - NQ) % CS;
                const int c = 16 * kb + lr;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int t = 32 * s + kperm(lg, e);
                    x[e] = (t < C) ? sP[t][c] * sKF[t >> 4][c] : 0.f;
                }
                dst = rec + R::KG_OFF + ((size_t)(kb * CS + s) * 64 + lane) * F::BYTES;
            }
            F::store(dst, x);
        }
    }
    // power-of-two scale of v for the fp16 product T v (exact)
    float vscale = 1.0f;
    if constexpr (!PRECISE) {
        float m = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) m = fmaxf(m, sVmax[w]);
        vscale = pow2_scale_for(m, 12);
    }
    const float vinv = inv_pow2(vscale);
    __syncthreads();

    // ---- phase 3: M fragments out; v (scaled) into sQ --------------------------
    for (int f = wave; f < NB * CS; f += NW) {
        const int tb = f / CS, s = f % CS;
        const int t = 16 * tb + lr;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int tp = 32 * s + kperm(lg, e);
            x[e] = (tp <= t && tp < C) ? sT[t][tp] : 0.f;
        }
        F::store(rec + R::M_OFF + ((size_t)(tb * CS + s) * 64 + lane) * F::BYTES, x);
    }
#pragma unroll
    for (int it = 0; it < RIT; ++it) {
        const int grp = wave + NW * it;
        if (grp >= RG) break;
        const int t = 4 * grp + lg;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = vreg[it][e] * vinv;
        *(f32x4 *)&sQ[t][c8] = f32x4{x[0], x[1], x[2], x[3]};
        *(f32x4 *)&sQ[t][c8 + 4] = f32x4{x[4], x[5], x[6], x[7]};
    }
    __syncthreads();

    // ---- phase 4: T = (I + A)^-1 diag(beta) by blocked forward substitution ---
    if (tid < 16 * NB) {                       // diagonal 16x16 blocks, one column each
        const int a = tid >> 4, c = tid & 15, o = 16 * a;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = (i == c) ? 1.0f : 0.0f;
#pragma unroll
            for (int jj = 0; jj < i; ++jj) acc -= sA[o + i][o + jj] * x[jj];
            x[i] = (i < c) ? 0.0f : acc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sT[o + i][o + c] = x[i];
    }
    for (int idx = tid; idx < C * C; idx += NT) {   // zero the blocks above the diagonal
        const int i = idx / C, j = idx % C;
        if ((j >> 4) > (i >> 4)) sT[i][j] = 0.0f;
    }
    __syncthreads();
    for (int d = 1; d < NB; ++d) {
        const int ii = (tid >> 4) & 15, jj = tid & 15;
        const bool act = tid < 256;
        for (int a = d; act && a < NB; ++a) {     // P = sum_{c=b}^{a-1} A_ac X_cb
            const int b = a - d;
            float acc = 0.f;
            for (int c = b; c < a; ++c)
#pragma unroll
                for (int m = 0; m < 16; ++m) acc += sA[16 * a + ii][16 * c + m] * sT[16 * c + m][16 * b + jj];
            sInv[a - d][ii][jj] = acc;
        }
        __syncthreads();
        for (int a = d; act && a < NB; ++a) {     // X_ab = -X_aa P
            const int b = a - d;
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m) acc += sT[16 * a + ii][16 * a + m] * sInv[a - d][m][jj];
            sT[16 * a + ii][16 * b + jj] = -acc;
        }
        __syncthreads();
    }
    for (int idx = tid; idx < C * C; idx += NT) {   // T = X diag(beta)
        const int i = idx / C, j = idx % C;
        sT[i][j] *= sBeta[j];
    }
    __syncthreads();

    // ---- phase 5: W^T = (kh e^G)^T T^T and Ub = T v (MFMA) --------------------
    {
        // W^T: wave owns channel blocks 2s, 2s+1 (s = wave % 4), i.e. both halves
        // of W's operand fragment for k-step s, for row blocks tb = 2 (wave / 4) + {0, 1}.
        const int s = wave & 3;
        const int ca = 32 * s + lr, cb = ca + 16;
        float a0[CS][8], a1[CS][8];
#pragma unroll
        for (int sp = 0; sp < CS; ++sp)
#pragma unroll
            for (int e = 0; e < 8; ++e) {        // e^{G_j} kh_j = (kh P_j) QF
                const int jx = 32 * sp + 8 * lg + e;
                a0[sp][e] = (jx < C) ? sK[jx][ca] * sQF[jx >> 4][ca] : 0.f;
                a1[sp][e] = (jx < C) ? sK[jx][cb] * sQF[jx >> 4][cb] : 0.f;
            }
        for (int tb = 2 * (wave >> 2); tb < NB && tb < 2 * (wave >> 2) + 2; ++tb) {
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
            const int i = 16 * tb + lr;
#pragma unroll
            for (int sp = 0; sp < CS; ++sp) {
                if (32 * sp > 16 * tb + 15) continue;      // T is lower triangular
                float bT[8];
                const int j0 = 32 * sp + 8 * lg;
                if (j0 < C) load8(&sT[i][j0], bT);
                else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) bT[e] = 0.f;
                }
                if constexpr (PRECISE) {
                    acc0 = mfma_f32x8(a0[sp], bT, acc0);
                    acc1 = mfma_f32x8(a1[sp], bT, acc1);
                } else {
                    acc0 = mfma_f16(a0[sp], bT, acc0);
                    acc1 = mfma_f16(a1[sp], bT, acc1);
                }
            }
            float x[8] = {acc0[0], acc0[1], acc0[2], acc0[3], acc1[0], acc1[1], acc1[2], acc1[3]};
            F::store(rec + R::W_OFF + ((size_t)(tb * 4 + s) * 64 + lane) * F::BYTES, x);
        }
        // Ub tiles (tb, vb = wave): T rows against the (scaled) v columns
        const int vb = wave;
        const int col = 16 * vb + lr;
        float bV[CS][8];
#pragma unroll
        for (int sp = 0; sp < CS; ++sp)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int jx = 32 * sp + 8 * lg + e;
                bV[sp][e] = (jx < C) ? sQ[jx][col] : 0.f;
            }
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            const int i = 16 * tb + lr;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sp = 0; sp < CS; ++sp) {
                if (32 * sp > 16 * tb + 15) continue;
                float aT[8];
                const int j0 = 32 * sp + 8 * lg;
                if (j0 < C) load8(&sT[i][j0], aT);
                else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) aT[e] = 0.f;
                }
                if constexpr (PRECISE) acc = mfma_f32x8(aT, bV[sp], acc);
                else acc = mfma_f16(aT, bV[sp], acc);
            }
            *(f32x4 *)(rec + R::UB_OFF + ((size_t)(vb * NB + tb) * 64 + lane) * 16) = acc * vscale;
        }
    }
}

// =============================================================================
// Inter-chunk kernel: one workgroup (4 waves) per (sequence, head, 64-row half
// of the state); each wave owns 16 state rows held in MFMA accumulators as S^T.
// Shared per-chunk operands are staged through LDS (double-buffered when they
// fit) while the previous chunk computes.
// =============================================================================
template <int C, bool PRECISE>
struct InterCfg {
    using R = Record<C, PRECISE>;
    static constexpr size_t BUF = R::SHARED_BYTES + 4 * R::UB_VB_BYTES;
    static constexpr int NBUF = (2 * BUF <= 160 * 1024) ? 2 : 1;
    static constexpr int N16 = (int)(BUF / 16);
    static constexpr int PER = (N16 + 255) / 256;
};

template <int C, typename Tout, bool PRECISE>
__global__ __launch_bounds__(256) void inter_kernel(PrefillArgs p, int nchains)
{
    using G = ChunkGeom<C>;
    using R = Record<C, PRECISE>;
    using F = Frag<PRECISE>;
    using CFG = InterCfg<C, PRECISE>;
    constexpr int NB = G::NB, CS = G::CS;
    extern __shared__ __align__(16) unsigned char smem[];

    // workgroup -> (chain, half); both halves of a chain land on the same XCD
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int chain = (local >> 1) * 8 + xcd;
    const int vg = local & 1;
    if (chain >= nchains) return;
    const int H = p.H;
    const int n = chain / H, h = chain % H;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int vb = 4 * vg + wave;
    const int vrow = 16 * vb + lr;               // this lane's state row

    const int64_t s0 = p.cu_seqlens[n];
    const int64_t len = p.cu_seqlens[n + 1] - s0;
    const int nch = (int)((len + C - 1) / C);
    const int64_t slot0 = s0 / C + n;

    // state S^T tiles: lane holds S[vrow][16 kb + 4 lg + i]
    f32x4 S[8];
    const size_t sbase = ((size_t)chain * kHeadDim + vrow) * kHeadDim;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        if (p.h0) S[kb] = *(const f32x4 *)(p.h0 + sbase + 16 * kb + 4 * lg);
        else S[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    auto rec_of = [&](int jc) -> const unsigned char * {
        return p.ws + ((size_t)(slot0 + jc) * H + h) * R::BYTES;
    };
    f32x4 stage[CFG::PER];
    auto fetch = [&](int jc) {
        const unsigned char *r = rec_of(jc);
        const f32x4 *sh = (const f32x4 *)r;
        const f32x4 *ub = (const f32x4 *)(r + R::UB_OFF + (size_t)4 * vg * R::UB_VB_BYTES);
        constexpr int SH16 = (int)(R::SHARED_BYTES / 16);
#pragma unroll
        for (int i = 0; i < CFG::PER; ++i) {
            const int idx = tid + 256 * i;
            if (idx < CFG::N16) stage[i] = (idx < SH16) ? sh[idx] : ub[idx - SH16];
        }
    };
    auto commit = [&](int buf) {
        f32x4 *dst = (f32x4 *)(smem + (size_t)buf * CFG::BUF);
#pragma unroll
        for (int i = 0; i < CFG::PER; ++i) {
            const int idx = tid + 256 * i;
            if (idx < CFG::N16) dst[idx] = stage[i];
        }
    };

    Tout *__restrict__ o = (Tout *)p.o;
    if (nch > 0) {
        fetch(0);
        commit(0);
        __syncthreads();
    }
    for (int jc = 0; jc < nch; ++jc) {
        const int buf = (CFG::NBUF == 2) ? (jc & 1) : 0;
        if (CFG::NBUF == 2 && jc + 1 < nch) fetch(jc + 1);
        const unsigned char *B = smem + (size_t)buf * CFG::BUF;
        const int64_t t0 = s0 + (int64_t)jc * C;
        const int L = (len - (int64_t)jc * C) < C ? (int)(len - (int64_t)jc * C) : C;

        // B operand from the state: k-step s covers channels 32s + kperm(lg, e)
        float sscale = 1.0f;
        if constexpr (!PRECISE) {
            float m = 0.f;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(S[kb][i]));
            sscale = pow2_scale_for(wave_max(m), 14);
        }
        typename F::T bS[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            float x[8] = {S[2 * s][0], S[2 * s][1], S[2 * s][2], S[2 * s][3],
                          S[2 * s + 1][0], S[2 * s + 1][1], S[2 * s + 1][2], S[2 * s + 1][3]};
            bS[s] = F::make(x, inv_pow2(sscale));
        }

        // U = Ub - W S^T ; O1 = qg S^T
        f32x4 U[NB], O[NB];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            f32x4 aw = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const size_t fo = ((size_t)(tb * 4 + s) * 64 + lane) * F::BYTES;
                aw = F::mma(F::load(B + R::W_OFF + fo), bS[s], aw);
                aq = F::mma(F::load(B + R::QG_OFF + fo), bS[s], aq);
            }
            const f32x4 ub = *(const f32x4 *)(B + R::SHARED_BYTES +
                                              ((size_t)(wave * NB + tb) * 64 + lane) * 16);
            U[tb] = ub - aw * sscale;
            O[tb] = aq * sscale;
        }

        // B operand from U: k-step s over t covers rows 32s + kperm(lg, e)
        float uscale = 1.0f;
        if constexpr (!PRECISE) {
            float m = 0.f;
#pragma unroll
            for (int tb = 0; tb < NB; ++tb)
#pragma unroll
                for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(U[tb][i]));
            uscale = pow2_scale_for(wave_max(m), 14);
        }
        typename F::T bU[CS];
#pragma unroll
        for (int s = 0; s < CS; ++s) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = (2 * s < NB) ? U[2 * s][e] : 0.f;
                x[e + 4] = (2 * s + 1 < NB) ? U[2 * s + 1][e] : 0.f;
            }
            bU[s] = F::make(x, inv_pow2(uscale));
        }

        // O += M U, then store the valid rows
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            f32x4 am = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < CS; ++s) {
                if (32 * s > 16 * tb + 15) continue;       // M is lower triangular
                am = F::mma(F::load(B + R::M_OFF + ((size_t)(tb * CS + s) * 64 + lane) * F::BYTES),
                            bU[s], am);
            }
            const f32x4 out = O[tb] + am * uscale;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tb + 4 * lg + i;
                if (t < L) o[((size_t)(t0 + t) * H + h) * kHeadDim + vrow] = from_f32<Tout>(out[i]);
            }
        }

        // S^T <- diag(GamC) S^T + kg^T U
        const float *gc = (const float *)(B + R::GC_OFF);
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < CS; ++s)
                acc = F::mma(F::load(B + R::KG_OFF + ((size_t)(kb * CS + s) * 64 + lane) * F::BYTES),
                             bU[s], acc);
            const f32x4 gv = *(const f32x4 *)(gc + 16 * kb + 4 * lg);
            S[kb] = S[kb] * gv + acc * uscale;
        }

        if (jc + 1 < nch) {
            if (CFG::NBUF == 1) {
                __syncthreads();            // everyone is done with the single buffer
                fetch(jc + 1);
            }
            commit(CFG::NBUF == 2 ? ((jc + 1) & 1) : 0);
            __syncthreads();
        }
    }

    if (p.ht) {
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
            *(f32x4 *)(p.ht + sbase + 16 * kb + 4 * lg) = S[kb];
    }
}

// ---- launchers ----------------------------------------------------------------

template <int C, typename Tin, typename Tout>
static hipError_t launch_prefill_t(const PrefillArgs &a) {
    constexpr bool PRECISE = std::is_same<Tin, float>::value;
    const int64_t slots = num_slots(a.T, a.N, C);
    if ((a.stages & 1) && slots > 0) {
        dim3 grid((unsigned)slots, (unsigned)a.H);
        intra_kernel<C, Tin, PRECISE><<<grid, 64 * kIntraWaves, 0, a.stream>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int nchains = a.N * a.H;
    if ((a.stages & 2) && nchains > 0) {
        using CFG = InterCfg<C, PRECISE>;
        const size_t lds = (size_t)CFG::NBUF * CFG::BUF;
        hipError_t e = hipFuncSetAttribute((const void *)inter_kernel<C, Tout, PRECISE>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        const unsigned groups = (unsigned)(8 * 2 * ((nchains + 7) / 8));
        inter_kernel<C, Tout, PRECISE><<<groups, 256, lds, a.stream>>>(a, nchains);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <int C>
static hipError_t launch_prefill_c(const PrefillArgs &a) {
    if (a.in_bf16)
        return a.out_bf16 ? launch_prefill_t<C, __bf16, __bf16>(a) : launch_prefill_t<C, __bf16, float>(a);
    return a.out_bf16 ? launch_prefill_t<C, float, __bf16>(a) : launch_prefill_t<C, float, float>(a);
}

hipError_t launch_prefill(const PrefillArgs &a) {
    switch (a.chunk) {
        case 16: return launch_prefill_c<16>(a);
        case 32: return launch_prefill_c<32>(a);
        case 64: return launch_prefill_c<64>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
